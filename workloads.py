"""Seeded synthetic inputs for the speculative-sampling verifier.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no verifier arithmetic: it draws logits, draft-logit noise and draft
tokens (the drafter's side of a speculative round), and nothing else.  The
verifier's own random numbers (accept uniforms, race exponentials) are not
drawn here; both the GPU library and the oracle derive them from the Philox
key (seed) on their own.

Recipe (all torch generators seeded with ``data_seed``; requests generated in
fixed-size chunks so that the bytes do not depend on the device's memory):
  target logits  Lt[b, j, :] ~ N(0, sigma_t^2) i.i.d., rounded to the dtype
                 (bf16: round-to-nearest-even).
  draft logits   Ld[b, j, :] = Lt[b, j, :] + sigma_b * N(0, 1), with sigma_b
                 fixed or drawn per request from U[lo, hi], rounded to dtype.
  draft tokens   prob:   x ~ softmax over the top-k set of Ld/T (Gumbel-max:
                         argmax of Ld/T + Gumbel noise over the kept tokens;
                         the kept set is the first k of a stable descending
                         sort, i.e. ties to the lowest index);
                 onehot: x = argmax(Lt + N(0, 1)) (greedy drafter);
                 greedy: x = argmax Lt with probability ``greedy_match``,
                         else a uniform draw from the other V - 1 ids.
                 batch:  per request, by its own settings: temperature 0 ->
                         x = argmax Ld (a greedy drafter); else a draw from
                         the draft's temperature / top-k law as for prob (the
                         drafter does not apply top-p; a draft outside the
                         nucleus is a valid input that the verifier rejects).
                 match:  token-only drafts for sampler-match (entry "match",
                         settings as for batch).  The drafter's noisy row of
                         node i (Lt of that row + sigma_b N(0, 1)) proposes
                         its children: the k-th child of a node (by index)
                         takes the k-th token of a draw without replacement
                         (Gumbel top-k of that row / T over its top-k set;
                         temperature 0: the k-th largest logit).  A chain
                         (no ``parents``) is the batch recipe with one child
                         per node.  With ``peak`` > 0 every target row gets
                         +peak on one uniformly drawn token (a confident
                         target, as where a reply copies its prompt).
  batch settings (entry "batch" / "match") each request takes one of the
                 workload's ``mix`` classes (temperature, top_k, top_p),
                 uniformly, from a generator seeded with data_seed + 1.
The five workloads mirror the shapes of the reference pages' setting scaled
to a batch (gamma 3..8 as on the pages, temperatures 0 / 0.7 / 0.8 / 1,
acceptance rates spanning the 0.5..0.9 range quoted for good drafter pairs);
the batch workload mixes greedy, top-k, top-p and top-k + top-p requests on
the fp32 shape of the third.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    entry: str            # "prob" | "onehot" | "greedy"
    B: int                # requests
    G: int                # gamma: draft positions per request
    V: int                # vocabulary size
    dtype: str            # "f32" | "bf16"
    temperature: float    # 0 for greedy
    top_k: int            # 0 = off
    target_sigma: float
    draft_sigma: tuple    # (lo, hi); lo == hi for a fixed sigma
    greedy_match: float = 0.8
    data_seed: int = 0
    verify_seed: int = 42
    chunk: int = 8        # requests generated per generator call
    mix: tuple = ()       # entry "batch": ((temperature, top_k, top_p), ...) request classes
    lengths: tuple = ()   # entry "batch": (lo, hi) draft positions per request, uniform (ragged rows)
    sigma_pos: tuple = ()  # draft noise per position (G values), replacing draft_sigma
    draft_probs: bool = False  # entry "batch": the drafter hands over fp32 probabilities
    parents: tuple = ()   # entry "match": parent node of draft nodes 1..G (empty: a chain)
    peak: float = 0.0     # logit bonus of one token per target row (0: none)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def target_rows(self) -> int:
        return self.B * (self.G + 1)

    @property
    def draft_rows(self) -> int:
        return self.B * self.G if self.entry in ("prob", "batch") else 0

    @property
    def ragged(self) -> bool:
        return self.entry in ("batch", "match") and bool(self.lengths)

    @property
    def has_settings(self) -> bool:
        """Per-request settings (spec_verify_batch)."""
        return self.entry in ("batch", "match")

    @property
    def draft_lengths(self) -> np.ndarray:
        """Draft positions per request (all G unless ragged)."""
        if self.ragged:
            gen = torch.Generator(device="cpu")
            gen.manual_seed(self.data_seed + 2)
            lo, hi = self.lengths
            return torch.randint(lo, hi + 1, (self.B,), generator=gen, dtype=torch.int32).numpy()
        return np.full(self.B, self.G, dtype=np.int32)

    @property
    def has_draft_logits(self) -> bool:
        return self.entry in ("prob", "batch")

    @property
    def logit_bytes(self) -> int:
        """Bytes of every logit row read once: the algorithmic traffic (for a
        batch workload, the draft rows of its sampled requests only)."""
        if self.entry == "match":
            return int((self.draft_lengths + 1).sum()) * self.V * self.elem_bytes
        if self.entry != "batch":
            return (self.target_rows + self.draft_rows) * self.V * self.elem_bytes
        g = self.draft_lengths
        sampled = (batch_settings(self)["temperature"] > 0).numpy() if self.mix else np.ones(self.B, bool)
        target = int((g + 1).sum()) * self.V * self.elem_bytes
        # Draft probabilities are gathered (q(x_j)) and one residual row per
        # rejected request is raced, not streamed by the row pass.
        draft = 0 if self.draft_probs else int(g[sampled].sum()) * self.V * self.elem_bytes
        return target + draft

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 8 requests, gamma 4, V 32000, fp32, T = 1, draft = target + N(0, 1).
    "prob_f32_b8_g4_v32000": Workload("prob_f32_b8_g4_v32000", "prob", 8, 4, 32000, "f32", 1.0, 0,
                                      3.0, (1.0, 1.0)),
    # 64 requests, gamma 5, V 128256, bf16, greedy (T = 0), 0.8 argmax matches.
    "greedy_bf16_b64_g5_v128256": Workload("greedy_bf16_b64_g5_v128256", "greedy", 64, 5, 128256, "bf16",
                                           0.0, 0, 2.5, (0.0, 0.0), greedy_match=0.8),
    # 256 requests, gamma 7, V 151936, fp32, T = 0.8, sigma_b ~ U[0.5, 2].
    "prob_f32_b256_g7_v151936": Workload("prob_f32_b256_g7_v151936", "prob", 256, 7, 151936, "f32", 0.8, 0,
                                         3.0, (0.5, 2.0)),
    # 512 requests, gamma 3, V 262144, bf16, T = 1, greedy drafter, one-hot q.
    "onehot_bf16_b512_g3_v262144": Workload("onehot_bf16_b512_g3_v262144", "onehot", 512, 3, 262144, "bf16",
                                            1.0, 0, 3.0, (1.0, 1.0)),
    # 1024 requests, gamma 8, V 256000, bf16, T = 0.7 then top-64 on p and q.
    "prob_topk64_bf16_b1024_g8_v256000": Workload("prob_topk64_bf16_b1024_g8_v256000", "prob", 1024, 8, 256000,
                                                  "bf16", 0.7, 64, 3.0, (0.3, 2.5)),
}

# Per-request settings in one call (spec_verify_batch): greedy, top-k 50,
# top-p 0.9, top-k 40 then top-p 0.95, a quarter each, on the fp32 shape of
# prob_f32_b256_g7_v151936; the same with ragged draft lengths 1..7 and the
# drafter's probabilities as the draft input.
_MIX4 = ((0.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.8, 40, 0.95))
BATCH_WORKLOADS = {
    "batch_mixed_f32_b256_g7_v151936": Workload(
        "batch_mixed_f32_b256_g7_v151936", "batch", 256, 7, 151936, "f32", 1.0, 0, 3.0, (0.5, 2.0), mix=_MIX4),
    "batch_ragged_probs_f32_b256_g7_v151936": Workload(
        "batch_ragged_probs_f32_b256_g7_v151936", "batch", 256, 7, 151936, "f32", 1.0, 0, 3.0, (0.5, 2.0),
        mix=_MIX4, lengths=(1, 7), draft_probs=True),
}
ALL_WORKLOADS = {**WORKLOADS, **BATCH_WORKLOADS}

# Multi-round workload with acceptance decaying along the draft: the draft
# noise of position j is chosen so that sum_y min(p, q) averages 0.951, 0.889
# and 0.852 at gamma = 3, the per-position rates of the Gemma run on the
# draft-model page (section "맥북 실측: Gemma 4 12B").  The noise levels come
# from tests/golden/make_decay_sigmas.py (the oracle's beta, bisection); a CPU
# test re-checks them.
DECAY_ALPHAS = (0.951, 0.889, 0.852)
DECAY_SIGMAS = (0.1210, 0.2765, 0.3707)
ROUNDS_WORKLOADS = {
    "rounds_decay_bf16_b512_g3_v128256": Workload(
        "rounds_decay_bf16_b512_g3_v128256", "prob", 512, 3, 128256, "bf16", 1.0, 0, 3.0, (0.0, 0.0),
        sigma_pos=DECAY_SIGMAS),
}
ALL_WORKLOADS.update(ROUNDS_WORKLOADS)

# Sampler-match over token-only drafts: prompt lookup's chains (at most 7
# proposals per round, a verify block of 8) and a tree with second choices at
# depths 1 and 2, on a 151936-token vocabulary in bf16.  Requests mix
# temperature 0, top-k 20 then top-p 0.8, top-p 0.9 alone and plain sampling;
# target rows carry a confident token (+18 logits over N(0, 9)), as where a
# reply copies its prompt.
_MIX_MATCH = ((0.0, 0, 1.0), (0.7, 20, 0.8), (1.0, 0, 0.9), (0.8, 0, 1.0))
TREE7 = (0, 0, 1, 1, 3, 5, 6)
MATCH_WORKLOADS = {
    "match_lookup_bf16_b256_g7_v151936": Workload(
        "match_lookup_bf16_b256_g7_v151936", "match", 256, 7, 151936, "bf16", 1.0, 0, 3.0, (0.5, 2.0),
        mix=_MIX_MATCH, peak=18.0),
    "match_tree_bf16_b256_g7_v151936": Workload(
        "match_tree_bf16_b256_g7_v151936", "match", 256, 7, 151936, "bf16", 1.0, 0, 3.0, (0.5, 2.0),
        mix=_MIX_MATCH, peak=18.0, parents=TREE7),
}
ALL_WORKLOADS.update(MATCH_WORKLOADS)

WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "prob_topk64_bf16_b1024_g8_v256000"


def _gumbel_argmax(scores: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    """argmax(scores + Gumbel) along the last axis (lowest index on ties)."""
    u = torch.rand(scores.shape, generator=gen, device=scores.device, dtype=torch.float32)
    g = -torch.log(-torch.log(u))
    return torch.argmax(scores + g, dim=-1)


def _draft_tokens_prob(ld: torch.Tensor, temperature: float, top_k: int, gen: torch.Generator) -> torch.Tensor:
    V = ld.shape[-1]
    z = ld.float() / temperature
    if 0 < top_k < V:
        vals, idx = torch.sort(z, dim=-1, descending=True, stable=True)
        pick = _gumbel_argmax(vals[..., :top_k], gen)
        return torch.gather(idx[..., :top_k], -1, pick.unsqueeze(-1)).squeeze(-1)
    return _gumbel_argmax(z, gen)


def batch_settings(wl: Workload, device="cpu") -> dict:
    """Per-request settings of a batch workload: temperature [B] float32,
    top_k [B] int32, top_p [B] float32 (one mix class per request)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(wl.data_seed + 1)
    cls = torch.randint(0, len(wl.mix), (wl.B,), generator=gen)
    t = torch.tensor([wl.mix[c][0] for c in cls.tolist()], dtype=torch.float32)
    k = torch.tensor([wl.mix[c][1] for c in cls.tolist()], dtype=torch.int32)
    p = torch.tensor([wl.mix[c][2] for c in cls.tolist()], dtype=torch.float32)
    return {"temperature": t.to(device), "top_k": k.to(device), "top_p": p.to(device)}


def generate(wl: Workload, device="cpu", requests: range | None = None) -> dict:
    """Inputs of ``wl`` on ``device``: target_logits [B, G+1, V], draft_logits
    [B, G, V] (prob only, else None), draft_tokens [B, G] int32.

    ``requests`` restricts generation to whole chunks covering that range and
    returns only those requests (same bytes as a full generation).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.data_seed)
    B, G, V = wl.B, wl.G, wl.V
    lo_req, hi_req = (0, B) if requests is None else (requests.start, requests.stop)
    lt_all = torch.empty((hi_req - lo_req, G + 1, V), dtype=wl.torch_dtype, device=device)
    ld_all = (torch.empty((hi_req - lo_req, G, V), dtype=wl.torch_dtype, device=device)
              if wl.has_draft_logits else None)
    x_all = torch.empty((hi_req - lo_req, G), dtype=torch.int32, device=device)
    settings = batch_settings(wl) if wl.has_settings else None
    for c0 in range(0, B, wl.chunk):
        c1 = min(B, c0 + wl.chunk)
        sub = None if settings is None else {k: v[c0:c1] for k, v in settings.items()}
        if c1 <= lo_req:
            # Draw and discard so that later chunks see the same stream.
            _chunk(wl, c1 - c0, gen, device, sub)
            continue
        if c0 >= hi_req:
            break
        lt, ld, x = _chunk(wl, c1 - c0, gen, device, sub)
        a, bnd = max(c0, lo_req), min(c1, hi_req)
        lt_all[a - lo_req: bnd - lo_req] = lt[a - c0: bnd - c0]
        if ld_all is not None:
            ld_all[a - lo_req: bnd - lo_req] = ld[a - c0: bnd - c0]
        x_all[a - lo_req: bnd - lo_req] = x[a - c0: bnd - c0]
    res = {"target_logits": lt_all, "draft_logits": ld_all, "draft_tokens": x_all}
    if settings is not None:
        res.update({k: v[lo_req:hi_req].to(device) for k, v in settings.items()})
    if wl.entry == "batch" and wl.draft_probs:
        res["draft_probs"] = _drafter_probs(ld_all, res["temperature"], res["top_k"])
    if wl.ragged:
        res["lengths"] = torch.from_numpy(wl.draft_lengths[lo_req:hi_req]).to(device)
    if wl.entry == "match" and wl.parents:
        res["parents"] = torch.tensor(wl.parents, dtype=torch.int32, device=device).repeat(hi_req - lo_req, 1)
    return res


def _drafter_probs(ld: torch.Tensor, temperature: torch.Tensor, top_k: torch.Tensor) -> torch.Tensor:
    """The drafter's own sampling law, handed over as fp32 probabilities:
    softmax of its logits / T over its top-k set (the law its tokens were
    drawn from); a temperature-0 drafter hands over a one-hot at its argmax."""
    q = torch.zeros(ld.shape, dtype=torch.float32, device=ld.device)
    for r in range(ld.shape[0]):
        t, k = float(temperature[r]), int(top_k[r])
        z = ld[r].float()
        if t == 0.0:
            q[r].scatter_(-1, torch.argmax(z, dim=-1, keepdim=True), 1.0)
            continue
        z = z / t
        if 0 < k < z.shape[-1]:
            vals, idx = torch.sort(z, dim=-1, descending=True, stable=True)
            q[r].scatter_(-1, idx[..., :k], torch.softmax(vals[..., :k], dim=-1))
        else:
            q[r] = torch.softmax(z, dim=-1)
    return q


def pack_ragged(inp: dict, lengths) -> dict:
    """Packed rows of a ragged batch (data layout only): request b keeps
    target rows 0..g_b and draft rows / tokens 0..g_b-1, request after
    request; cu [B+1] int32 holds the cumulative draft counts."""
    g = [int(v) for v in lengths]
    cu = np.zeros(len(g) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(g)
    out = {"cu_draft": torch.from_numpy(cu).to(inp["target_logits"].device),
           "target_logits": torch.cat([inp["target_logits"][b, :g[b] + 1] for b in range(len(g))]),
           "draft_tokens": torch.cat([inp["draft_tokens"][b, :g[b]] for b in range(len(g))])}
    for key in ("draft_logits", "draft_probs", "parents"):
        if inp.get(key) is not None:
            out[key] = torch.cat([inp[key][b, :g[b]] for b in range(len(g))])
    return out


def with_stride(rows: torch.Tensor, width: int, fill: float) -> torch.Tensor:
    """Rows [..., V] copied into a [..., width] buffer whose padding holds
    `fill` (a value that would change the results if it were ever read)."""
    buf = torch.full(rows.shape[:-1] + (width,), fill, dtype=rows.dtype, device=rows.device)
    buf[..., :rows.shape[-1]] = rows
    return buf


def _chunk(wl: Workload, c: int, gen: torch.Generator, device, settings=None):
    G, V = wl.G, wl.V
    lt = torch.randn((c, G + 1, V), generator=gen, device=device, dtype=torch.float32) * wl.target_sigma
    if wl.peak > 0.0:
        at = torch.randint(0, V, (c, G + 1, 1), generator=gen, device=device)
        lt.scatter_add_(-1, at, torch.full((c, G + 1, 1), wl.peak, device=device))
    lt = lt.to(wl.torch_dtype)
    ld = None
    if wl.entry == "match":
        return lt, None, _match_tokens(wl, lt, c, gen, device, settings)
    if wl.has_draft_logits:
        lo, hi = wl.draft_sigma
        sig = lo + (hi - lo) * torch.rand((c, 1, 1), generator=gen, device=device, dtype=torch.float32)
        if wl.sigma_pos:
            sig = torch.tensor(wl.sigma_pos, dtype=torch.float32, device=device).reshape(1, G, 1)
        noise = torch.randn((c, G, V), generator=gen, device=device, dtype=torch.float32)
        ld = (lt[:, :G].float() + sig * noise).to(wl.torch_dtype)
    if wl.entry == "batch":
        xs = []
        for r in range(c):
            t, k = float(settings["temperature"][r]), int(settings["top_k"][r])
            if t == 0.0:
                xs.append(torch.argmax(ld[r].float(), dim=-1))
            else:
                xs.append(_draft_tokens_prob(ld[r], t, k, gen))
        x = torch.stack(xs)
    elif wl.entry == "prob":
        x = _draft_tokens_prob(ld, wl.temperature, wl.top_k, gen)
    elif wl.entry == "onehot":
        noise = torch.randn((c, G, V), generator=gen, device=device, dtype=torch.float32)
        x = torch.argmax(lt[:, :G].float() + noise * wl.draft_sigma[0], dim=-1)
    elif wl.entry == "greedy":
        amax = torch.argmax(lt[:, :G].float(), dim=-1)
        match = torch.rand((c, G), generator=gen, device=device) < wl.greedy_match
        other = torch.randint(0, max(V - 1, 1), (c, G), generator=gen, device=device)
        other = other + (other >= amax).to(other.dtype)
        x = torch.where(match, amax, other) if V > 1 else amax
    else:
        raise ValueError(wl.entry)
    return lt, ld, x.to(torch.int32)


def _match_tokens(wl: Workload, lt: torch.Tensor, c: int, gen: torch.Generator, device, settings) -> torch.Tensor:
    """Token-only drafts of a chain or tree (the drafter's rows are noisy
    copies of the parents' target rows; see the module recipe)."""
    G, V = wl.G, wl.V
    par = list(wl.parents) if wl.parents else list(range(G))
    lo, hi = wl.draft_sigma
    sig = lo + (hi - lo) * torch.rand((c, 1, 1), generator=gen, device=device, dtype=torch.float32)
    noise = torch.randn((c, G, V), generator=gen, device=device, dtype=torch.float32)
    ld = lt[:, :G].float() + sig * noise  # drafter row of node j, j < G (the nodes that can be parents)
    nchild = [par.count(j) for j in range(G)]
    rank = [par[:i].count(par[i]) for i in range(G)]  # child order under its parent
    x = torch.empty((c, G), dtype=torch.int64, device=device)
    for r in range(c):
        t, k = float(settings["temperature"][r]), int(settings["top_k"][r])
        for j in range(G):
            if not nchild[j]:
                continue
            z = ld[r, j]
            if t == 0.0:
                order = torch.argsort(z, descending=True, stable=True)[:nchild[j]]
            else:
                z = z / t
                keep = torch.argsort(z, descending=True, stable=True)
                if 0 < k < V:
                    keep = keep[:k]
                u = torch.rand(keep.shape, generator=gen, device=device, dtype=torch.float32)
                gz = z[keep] - torch.log(-torch.log(u))
                order = keep[torch.argsort(gz, descending=True, stable=True)[:nchild[j]]]
            for i in range(G):
                if par[i] == j:
                    x[r, i] = order[min(rank[i], order.numel() - 1)]
    return x


def to_host_arrays(t: torch.Tensor | None):
    """float32 -> np.float32; bfloat16 -> np.uint16 bit patterns (for the oracle)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


__all__ = ["Workload", "WORKLOADS", "BATCH_WORKLOADS", "ALL_WORKLOADS", "WORKLOAD_ORDER", "HEADLINE",
           "ROUNDS_WORKLOADS", "DECAY_ALPHAS",
           "generate", "batch_settings", "pack_ragged", "with_stride", "to_host_arrays"]
