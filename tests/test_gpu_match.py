"""GPU parity of sampler-match verification (spec_verify_batch with
SV_DRAFT_MATCH) against the fp64 oracle: chains and trees, every kind of
request (temperature 0, top-k, top-p, both, plain sampling), ragged lengths,
invalid trees and tokens, and the statistics outputs.

Bar (oracle/parity.py, compare_batch): invalid and temperature-0 requests
exact; sampled requests p_parent(x_i) within 1e-5, tokens and lengths
identical unless a race of a node on the walk had a near-tie (relative
margin 1e-4) or a top-p decision lay within 1e-9 of flipping.  The accepted
node path is compared exactly wherever the tokens are.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.parity import assert_parity_batch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MIX_ALL = ((0.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.8, 40, 0.95), (1.3, 0, 1.0), (0.5, 1, 1.0),
           (1.0, 300, 0.5), (0.9, 0, 0.3))
BASE = "match_lookup_bf16_b256_g7_v151936"


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def make(B, G, V, dtype, *, parents=(), lengths=(), peak=18.0, seed=0, mix=MIX_ALL):
    wl = workloads.MATCH_WORKLOADS[BASE].scaled(B=B, G=G, V=V, dtype=dtype, mix=mix, data_seed=seed,
                                                 lengths=lengths, parents=tuple(parents), peak=peak)
    return workloads.generate(wl)


def random_tree(G, seed):
    rng = np.random.default_rng(seed)
    # Mostly deep: the previous node as parent half of the time.
    return tuple(int(i - 1 if rng.random() < 0.5 else rng.integers(0, i)) for i in range(1, G + 1))


def run_gpu(sv, inp, *, ragged=False, seed=42, counters=None):
    B, G1, V = inp["target_logits"].shape
    G = G1 - 1
    lt, x, par, cu = inp["target_logits"], inp["draft_tokens"], inp.get("parents"), None
    if ragged:
        pk = workloads.pack_ragged(inp, inp["lengths"])
        lt, x, cu, par = pk["target_logits"], pk["draft_tokens"], pk["cu_draft"].to(DEV), pk.get("parents")
    mk = max(1, int(inp["top_k"].max()))
    res = sv.verify_batch(lt.to(DEV), x.to(DEV), None, draft_kind=sv.SV_DRAFT_MATCH, cu_draft=cu, gamma=G,
                          temperature=inp["temperature"].to(DEV), top_k=inp["top_k"].to(DEV),
                          top_p=inp["top_p"].to(DEV), max_top_k=mk, seed=seed,
                          parents=None if par is None else par.to(DEV).contiguous(), beta=True, counters=counters)
    torch.cuda.synchronize()
    res["error_code"] = sv.sv_read_device_error(res["workspace"])
    out = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}
    if ragged:  # per-position outputs back to [B, G]
        g = inp["lengths"].numpy()
        for key in ("p_draft", "q_draft", "beta"):
            flat, padded, off = out[key], np.full((B, G), np.nan, np.float32), 0
            for b in range(B):
                padded[b, :g[b]] = flat[off:off + g[b]]
                off += g[b]
            out[key] = padded
    return out


def run_oracle(inp, *, ragged=False, seed=42, req_ids=None):
    h = workloads.to_host_arrays
    par = inp.get("parents")
    return oracle.verify_batch(h(inp["target_logits"]), None, h(inp["draft_tokens"]), inp["temperature"].numpy(),
                               inp["top_k"].numpy(), inp["top_p"].numpy(), max_top_k=max(1, int(inp["top_k"].max())),
                               seed=seed, diagnostics=True, match=True, req_ids=req_ids,
                               parents=None if par is None else par.numpy(),
                               lengths=inp["lengths"].numpy() if ragged else None)


def check_paths(got, ref):
    """Accepted node paths: exact on every request whose tokens and length
    equal the oracle's (all of them unless an exemption was used)."""
    differ = 0
    for r in range(ref["num_accepted"].shape[0]):
        if got["num_accepted"][r] != ref["num_accepted"][r] or (got["out_tokens"][r] != ref["out_tokens"][r]).any():
            differ += 1
            continue
        np.testing.assert_array_equal(got["path_nodes"][r], ref["path_nodes"][r], err_msg=f"request {r}")
    return differ


def check(sv, inp, *, ragged=False, seed=42):
    print(f"[match] shape={tuple(inp['target_logits'].shape)} dtype={inp['target_logits'].dtype} "
          f"tree={inp.get('parents') is not None} ragged={ragged}", flush=True)
    got = run_gpu(sv, inp, ragged=ragged, seed=seed)
    ref = run_oracle(inp, ragged=ragged, seed=seed)
    rep = assert_parity_batch(got, ref)
    rep["path_differ"] = check_paths(got, ref)
    # beta of a token-only draft is its acceptance probability p_parent(x).
    both = ~np.isnan(got["p_draft"])
    np.testing.assert_array_equal(got["beta"][both], got["p_draft"][both])
    want = (1 if ref["bad_token"].any() else 0) | (2 if ref["bad_param"].any() else 0)
    assert got["error_code"] == want
    print(f"[match] {rep} mean accepted {ref['num_accepted'].mean():.2f}", flush=True)
    return got, ref, rep


@pytest.mark.parametrize("dtype,V", [("f32", 20011), ("bf16", 30001), ("f32", 4099), ("bf16", 517)])
def test_chain_parity(sv, dtype, V):
    got, ref, rep = check(sv, make(32, 5, V, dtype, seed=V % 7))
    assert 0 < rep["greedy_requests"] < 32
    assert ref["num_accepted"].max() >= 3  # deep paths are exercised


def test_chain_parity_flat_rows(sv):
    """No confident token: low acceptance, most walks end at the root."""
    check(sv, make(32, 4, 12007, "bf16", peak=0.0, seed=3))


@pytest.mark.parametrize("shape", ["tree7", "star", "binary", "random"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_parity(sv, shape, dtype):
    parents = {"tree7": workloads.TREE7, "star": (0, 0, 0, 0, 0, 0), "binary": (0, 0, 1, 1, 2, 2, 3, 3, 4, 4),
               "random": random_tree(12, 5)}[shape]
    got, ref, rep = check(sv, make(24, len(parents), 9001, dtype, parents=parents, seed=len(parents)))
    assert (ref["path_nodes"][:, 0] >= 0).any()


def test_tree_wider_than_a_wave(sv):
    """150 nodes: the child search spans three 64-lane ballots."""
    parents = random_tree(150, 11)
    check(sv, make(6, 150, 3001, "f32", parents=parents, seed=2, mix=((0.0, 0, 1.0), (0.8, 0, 1.0), (0.7, 20, 0.9))))


@pytest.mark.parametrize("tree", [False, True])
def test_ragged(sv, tree):
    inp = make(30, 7, 7001, "bf16", parents=workloads.TREE7 if tree else (), lengths=(0, 7), seed=4)
    assert (inp["lengths"] == 0).any() and (inp["lengths"] == 7).any()
    check(sv, inp, ragged=True)


def test_invalid_trees_settings_and_tokens(sv):
    inp = make(12, 5, 3001, "f32", parents=(0, 0, 1, 2, 2), seed=6, mix=((0.8, 10, 0.9), (0.0, 0, 1.0)))
    par, x, t = inp["parents"].clone(), inp["draft_tokens"].clone(), inp["temperature"].clone()
    par[0, 2] = 3   # node 3's parent is not earlier
    par[1, 0] = -1  # negative parent
    par[2, 4] = 5   # a node is its own parent
    t[3] = float("nan")
    x[4, 0] = -5    # bad tokens: never accepted, p = q = 0
    x[5, 3] = 3001
    inp.update(parents=par, draft_tokens=x, temperature=t)
    got, ref, rep = check(sv, inp)
    assert rep["invalid_requests"] == 4
    assert got["error_code"] == 3
    assert (got["path_nodes"][:4] == -1).all()


def test_greedy_chain_equals_greedy_entry(sv):
    """At temperature 0 a chain under sampler-match is the argmax rule."""
    wl = workloads.WORKLOADS["greedy_bf16_b64_g5_v128256"].scaled(B=16, V=20001)
    inp = workloads.generate(wl)
    lt, x = inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV)
    t0 = torch.zeros(16, dtype=torch.float32, device=DEV)
    a = sv.verify_batch(lt, x, None, draft_kind=sv.SV_DRAFT_MATCH, temperature=t0, seed=3)
    b = sv.verify("greedy", lt, x, temperature=0.0, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(a["out_tokens"], b["out_tokens"]) and torch.equal(a["num_accepted"], b["num_accepted"])
    n = a["num_accepted"].cpu()
    pn = a["path_nodes"].cpu()
    for r in range(16):
        assert pn[r, :n[r]].tolist() == list(range(1, n[r] + 1)) and (pn[r, n[r]:] == -1).all()


def test_counters(sv):
    inp = make(10, 6, 2003, "bf16", parents=workloads.TREE7[:6], lengths=(0, 6), seed=8)
    counters = torch.zeros((10, 3), dtype=torch.int64, device=DEV)
    n_sum = np.zeros(10, np.int64)
    for call in range(2):
        res = run_gpu(sv, inp, ragged=True, seed=call, counters=counters)
        n_sum += res["num_accepted"]
    c = counters.cpu().numpy()
    np.testing.assert_array_equal(c[:, 0], 2 * inp["lengths"].numpy())
    np.testing.assert_array_equal(c[:, 1], n_sum)
    np.testing.assert_array_equal(c[:, 2], 2)


@pytest.mark.parametrize("name", list(workloads.MATCH_WORKLOADS))
def test_full_size_every_request(sv, name):
    wl = workloads.MATCH_WORKLOADS[name]
    print(f"[full] {name}: generating on the GPU", flush=True)
    inp = workloads.generate(wl, device=DEV)
    torch.cuda.synchronize()
    mk = max(k for _, k, _ in wl.mix)
    res = sv.verify_batch(inp["target_logits"], inp["draft_tokens"], None, draft_kind=sv.SV_DRAFT_MATCH,
                          temperature=inp["temperature"], top_k=inp["top_k"], top_p=inp["top_p"], max_top_k=mk,
                          seed=wl.verify_seed, parents=inp.get("parents"))
    torch.cuda.synchronize()
    assert sv.sv_read_device_error(res["workspace"]) == 0
    got = {k: v.cpu().numpy() for k, v in res.items() if k != "workspace"}
    n, out, pn, x = got["num_accepted"], got["out_tokens"], got["path_nodes"], inp["draft_tokens"].cpu().numpy()
    par = np.array(wl.parents) if wl.parents else np.arange(wl.G)
    for r in range(wl.B):  # every accepted node is a child of the one before, with its token emitted
        prev = 0
        for d in range(n[r]):
            assert par[pn[r, d] - 1] == prev and out[r, d] == x[r, pn[r, d] - 1]
            prev = pn[r, d]
        assert 0 <= out[r, n[r]] < wl.V and (out[r, n[r] + 1:] == -1).all() and (pn[r, n[r]:] == -1).all()
    print(f"[full] {name}: mean accepted {n.mean():.3f}", flush=True)
    ids = np.arange(wl.B, dtype=np.int32)  # every request
    sub = {k: v[ids.tolist()].cpu() for k, v in inp.items() if v is not None}
    del inp
    torch.cuda.empty_cache()
    ref = run_oracle(sub, seed=wl.verify_seed, req_ids=ids)
    gsub = {k: v[ids] for k, v in got.items()}
    rep = assert_parity_batch(gsub, ref)
    rep["path_differ"] = check_paths(gsub, ref)
    print(f"[full] {name}: {rep}", flush=True)
