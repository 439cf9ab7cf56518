"""GPU parity of the single-read top-k pass on rows built against a running
threshold: ascending rows (every vector beats every earlier one, so every
step stashes candidates and the stash flushes and compacts continually),
descending rows (the first batch holds the whole top-k), constant rows (one
tie group: the lowest indices win), sawtooth rows (the top values recur in
every period) and two-level rows (a fifth of the tokens tie at the top), in
fp32 and bf16 (where rounding turns the ramps into runs of equal values), at
every candidate-capacity tier of k.  Draft tokens are drawn from the draft
row's own top-k set, so the accept test and the residual race both run.

Bar (oracle/parity.py): p(x_j), q(x_j) within 1e-5; tokens and lengths
identical outside near-ties.
"""

import pytest
import torch

import oracle
import workloads
from oracle.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATTERNS = ["ascending", "descending", "constant", "sawtooth", "two_level"]


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def pattern(V, name, shift):
    y = torch.arange(V, dtype=torch.float64)
    if name == "ascending":
        return y / V * 20.0 - 10.0 + shift
    if name == "descending":
        return 10.0 - y / V * 20.0 + shift
    if name == "constant":
        return torch.full((V,), shift)
    if name == "sawtooth":
        return (y % 977) / 977.0 * 8.0 + shift
    return torch.where(y % 5 == 0, 3.0 + shift, shift)


def make_input(B, G, V, name, dtype, k, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lt = torch.stack([torch.stack([pattern(V, name, 0.01 * (b * (G + 1) + j)) for j in range(G + 1)])
                      for b in range(B)]).to(dt)
    ld = torch.stack([torch.stack([pattern(V, name, -0.02 * (b * G + j)) for j in range(G)])
                      for b in range(B)]).to(dt)
    order = torch.sort(ld.float(), dim=-1, descending=True, stable=True).indices
    pick = torch.randint(0, k, (B, G, 1), generator=g)
    x = torch.gather(order, -1, pick)[..., 0].to(torch.int32)
    return lt, ld, x


@pytest.mark.parametrize("k", [1, 64, 300, 1000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", PATTERNS)
def test_topk_patterns(sv, name, dtype, k):
    B, G, V, T = 4, 3, 30001, 0.9
    lt, ld, x = make_input(B, G, V, name, dtype, k, seed=len(name) + k)
    print(f"[topk-pattern] {name} {dtype} k={k} B={B} G={G} V={V}", flush=True)
    for entry in ("prob", "onehot"):
        res = sv.verify(entry, lt.to(DEV), x.to(DEV), ld.to(DEV) if entry == "prob" else None, temperature=T,
                        top_k=k, seed=11)
        torch.cuda.synchronize()
        got = {kk: v.cpu().numpy() for kk, v in res.items() if kk != "workspace"}
        h = workloads.to_host_arrays
        ref = oracle.verify(oracle.MODE_PROB if entry == "prob" else oracle.MODE_ONEHOT, h(lt),
                            h(ld) if entry == "prob" else None, h(x), temperature=T, top_k=k, seed=11,
                            diagnostics=True)
        print(f"[topk-pattern]   {entry} {assert_parity(entry, got, ref)}", flush=True)
