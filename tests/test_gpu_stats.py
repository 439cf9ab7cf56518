"""GPU statistics of spec_verify_batch against the fp64 oracle: the
per-position acceptance probability beta = sum_y min(p(y), q(y)) on every
path, the per-request counters across calls, and the multi-round driver on
rows whose acceptance decays along the draft.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MIX = ((0.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.8, 40, 0.95), (1.2, 0, 1.0), (0.6, 300, 0.8))


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def make(B, G, V, dtype, *, lengths=None, probs=False, seed=0):
    wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(
        B=B, G=G, V=V, dtype=dtype, mix=MIX, data_seed=seed, lengths=lengths or (), draft_probs=probs)
    return workloads.generate(wl)


def beta_case(sv, inp, kind, ragged=False):
    print(f"[beta] kind={kind} ragged={ragged} shape={tuple(inp['target_logits'].shape)} "
          f"dtype={inp['target_logits'].dtype}", flush=True)
    B, G1, V = inp["target_logits"].shape
    G = G1 - 1
    draft = {"logits": inp.get("draft_logits"), "probs": inp.get("draft_probs"), "onehot": None}[kind]
    lt, x, cu = inp["target_logits"], inp["draft_tokens"], None
    if ragged:
        pk = workloads.pack_ragged(dict(inp, draft_logits=draft if kind == "logits" else None,
                                        draft_probs=draft if kind == "probs" else None), inp["lengths"])
        lt, x, cu = pk["target_logits"], pk["draft_tokens"], pk["cu_draft"].to(DEV)
        draft = pk.get("draft_logits") if kind == "logits" else pk.get("draft_probs")
    mk = int(inp["top_k"].max())
    res = sv.verify_batch(lt.to(DEV), x.to(DEV), None if draft is None else draft.to(DEV),
                          draft_kind={"logits": 0, "onehot": 1, "probs": 2}[kind], cu_draft=cu, gamma=G,
                          temperature=inp["temperature"].to(DEV), top_k=inp["top_k"].to(DEV),
                          top_p=inp["top_p"].to(DEV), max_top_k=mk, seed=5, beta=True)
    torch.cuda.synchronize()
    got = res["beta"].cpu().numpy()
    h = workloads.to_host_arrays
    ref = oracle.verify_batch(h(inp["target_logits"]), h(inp["draft_logits"]) if kind == "logits" else None,
                              h(inp["draft_tokens"]), inp["temperature"].numpy(), inp["top_k"].numpy(),
                              inp["top_p"].numpy(), max_top_k=mk, seed=5, diagnostics=True,
                              draft_probs=inp["draft_probs"].numpy() if kind == "probs" else None,
                              lengths=inp["lengths"].numpy() if ragged else None)
    g = inp["lengths"].numpy() if ragged else np.full(B, G)
    off = 0
    worst = 0.0
    for b in range(B):
        # Every request, near-cut ones included: a top-p stop within 1e-9 of
        # flipping moves beta by at most that much mass.
        mine = got[off:off + g[b]] if ragged else got[b, :g[b]]
        worst = max(worst, float(np.max(np.abs(mine - ref["beta"][b, :g[b]]), initial=0.0)))
        off += g[b] if ragged else 0
    print(f"[beta] max |d beta| = {worst:.3g}", flush=True)
    assert worst <= 1e-5


@pytest.mark.parametrize("kind", ["logits", "probs", "onehot"])
@pytest.mark.parametrize("dtype,V", [("f32", 9001), ("bf16", 20011)])
def test_beta_parity(sv, kind, dtype, V):
    beta_case(sv, make(24, 4, V, dtype, probs=True, seed=V % 5), kind)


@pytest.mark.parametrize("kind", ["logits", "probs"])
def test_beta_parity_ragged(sv, kind):
    beta_case(sv, make(20, 5, 7001, "bf16", lengths=(0, 5), probs=True, seed=9), kind, ragged=True)


def test_counters_accumulate(sv):
    """counters[b] += (draft positions, accepted, 1) per call; an invalid
    request is not counted."""
    inp = make(16, 4, 3001, "f32", lengths=(0, 4), seed=2)
    t = inp["temperature"].clone()
    t[3] = -1.0  # invalid: not verified, not counted
    pk = workloads.pack_ragged(inp, inp["lengths"])
    counters = torch.zeros((16, 3), dtype=torch.int64, device=DEV)
    counters[:, 2] = 7  # the library adds to what is there
    total_n = np.zeros(16, np.int64)
    for call in range(3):
        res = sv.verify_batch(pk["target_logits"].to(DEV), pk["draft_tokens"].to(DEV), pk["draft_logits"].to(DEV),
                              cu_draft=pk["cu_draft"].to(DEV), gamma=4, temperature=t.to(DEV),
                              top_k=inp["top_k"].to(DEV), top_p=inp["top_p"].to(DEV), max_top_k=300, seed=call,
                              counters=counters)
        torch.cuda.synchronize()
        total_n += res["num_accepted"].cpu().numpy()
    c = counters.cpu().numpy()
    g = inp["lengths"].numpy().astype(np.int64)
    ok = np.arange(16) != 3
    np.testing.assert_array_equal(c[ok, 0], 3 * g[ok])
    np.testing.assert_array_equal(c[ok, 1], total_n[ok])
    np.testing.assert_array_equal(c[ok, 2], 7 + 3)
    np.testing.assert_array_equal(c[3], [0, 0, 7])


def test_rounds_driver_decaying_acceptance(sv):
    """Rows whose acceptance decays 0.951 / 0.889 / 0.852 along the draft:
    the GPU's beta, the acceptance rates measured from n, and tokens per
    round against Eq. 1 with per-position rates (4 rounds x 512 requests)."""
    wl = workloads.ROUNDS_WORKLOADS["rounds_decay_bf16_b512_g3_v128256"]
    st = bench.rounds_driver(sv, wl, 4, DEV)
    print(f"[rounds] { {k: v for k, v in st.items() if not k.startswith('_')} }", flush=True)
    n = st["_n"]
    assert st["counters"] == {"draft_n": 4 * 512 * 3, "draft_n_accepted": int(n.sum()), "draft_rounds": 4 * 512}
    np.testing.assert_allclose(st["beta_by_position"], workloads.DECAY_ALPHAS, atol=0.015)
    # Measured acceptance follows beta (binomial; 4 sigma ~ 0.02-0.035).
    reach = [(n >= j).sum() for j in range(3)]
    for j in range(3):
        a, b = st["acceptance_by_position"][j], st["beta_by_position"][j]
        assert abs(a - b) <= 4.5 * np.sqrt(b * (1 - b) / reach[j]) + 1e-3, (j, a, b)
    # Tokens per round against Eq. 1 (standard error of the mean of n + 1).
    se = np.std(n + 1) / np.sqrt(n.size)
    assert abs(st["tokens_per_round"] - st["tokens_per_round_eq1"]) <= 4.5 * se, st
