"""GPU parity of spec_verify_batch (per-request temperature, top-k, top-p and
temperature-0 requests in one call) against the fp64 oracle.

Bar (oracle/parity.py, compare_batch): invalid and temperature-0 requests
exact; sampled requests p(x_j), q(x_j) within 1e-5 and tokens identical
outside near-ties (relative margin 1e-4) and outside top-p decisions within
1e-9 of flipping.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.parity import assert_parity, assert_parity_batch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# Every kind of request: greedy, top-k (1, 50, 300), top-p alone (0.3 / 0.9),
# top-k then top-p, plain temperature.
MIX_ALL = ((0.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.8, 40, 0.95), (1.3, 0, 1.0), (0.5, 1, 1.0),
           (1.0, 300, 0.5), (0.9, 0, 0.3))


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def gpu_batch(sv, inp, seed, max_top_k=None, onehot=False, stream=None):
    lt = inp["target_logits"].to(DEV)
    x = inp["draft_tokens"].to(DEV)
    ld = None if onehot or inp.get("draft_logits") is None else inp["draft_logits"].to(DEV)
    t = inp["temperature"].to(DEV)
    k = inp["top_k"].to(DEV) if inp.get("top_k") is not None else None
    p = inp["top_p"].to(DEV) if inp.get("top_p") is not None else None
    if max_top_k is None:
        max_top_k = int(inp["top_k"].max()) if k is not None else 0
    res = sv.verify_batch(lt, x, ld, temperature=t, top_k=k, top_p=p, max_top_k=max_top_k, seed=seed,
                          stream=stream)
    torch.cuda.synchronize()
    res["error_code"] = sv.sv_read_device_error(res["workspace"])
    return {kk: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for kk, v in res.items()}


def oracle_batch(inp, seed, max_top_k=1024, onehot=False, req_ids=None):
    h = workloads.to_host_arrays
    B = inp["target_logits"].shape[0]
    k = inp["top_k"] if inp.get("top_k") is not None else torch.zeros(B, dtype=torch.int32)
    p = inp["top_p"] if inp.get("top_p") is not None else torch.ones(B, dtype=torch.float32)
    ld = None if onehot or inp.get("draft_logits") is None else h(inp["draft_logits"].cpu())
    return oracle.verify_batch(h(inp["target_logits"].cpu()), ld, h(inp["draft_tokens"].cpu()),
                               inp["temperature"].cpu().numpy(), k.cpu().numpy(), p.cpu().numpy(),
                               max_top_k=max_top_k, seed=seed, req_ids=req_ids, diagnostics=True)


def check_batch(sv, inp, seed=42, onehot=False, max_top_k=None, **kw):
    print(f"[batch] shape={tuple(inp['target_logits'].shape)} dtype={inp['target_logits'].dtype} "
          f"onehot={onehot}", flush=True)
    got = gpu_batch(sv, inp, seed, max_top_k=max_top_k, onehot=onehot)
    mk = max_top_k if max_top_k is not None else (int(inp["top_k"].max()) if inp.get("top_k") is not None else 0)
    ref = oracle_batch(inp, seed, max_top_k=mk, onehot=onehot)
    rep = assert_parity_batch(got, ref, **kw)
    want = (1 if ref["bad_token"].any() else 0) | (2 if ref["bad_param"].any() else 0)
    assert got["error_code"] == want
    print(f"[batch] {rep}", flush=True)
    return got, ref, rep


def mixed(B, G, V, dtype="f32", mix=MIX_ALL, seed=0):
    wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(B=B, G=G, V=V, dtype=dtype, mix=mix,
                                                                             data_seed=seed)
    return workloads.generate(wl)


@pytest.mark.parametrize("dtype,V", [("f32", 20011), ("bf16", 30001), ("f32", 4099), ("bf16", 517)])
@pytest.mark.parametrize("onehot", [False, True])
def test_mixed_parity(sv, dtype, V, onehot):
    inp = mixed(32, 5, V, dtype, seed=V % 7)
    got, ref, rep = check_batch(sv, inp, onehot=onehot)
    assert rep["greedy_requests"] > 0 and rep["greedy_requests"] < 32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_residual_batch(sv, dtype):
    """Draft rows equal to the target rows and one out-of-range draft token
    per request, over every kind of request (and a top-k above the
    candidate capacity): valid tokens are accepted (p(x) = q(x)), the
    invalid one forces the rejection, and max(p - q, 0) is 0 at every token,
    so the recovered token is drawn from p (the zero-mass reading)."""
    G, V = 4, 20011
    inp = mixed(36, G, V, dtype, mix=MIX_ALL + ((0.8, 1500, 1.0),), seed=5)
    inp["draft_logits"] = inp["target_logits"][:, :G].clone()
    x = torch.argmax(inp["target_logits"][:, :G].float(), dim=-1).to(torch.int32)
    for b in range(x.shape[0]):
        x[b, (3 * b) % G] = -1 if b % 2 else V
    inp["draft_tokens"] = x
    got, ref, rep = check_batch(sv, inp, max_top_k=1500)
    assert (ref["num_accepted"] == np.array([(3 * b) % G for b in range(x.shape[0])])).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_uniform_settings_equal_single_entries(sv, dtype):
    """A batch whose requests share one setting is bit-identical to the
    single-setting entry point (same kernels' arithmetic, same streams)."""
    wl = workloads.WORKLOADS["prob_topk64_bf16_b1024_g8_v256000"].scaled(B=16, V=20001, dtype=dtype)
    inp = workloads.generate(wl)
    B = wl.B
    lt, x, ld = inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV), inp["draft_logits"].to(DEV)
    for T, k in ((0.7, 64), (0.9, 0)):
        t = torch.full((B,), T, dtype=torch.float32, device=DEV)
        kk = torch.full((B,), k, dtype=torch.int32, device=DEV)
        for onehot in (False, True):
            a = sv.verify_batch(lt, x, None if onehot else ld, temperature=t, top_k=kk, max_top_k=max(k, 1), seed=9)
            b = sv.verify("onehot" if onehot else "prob", lt, x, None if onehot else ld, temperature=T, top_k=k,
                          seed=9)
            torch.cuda.synchronize()
            for key in ("out_tokens", "num_accepted", "p_draft"):
                assert torch.equal(a[key], b[key]), (T, k, onehot, key)
            if not onehot:
                assert torch.equal(a["q_draft"], b["q_draft"])
    t0 = torch.zeros((B,), dtype=torch.float32, device=DEV)
    a = sv.verify_batch(lt, x, ld, temperature=t0, seed=9)
    b = sv.verify("greedy", lt, x, temperature=0.0, seed=9)
    torch.cuda.synchronize()
    assert torch.equal(a["out_tokens"], b["out_tokens"]) and torch.equal(a["num_accepted"], b["num_accepted"])


def _rows_case(rows_fn, B, G, V, dtype, T, top_p, seed=5, k=0):
    """Hand-built logits (rows_fn(rng, V) per row), drafts = target argmax or
    a random token."""
    rng = np.random.default_rng(seed)
    lt = np.stack([np.stack([rows_fn(rng, V) for _ in range(G + 1)]) for _ in range(B)]).astype(np.float32)
    ld = np.stack([np.stack([rows_fn(rng, V) for _ in range(G)]) for _ in range(B)]).astype(np.float32)
    x = np.where(rng.random((B, G)) < 0.5, np.argmax(lt[:, :G], axis=-1), rng.integers(0, V, (B, G)))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    return {"target_logits": torch.from_numpy(lt).to(tdt), "draft_logits": torch.from_numpy(ld).to(tdt),
            "draft_tokens": torch.from_numpy(x.astype(np.int32)),
            "temperature": torch.full((B,), T, dtype=torch.float32),
            "top_k": torch.full((B,), k, dtype=torch.int32),
            "top_p": torch.from_numpy(np.asarray(top_p, np.float32).reshape(-1).repeat(B // len(np.atleast_1d(top_p))))}


ROWS = {
    # every logit equal: one histogram bin holds the whole row; the cut is by index
    "flat": lambda rng, V: np.zeros(V),
    # integers: heavy exact ties
    "integers": lambda rng, V: np.round(rng.standard_normal(V) * 2.0),
    # a narrow band: every token within 1e-3 of the maximum
    "band": lambda rng, V: 5.0 + 1e-3 * rng.random(V),
    # two levels: 100 tokens far above the rest
    "two_level": lambda rng, V: np.where(np.arange(V) % (V // 100) == 0, 8.0, 0.0) + 0.01 * rng.standard_normal(V),
}


@pytest.mark.parametrize("rows", list(ROWS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_p_hard_rows(sv, rows, dtype):
    """Rows whose boundary bin holds far more than the collect capacity (the
    radix refinement) and rows of exact ties."""
    inp = _rows_case(ROWS[rows], 4, 2, 32000, dtype, 1.0, [0.3, 0.5, 0.9, 0.97])
    check_batch(sv, inp, max_top_k=0)


# Rows that move the nucleus pass's bin window: ascending logits (every
# token rises past the first look, so the row is binned again with its
# maximum known), a masked prefix (the first looks find no finite logit;
# whole chunks hold none), one token well above the rest near the row's end
# (the window moves up by more than its headroom; at T 0.05 by more than its
# width), and logits near 1e13 with tied maxima (bins past fp64's exact
# integers on the split passes' common grid).
WINDOW_ROWS = {
    "ascending": (1.0, lambda rng, V: np.sort(rng.standard_normal(V) * 3.0)),
    "masked_prefix": (1.0, lambda rng, V: np.where(np.arange(V) < (3 * V) // 5, -np.inf,
                                                   rng.standard_normal(V) * 3.0)),
    "late_spike": (1.0, lambda rng, V: np.where(np.arange(V) == V - 7, 11.0, rng.standard_normal(V))),
    "far_spike": (0.05, lambda rng, V: np.where(np.arange(V) == V - 7, 40.0, rng.standard_normal(V))),
    "huge_ties": (1.0, lambda rng, V: np.where(rng.random(V) < 0.01, 1e13,
                                               1e13 - 2.0 ** 37 * rng.integers(1, 50, V))),
}


@pytest.mark.parametrize("rows", list(WINDOW_ROWS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,V", [(4, 100003), (112, 20011)])
def test_top_p_window_rows(sv, rows, dtype, B, V):
    """Rows that move the window of the nucleus pass, on the split passes
    (20 rows, 16 chunks of 6272 tokens each) and one workgroup per row (560
    rows).  No top_p is a binary fraction: over ~200 tied maxima a stop at
    exactly top_p n of them is decided by the oracle's rounding alone, and
    p(x) = 1/n then differs by far more than the p bar."""
    T, fn = WINDOW_ROWS[rows]
    inp = _rows_case(fn, B, 2, V, dtype, T, [0.3, 0.55, 0.9, 0.97])
    check_batch(sv, inp, max_top_k=0)


def _rising_rows(n_high, first):
    """N(0, 0.01) logits with n_high tokens near 10 placed past index
    `first`: every one of them rises more than the window's headroom (5.5
    nats at T 1) above the largest logit a first look can see."""
    def fn(rng, V):
        r = rng.standard_normal(V) * 0.1
        r[first + rng.choice(V - first, n_high, replace=False)] = 10.0 + 0.01 * np.arange(n_high)
        return r
    return fn


@pytest.mark.parametrize("n_high", [256, 257])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_p_rise_list_capacity(sv, n_high, dtype):
    """As many tokens rising above the nucleus pass's window as its list
    holds (256), and one more (the row is then binned again with its
    maximum known), one workgroup per row (560 rows of 20011; the first
    look covers the first 4096 fp32 or 8192 bf16 elements)."""
    inp = _rows_case(_rising_rows(n_high, 8192), 112, 2, 20011, dtype, 1.0, [0.3, 0.55, 0.9, 0.97])
    check_batch(sv, inp, max_top_k=0)


@pytest.mark.parametrize("top_p", [1e-30, 0.5, float(np.nextafter(np.float32(1), np.float32(0))), 1.0])
def test_top_p_extremes(sv, top_p):
    inp = mixed(16, 4, 5003, "f32", mix=((0.9, 0, top_p), (0.8, 20, top_p)), seed=3)
    check_batch(sv, inp)


@pytest.mark.parametrize("k", [300, 1000])
def test_large_top_k_with_top_p(sv, k):
    inp = mixed(8, 3, 4099, "bf16", mix=((0.9, k, 0.9), (1.1, k, 0.5), (0.0, 0, 1.0)), seed=k)
    check_batch(sv, inp)


@pytest.mark.parametrize("onehot", [False, True])
def test_extreme_temperatures(sv, onehot):
    """Nearly one-hot laws (T 0.03 and 0.05: most masses underflow in fp32)
    and nearly flat ones (T 25), alone, under top-k and under top-p."""
    mix = ((0.05, 0, 0.9), (0.05, 40, 1.0), (25.0, 0, 0.5), (0.03, 0, 1.0), (25.0, 300, 0.95), (0.0, 0, 1.0))
    check_batch(sv, mixed(24, 5, 20011, "bf16", mix=mix, seed=9), onehot=onehot, max_top_k=300)


def test_invalid_settings_emit_nothing(sv):
    inp = mixed(8, 3, 1000, "f32", mix=((0.8, 10, 0.9),), seed=2)
    t, k, p = inp["temperature"].clone(), inp["top_k"].clone(), inp["top_p"].clone()
    t[0] = -1.0
    t[1] = float("nan")
    k[2] = -3
    k[3] = 50  # above max_top_k 20, below V
    p[4] = 0.0
    p[5] = 1.5
    inp.update(temperature=t, top_k=k, top_p=p)
    got, ref, rep = check_batch(sv, inp, max_top_k=20)
    assert rep["invalid_requests"] == 6
    assert got["error_code"] & 2


def test_stream_and_determinism(sv):
    inp = mixed(12, 4, 7001, "bf16", seed=4)
    a = gpu_batch(sv, inp, 42)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_batch(sv, inp, 42, stream=s)
    for key in ("out_tokens", "num_accepted", "p_draft", "q_draft"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("name", list(workloads.BATCH_WORKLOADS))
def test_full_size_batch_every_request(sv, name):
    wl = workloads.BATCH_WORKLOADS[name]
    print(f"[full] {name}: generating on the GPU", flush=True)
    inp = workloads.generate(wl, device=DEV)
    torch.cuda.synchronize()
    got = gpu_batch(sv, inp, wl.verify_seed, max_top_k=max(k for _, k, _ in wl.mix))
    n, out, x = got["num_accepted"], got["out_tokens"], inp["draft_tokens"].cpu().numpy()
    assert ((n >= 0) & (n <= wl.G)).all()
    for r in range(wl.B):
        assert (out[r, :n[r]] == x[r, :n[r]]).all()
        assert 0 <= out[r, n[r]] < wl.V
        assert (out[r, n[r] + 1:] == -1).all()
    assert got["error_code"] == 0
    ids = np.arange(wl.B, dtype=np.int32)  # every request
    sub = {k: v[ids.tolist()].cpu() for k, v in inp.items() if v is not None}
    del inp
    torch.cuda.empty_cache()
    ref = oracle_batch(sub, wl.verify_seed, max_top_k=max(k for _, k, _ in wl.mix), req_ids=ids)
    gsub = {k: v[ids] for k, v in got.items() if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == wl.B}
    rep = assert_parity_batch(gsub, ref)
    print(f"[full] {name}: {rep}", flush=True)


@pytest.mark.parametrize("B,G,V,onehot", [(1, 1, 5003, True), (3, 2, 97, False), (102, 2, 5003, False),
                                          (103, 2, 5003, False), (40, 6, 20011, False)])
def test_top_p_row_counts(sv, B, G, V, onehot):
    """Top-p rows without top-k, as many as select each path of the nucleus
    pass: up to 512 rows split across workgroups (2 rows: 16 chunks each; 510
    rows: 2), 515 and 520 rows one workgroup each; a vocabulary of 97 leaves
    most chunks empty."""
    inp = mixed(B, G, V, "f32", mix=((1.0, 0, 0.9), (0.8, 0, 0.6)), seed=B)
    rows = B * (G + 1) + (0 if onehot else B * G)
    print(f"[batch] top-p rows {rows}", flush=True)
    check_batch(sv, inp, onehot=onehot)


@pytest.mark.parametrize("rows", ["flat", "integers", "band"])
def test_top_p_hard_rows_one_workgroup_each(sv, rows):
    """The hard rows above, 560 of them (more than the split path takes): the
    one-workgroup-per-row path with its refinement of over-full bins."""
    inp = _rows_case(ROWS[rows], 112, 2, 4099, "f32", 1.0, [0.3, 0.5, 0.9, 0.97])
    check_batch(sv, inp, max_top_k=0)
