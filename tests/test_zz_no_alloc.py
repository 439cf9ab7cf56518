"""spec_verify_prob_noalloc (no workspace argument, the library's static
device scratch) against spec_verify_prob with a caller workspace, through
the C ABI: bit-identical outputs and error words on two calls in a row, the
second with a smaller input, then a full-row call after them."""

import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def _both(sv, wl, inp):
    lt = inp["target_logits"].to(DEV)
    ld = inp["draft_logits"].to(DEV)
    x = inp["draft_tokens"].to(DEV)
    B, G = x.shape
    params = sv.make_params(B, G, wl.V, wl.torch_dtype, wl.temperature, wl.top_k, wl.verify_seed)
    res = []
    for noalloc in (False, True):
        out = torch.full((B, G + 1), -7, dtype=torch.int32, device=DEV)
        nacc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        pd = torch.full((B, G), -7.0, dtype=torch.float32, device=DEV)
        qd = torch.full((B, G), -7.0, dtype=torch.float32, device=DEV)
        if noalloc:
            err = torch.full((1,), -7, dtype=torch.int32, device=DEV)
            sv.spec_verify_prob_noalloc(params, lt, ld, x, out, nacc, pd, qd, err)
            torch.cuda.synchronize()
            code = int(err.item())
        else:
            ws = sv.alloc_workspace(params, DEV)
            sv.spec_verify_prob(params, lt, ld, x, out, nacc, pd, qd, ws)
            torch.cuda.synchronize()
            code = sv.sv_read_device_error(ws)
        res.append({"out": out.cpu().numpy(), "n": nacc.cpu().numpy(), "p": pd.cpu().numpy(),
                    "q": qd.cpu().numpy(), "err": code})
    return res


def test_noalloc_equals_workspace_entry(sv):
    cases = [
        # (workload, overrides, a draft token planted out of range)
        ("prob_topk64_bf16_b1024_g8_v256000", dict(B=64, V=50000), True),
        ("prob_topk64_bf16_b1024_g8_v256000", dict(B=5, G=3, V=20011), False),
        ("prob_f32_b8_g4_v32000", {}, False),
    ]
    for name, over, bad in cases:
        wl = workloads.WORKLOADS[name].scaled(**over)
        print(f"[noalloc] {name} {over} bad_token={bad}", flush=True)
        inp = workloads.generate(wl)
        if bad:
            inp["draft_tokens"][3, 1] = wl.V
        ref, got = _both(sv, wl, inp)
        for key in ("out", "n", "p", "q"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{name} {over}: {key}")
        assert got["err"] == ref["err"] == (1 if bad else 0)
        assert (ref["n"] >= 0).all() and (ref["out"] != -7).all()


def test_noalloc_limits(sv):
    p = sv.make_params(4096, 8, 256000, sv.SV_BF16, 0.7, 1024, 1)
    assert sv.sv_workspace_bytes(p) > sv.SV_NOALLOC_SCRATCH_BYTES
    lib = sv.load_library()
    fake = torch.empty(16, dtype=torch.int32, device=DEV)
    f = sv._ptr(fake)
    assert lib.spec_verify_prob_noalloc(ctypes.byref(p), f, f, f, f, f, None, None, None, None) == sv.SV_ERR_SCRATCH
    p2 = sv.make_params(4, 2, 5000, sv.SV_BF16, 0.7, 2000, 1)
    assert lib.spec_verify_prob_noalloc(ctypes.byref(p2), f, f, f, f, f, None, None, None, None) == sv.SV_ERR_UNSUPPORTED


def test_noalloc_captured_in_graph(sv):
    """The no-alloc call captured into a HIP graph (no workspace to allocate
    during capture) and replayed three times, with eager calls of other
    seeds on the same scratch between the replays: every replay equals the
    eager result bit for bit."""
    wl = workloads.WORKLOADS["prob_topk64_bf16_b1024_g8_v256000"].scaled(B=12, V=20011)
    inp = workloads.generate(wl)
    lt, ld, x = inp["target_logits"].to(DEV), inp["draft_logits"].to(DEV), inp["draft_tokens"].to(DEV)
    B, G = x.shape

    def call(seed):
        params = sv.make_params(B, G, wl.V, wl.torch_dtype, wl.temperature, wl.top_k, seed)
        r = {"out_tokens": torch.empty((B, G + 1), dtype=torch.int32, device=DEV),
             "num_accepted": torch.empty((B,), dtype=torch.int32, device=DEV),
             "p_draft": torch.empty((B, G), dtype=torch.float32, device=DEV),
             "q_draft": torch.empty((B, G), dtype=torch.float32, device=DEV)}
        sv.spec_verify_prob_noalloc(params, lt, ld, x, r["out_tokens"], r["num_accepted"], r["p_draft"],
                                    r["q_draft"])
        return r

    keys = ("out_tokens", "num_accepted", "p_draft", "q_draft")
    eager = {k: v.clone() for k, v in call(42).items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(42)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = call(42)
    for rep in range(3):
        other = call(1000 + rep)
        torch.cuda.synchronize()
        for k in keys:
            res[k].fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        print(f"[noalloc-graph] replay {rep}", flush=True)
        for k in keys:
            assert torch.equal(res[k], eager[k]), (rep, k)
        assert not torch.equal(other["out_tokens"], eager["out_tokens"])
