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
