"""GPU parity at size extremes, against the oracle: a vocabulary of about a
million tokens (1,000,003: a ragged tail after every split, key indices
above 2^19) and many tiny requests (40,000 requests over a vocabulary of 37:
request-level grids far larger than any workload's, and rows shorter than a
wave), for every entry point and, for the batch call, per-request settings
with top-k and top-p; and the largest draft length the library takes."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.parity import assert_parity, assert_parity_batch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MODES = {"prob": oracle.MODE_PROB, "onehot": oracle.MODE_ONEHOT, "greedy": oracle.MODE_GREEDY}
W = workloads.WORKLOADS


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def single(sv, entry, inp, T, k, seed):
    h = workloads.to_host_arrays
    ld = inp["draft_logits"].to(DEV) if entry == "prob" else None
    res = sv.verify(entry, inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV), ld, temperature=T, top_k=k,
                    seed=seed)
    torch.cuda.synchronize()
    got = {kk: v.cpu().numpy() for kk, v in res.items() if kk != "workspace"}
    ref = oracle.verify(MODES[entry], h(inp["target_logits"]), h(inp["draft_logits"]) if entry == "prob" else None,
                        h(inp["draft_tokens"]), temperature=T, top_k=k, seed=seed, diagnostics=entry != "greedy")
    return assert_parity(entry, got, ref)


@pytest.mark.parametrize("entry,k,dtype", [("prob", 0, "f32"), ("prob", 64, "bf16"), ("prob", 700, "f32"),
                                           ("onehot", 0, "bf16"), ("greedy", 0, "f32")])
def test_million_token_vocabulary(sv, entry, k, dtype):
    name = {"prob": "prob_f32_b256_g7_v151936", "onehot": "onehot_bf16_b512_g3_v262144",
            "greedy": "greedy_bf16_b64_g5_v128256"}[entry]
    wl = W[name].scaled(B=3, G=2, V=1_000_003, dtype=dtype)
    inp = workloads.generate(wl)
    T = wl.temperature if entry != "greedy" else 0.0
    print(f"[extreme] {entry} k={k} {dtype} V=1000003", flush=True)
    print(f"[extreme]   {single(sv, entry, inp, T, k, 21)}", flush=True)


@pytest.mark.parametrize("entry,k", [("prob", 5, ), ("prob", 0), ("onehot", 3), ("greedy", 0)])
def test_many_tiny_requests(sv, entry, k):
    name = {"prob": "prob_f32_b8_g4_v32000", "onehot": "onehot_bf16_b512_g3_v262144",
            "greedy": "greedy_bf16_b64_g5_v128256"}[entry]
    wl = W[name].scaled(B=40000, G=3, V=37)
    inp = workloads.generate(wl)
    T = wl.temperature if entry != "greedy" else 0.0
    print(f"[extreme] {entry} k={k} B=40000 V=37", flush=True)
    print(f"[extreme]   {single(sv, entry, inp, T, k, 22)}", flush=True)


def test_many_tiny_requests_batch(sv):
    mix = ((0.0, 0, 1.0), (0.7, 5, 1.0), (1.0, 0, 0.8), (0.9, 7, 0.9), (1.3, 0, 1.0))
    wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(B=30000, G=3, V=37, mix=mix)
    inp = workloads.generate(wl)
    print("[extreme] batch B=30000 V=37", flush=True)
    res = sv.verify_batch(inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV), inp["draft_logits"].to(DEV),
                          temperature=inp["temperature"].to(DEV), top_k=inp["top_k"].to(DEV),
                          top_p=inp["top_p"].to(DEV), max_top_k=7, seed=23, beta=True)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in res.items() if k != "workspace"}
    h = workloads.to_host_arrays
    ref = oracle.verify_batch(h(inp["target_logits"]), h(inp["draft_logits"]), h(inp["draft_tokens"]),
                              inp["temperature"].numpy(), inp["top_k"].numpy(), inp["top_p"].numpy(), max_top_k=7,
                              seed=23, diagnostics=True)
    print(f"[extreme]   {assert_parity_batch(got, ref)}", flush=True)
    both = ~np.isnan(ref["beta"])
    assert float(np.abs(got["beta"][both] - ref["beta"][both]).max()) <= 1e-5


@pytest.mark.parametrize("entry,k", [("prob", 0), ("prob", 16), ("onehot", 16), ("greedy", 0)])
def test_largest_gamma(sv, entry, k):
    """gamma = 16384, the largest supported (the top-k accept pass keeps one
    flag per position in LDS), over a short vocabulary; draft rows equal to
    the target's so that long accepted runs occur."""
    name = {"prob": "prob_f32_b8_g4_v32000", "onehot": "onehot_bf16_b512_g3_v262144",
            "greedy": "greedy_bf16_b64_g5_v128256"}[entry]
    wl = W[name].scaled(B=2, G=16384, V=41)
    inp = workloads.generate(wl)
    if entry == "prob":
        inp["draft_logits"] = inp["target_logits"][:, :-1].clone()
    T = wl.temperature if entry != "greedy" else 0.0
    print(f"[extreme] {entry} k={k} gamma=16384 V=41", flush=True)
    print(f"[extreme]   {single(sv, entry, inp, T, k, 24)}", flush=True)
