"""Seeded random configurations of spec_verify_batch (and of the
single-setting entry points) against the fp64 oracle: shapes (B, G and V from 1 up), logit types, draft kinds (logits,
one-hot, probabilities, token-only under sampler-match with random trees),
dense and ragged layouts with zero-length drafts, row strides, random
per-request settings (temperature 0 to 2.5, top-k from 1 to past the
candidate capacity and V, top-p from 1e-6 to 1) and some out-of-range draft
tokens.  Each case prints its configuration before it runs.  Bar: as in
test_gpu_batch.py (oracle/parity.py, compare_batch)."""

import numpy as np
import pytest

from test_gpu_layout import check, make, sv  # noqa: F401  (sv: the module fixture)
from test_gpu_match import check as match_check
from test_gpu_match import make as match_make
from test_gpu_match import random_tree
from test_gpu_parity import check as single_check

import workloads

pytestmark = pytest.mark.gpu

N_CASES = 64
N_MATCH_CASES = 32
N_SINGLE_CASES = 64
_T = (0.0, 0.05, 0.3, 0.7, 1.0, 2.5)
_K = (0, 1, 2, 20, 64, 65, 300, 1000, 1025)
_P = (1.0, 0.999999, 0.9, 0.5, 0.1, 1e-6)


def fuzz_case(i: int) -> dict:
    rng = np.random.default_rng(7000 + i)
    V = int(rng.choice([1, 2, 3, 17, 63, 64, 65, 511, 1000, 4097, 9001, 20011]))
    G = int(rng.integers(1, 13))
    mix = tuple((float(rng.choice(_T)), int(min(int(rng.choice(_K)), V)), float(rng.choice(_P)))
                for _ in range(int(rng.integers(1, 5))))
    return dict(B=int(rng.integers(1, 34)), G=G, V=V, dtype=str(rng.choice(["f32", "bf16"])),
                kind=str(rng.choice(["logits", "onehot", "probs"])), ragged=bool(rng.integers(0, 2)),
                pad_t=int(rng.choice([0, 0, 3, 64])), pad_d=int(rng.choice([0, 0, 5])), mix=mix,
                bad=int(rng.integers(0, 3)), seed=int(rng.integers(0, 1 << 30)))


def fuzz_inputs(c: dict) -> dict:
    inp = make(c["B"], c["G"], c["V"], c["dtype"], lengths=(0, c["G"]) if c["ragged"] else None,
               probs=c["kind"] == "probs", seed=c["seed"] % 1000, mix=c["mix"])
    x = inp["draft_tokens"].clone()
    rng = np.random.default_rng(c["seed"])
    for _ in range(c["bad"]):  # out-of-range draft tokens
        b, j = int(rng.integers(0, c["B"])), int(rng.integers(0, c["G"]))
        x[b, j] = -1 if rng.random() < 0.5 else c["V"]
    inp["draft_tokens"] = x
    return inp


# Batch configurations with the draft given as fp32 probabilities that
# randomized sweeps found: 100684 and 100972, T = 0.05 on 3 tokens, a
# rejection whose residual (1e-66) lies below fp32's range and a draft
# probability that is an fp32 denormal (9.5e-44), which the hardware
# logarithm would take as 0; 101291 and 103609, a nucleus cut (top-p 1e-6,
# 0.1) that keeps one of two tokens tied at the maximum, so that the tied
# token past the cut must count neither in the kept mass nor in the race.
BATCH_RESIDUALS = (100684, 100972, 101291, 103609)


@pytest.mark.parametrize("i", BATCH_RESIDUALS)
def test_batch_residual_races(sv, i):  # noqa: F811
    c = fuzz_case(i)
    assert c["kind"] == "probs"
    print(f"[batch residual] case {i}: {c}", flush=True)
    check(sv, fuzz_inputs(c), c["kind"], c["ragged"], pad_t=c["pad_t"], pad_d=c["pad_d"], seed=c["seed"])


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz(sv, i):  # noqa: F811
    c = fuzz_case(i)
    print(f"[fuzz] case {i}: {c}", flush=True)
    check(sv, fuzz_inputs(c), c["kind"], c["ragged"], pad_t=c["pad_t"], pad_d=c["pad_d"], seed=c["seed"])


def match_case(i: int) -> dict:
    rng = np.random.default_rng(9000 + i)
    V = int(rng.choice([1, 2, 5, 64, 65, 1000, 4097, 9001]))
    G = int(rng.integers(1, 12))
    mix = tuple((float(rng.choice(_T)), int(min(int(rng.choice(_K)), V)), float(rng.choice(_P)))
                for _ in range(int(rng.integers(1, 5))))
    shape = str(rng.choice(["chain", "tree"]))
    return dict(B=int(rng.integers(1, 30)), G=G, V=V, dtype=str(rng.choice(["f32", "bf16"])), mix=mix,
                parents=random_tree(G, 9000 + i) if shape == "tree" else (), ragged=bool(rng.integers(0, 2)),
                peak=float(rng.choice([6.0, 18.0])), bad=int(rng.integers(0, 3)), seed=int(rng.integers(0, 1 << 30)))


@pytest.mark.parametrize("i", range(N_MATCH_CASES))
def test_fuzz_match(sv, i):  # noqa: F811
    c = match_case(i)
    print(f"[fuzz-match] case {i}: {c}", flush=True)
    inp = match_make(c["B"], c["G"], c["V"], c["dtype"], parents=c["parents"],
                     lengths=(0, c["G"]) if c["ragged"] else (), peak=c["peak"], seed=c["seed"] % 1000,
                     mix=c["mix"])
    x = inp["draft_tokens"].clone()
    rng = np.random.default_rng(c["seed"])
    for _ in range(c["bad"]):
        b, j = int(rng.integers(0, c["B"])), int(rng.integers(0, c["G"]))
        x[b, j] = -1 if rng.random() < 0.5 else c["V"]
    inp["draft_tokens"] = x
    match_check(sv, inp, ragged=c["ragged"], seed=c["seed"])


_SINGLE_BASE = {"prob": "prob_f32_b256_g7_v151936", "onehot": "onehot_bf16_b512_g3_v262144",
                "greedy": "greedy_bf16_b64_g5_v128256"}


def single_case(i: int) -> dict:
    rng = np.random.default_rng(11000 + i)
    entry = str(rng.choice(["prob", "onehot", "greedy"], p=[0.45, 0.35, 0.2]))
    V = int(rng.choice([1, 2, 7, 64, 65, 777, 4097, 20011]))
    G = int(rng.choice([1, 3, 8, 16, 63, 64, 70]))
    T = 0.0 if entry == "greedy" else float(rng.choice([0.05, 0.3, 0.8, 1.0, 2.5]))
    k = 0 if entry == "greedy" else int(min(int(rng.choice([0, 1, 20, 64, 65, 300, 1000, 1025])), V))
    return dict(entry=entry, B=int(rng.integers(1, 25)), G=G, V=V, dtype=str(rng.choice(["f32", "bf16"])), T=T,
                k=k, bad=int(rng.integers(0, 3)), seed=int(rng.integers(0, 1 << 30)))


def single_inputs(c: dict) -> dict:
    wl = workloads.WORKLOADS[_SINGLE_BASE[c["entry"]]].scaled(B=c["B"], G=c["G"], V=c["V"], dtype=c["dtype"],
                                                              data_seed=c["seed"] % 1000)
    inp = workloads.generate(wl)
    x = inp["draft_tokens"].clone()
    rng = np.random.default_rng(c["seed"])
    for _ in range(c["bad"]):
        b, j = int(rng.integers(0, c["B"])), int(rng.integers(0, c["G"]))
        x[b, j] = -1 if rng.random() < 0.5 else c["V"]
    inp["draft_tokens"] = x
    return inp


@pytest.mark.parametrize("i", range(N_SINGLE_CASES))
def test_fuzz_single(sv, i):  # noqa: F811
    c = single_case(i)
    print(f"[fuzz-single] case {i}: {c}", flush=True)
    single_check(sv, c["entry"], single_inputs(c), T=c["T"], k=c["k"], seed=c["seed"])


# Configurations of single_case (prob entry, T = 0.05) in which a rejection
# falls where p and q both hold nearly all their mass on the same token (the
# draft tokens there were not drawn from q, so such rejections are common),
# found by randomized sweeps.  Full rows: in 5000 ... 5541 the residual is
# carried by the shared top token, with p - q of 1e-15 to 1e-8, which fp32
# rounds to 0; in 5160, 5211 and 5421 its p - q is below fp64's resolution at
# 1 (1e-19), as in the oracle, so the residual is carried by tokens far below
# the maximum (down to 3e-40); in 7768, 9270, 9366, 20867, 22450 those lie
# below 2^-190 (down to 1e-85; 21735: bf16).  30514: a top-k of 1025 (a cut
# over the full row) where a token with the same gap below both maxima carries
# the rows' masses off their maxima.  40154: top-20 candidates with a
# residual of 1e-109.  201617: a row that is not peaked (a token 0.125 below
# both maxima holds 8% of the mass) with normalisers that agree to 6e-9.  The single entry (for full rows, accept and race in
# one launch) and the batch entry with the same setting (separate accept,
# race and finish) both run the race; they must agree bit for bit, and with
# the oracle.
LOW_T_RESIDUALS = (5000, 5033, 5160, 5211, 5255, 5289, 5421, 5511, 5541, 7768, 9270, 9366, 20867, 21735, 22450,
                   30514, 40154, 201617)


@pytest.mark.parametrize("i", LOW_T_RESIDUALS)
def test_low_temperature_residual_races(sv, i):  # noqa: F811
    import torch
    c = single_case(i)
    assert c["entry"] == "prob" and c["T"] == 0.05
    print(f"[low-T residual] case {i}: {c}", flush=True)
    inp = single_inputs(c)
    got, _, _ = single_check(sv, "prob", inp, T=c["T"], k=c["k"], seed=c["seed"])
    dev = torch.device("cuda:0")
    B = c["B"]
    a = sv.verify_batch(inp["target_logits"].to(dev), inp["draft_tokens"].to(dev), inp["draft_logits"].to(dev),
                        temperature=torch.full((B,), c["T"], dtype=torch.float32, device=dev),
                        top_k=torch.full((B,), c["k"], dtype=torch.int32, device=dev), max_top_k=max(c["k"], 1),
                        seed=c["seed"])
    torch.cuda.synchronize()
    assert np.array_equal(a["out_tokens"].cpu().numpy(), got["out_tokens"])
    assert np.array_equal(a["num_accepted"].cpu().numpy(), got["num_accepted"])
