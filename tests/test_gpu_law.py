"""The vLLM page's worked 5-token example at its Monte Carlo size, on the GPU
(page "vLLM speculative decoding이 기각 토큰을 다시 뽑는 이유", section "Java로
규칙을 재현해 본 결과"; values in tests/golden/worked_example_5tok.txt):
2,000,000 requests with gamma 1 over a vocabulary of 5, target logits ln p,
draft logits ln q, draft tokens drawn from q (or argmax q for the greedy
drafter, the one-hot entry).  The GPU's acceptance rate must match the
page's within six binomial standard errors (plus the printed rounding), its
first-token law must lie within L1 0.003 of p, and every request must agree
with the oracle run on the same inputs and seed."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_5tok.txt")


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                r = line.split()
                rows[r[0]] = r[1:]
    return rows


@pytest.mark.parametrize("method", ["prob", "greedy"])
def test_five_token_table_on_gpu(sv, method):
    g = golden()
    p = np.array([float(v) for v in g["p"]])
    q = np.array([float(v) for v in g["q"]])
    n = int(g["trials"][0])
    printed = [float(v) for v in g[method]]
    rng = np.random.default_rng({"prob": 21, "greedy": 22}[method])
    lp = np.log(p).astype(np.float32)
    lq = np.log(q).astype(np.float32)
    lt = np.ascontiguousarray(np.broadcast_to(np.stack([lp, lp]), (n, 2, 5)))
    ld = np.ascontiguousarray(np.broadcast_to(lq[None], (n, 1, 5)))
    if method == "greedy":
        x = np.full((n, 1), int(np.argmax(q)), dtype=np.int32)
    else:
        x = rng.choice(5, size=(n, 1), p=q).astype(np.int32)
    entry = "prob" if method == "prob" else "onehot"
    print(f"[law] {method}: {n} requests, gamma 1, V 5", flush=True)
    res = sv.verify(entry, torch.from_numpy(lt).to(DEV), torch.from_numpy(x).to(DEV),
                    torch.from_numpy(ld).to(DEV) if entry == "prob" else None, temperature=1.0, top_k=0, seed=77)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in res.items() if k != "workspace"}
    acc = got["num_accepted"].mean()
    freq = np.bincount(got["out_tokens"][:, 0], minlength=5) / n
    l1 = np.abs(freq - p).sum()
    sd = math.sqrt(printed[0] * (1 - printed[0]) / n)
    print(f"[law] {method}: acceptance {acc:.4f} (page {printed[0]}), first-token law {np.round(freq, 4)}, "
          f"L1 {l1:.4f} (page {printed[6]})", flush=True)
    assert abs(acc - printed[0]) < 6 * sd + 1e-4
    assert l1 < 0.003
    ref = oracle.verify(oracle.MODE_PROB if entry == "prob" else oracle.MODE_ONEHOT, lt,
                        ld if entry == "prob" else None, x, temperature=1.0, seed=77, diagnostics=True)
    print(f"[law] {method}: against the oracle {assert_parity(entry, got, ref)}", flush=True)
