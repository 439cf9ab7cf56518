"""Finds the draft-noise level of each position of the decaying-acceptance
workload (workloads.ROUNDS_WORKLOADS): the sigma for which the oracle's
acceptance probability beta = sum_y min(p(y), q(y)), averaged over seeded
rows of the workload's shape, equals the per-position rate measured at
gamma = 3 on the draft-model page ("초안 모델로 생성 속도를 높이는 추측
디코딩", section "맥북 실측: Gemma 4 12B": 0.951, 0.889, 0.852).

Calls only the oracle and the seeded generator.  Prints the sigmas; they are
copied into workloads.DECAY_SIGMAS, and tests/test_oracle_pins.py re-checks
them.  Run from the repository root: python tests/golden/make_decay_sigmas.py
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import workloads  # noqa: E402


def mean_beta(sigma: float, rows: int = 48) -> float:
    base = workloads.ROUNDS_WORKLOADS["rounds_decay_bf16_b512_g3_v128256"]
    wl = base.scaled(B=rows, G=1, sigma_pos=(sigma,), data_seed=7)
    inp = workloads.generate(wl)
    h = workloads.to_host_arrays
    res = oracle.verify(oracle.MODE_PROB, h(inp["target_logits"]), h(inp["draft_logits"]),
                        h(inp["draft_tokens"]), temperature=wl.temperature, seed=1, diagnostics=True)
    return float(res["beta"].mean())


def solve(alpha: float) -> float:
    lo, hi = 0.0, 3.0
    for _ in range(22):
        mid = 0.5 * (lo + hi)
        if mean_beta(mid) > alpha:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    for a in workloads.DECAY_ALPHAS:
        s = solve(a)
        print(f"alpha {a}: sigma {s:.4f} (mean beta {mean_beta(s):.4f})", flush=True)
