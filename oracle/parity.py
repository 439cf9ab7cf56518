"""Comparison of a verifier result with the oracle's (test infrastructure).

The bar (the reduction-order caveat of the manual page "투기적 디코딩",
section "정확성 기준"; the thresholds are the verifier's stated tolerances): p(x_j) and q(x_j) within an absolute
tolerance on every request; accepted lengths and every emitted token
identical on every request.  Two kinds of request may differ without failing,
and each such difference counts as an exemption *used*:
  * a request with a near-tie decision (relative margin <= 1e-4: an accept
    test or a race, oracle margins) at position j0 may differ from j0 on,
    but must agree before it;
  * a request whose top-p stop lies within ``cut_tol`` of flipping (both
    sides sum fp64 masses, so only rounding can move it).
Flagged requests are compared like every other; exemptions used are bounded
by ``max_exempt_fraction`` (default 1e-4) of the B (G + 1) rows, so on calls
of fewer than 10,000 rows none may be used.  The greedy path compares exact
input values and has no exemption at all.
"""

from __future__ import annotations

import numpy as np

from . import near_tie_position


def _exempt_bound(rows: int, frac: float | None) -> float:
    return float("inf") if frac is None else np.floor(frac * rows)


def compare(entry: str, got: dict, ref: dict, prob_tol: float = 1e-5, tie: float = 1e-4) -> dict:
    out_g, out_r = np.asarray(got["out_tokens"]), ref["out_tokens"]
    n_g, n_r = np.asarray(got["num_accepted"]), ref["num_accepted"]
    nreq, G1 = out_r.shape
    rep = {"requests": int(nreq), "rows": int(nreq * G1), "max_dp": 0.0, "max_dq": 0.0,
           "near_tie_requests": 0, "near_tie_rows": 0, "mismatch_non_tie": 0, "mismatch_tie": 0, "bad": []}
    if entry == "greedy":
        diff = np.nonzero((out_g != out_r).any(axis=1) | (n_g != n_r))[0]
        rep["mismatch_non_tie"] = int(diff.size)
        rep["bad"] = diff[:10].tolist()
        if "target_argmax" in got:
            rep["argmax_mismatch"] = int((np.asarray(got["target_argmax"]) != ref["target_argmax"]).sum())
        return rep
    if nreq:
        rep["max_dp"] = float(np.max(np.abs(np.asarray(got["p_draft"], np.float64) - ref["p_draft"])))
        if "q_draft" in got and got["q_draft"] is not None:
            rep["max_dq"] = float(np.max(np.abs(np.asarray(got["q_draft"], np.float64) - ref["q_draft"])))
    pos = near_tie_position(ref, tie)
    rep["near_tie_requests"] = int((pos >= 0).sum())
    rep["near_tie_rows"] = near_tie_rows(ref, tie)
    for r in range(nreq):
        same = (n_g[r] == n_r[r]) and bool((out_g[r] == out_r[r]).all())
        if same:
            continue
        if pos[r] >= 0:
            j0 = int(pos[r])
            if (out_g[r, :j0] == out_r[r, :j0]).all() and n_g[r] >= j0:
                rep["mismatch_tie"] += 1
                continue
        rep["mismatch_non_tie"] += 1
        if len(rep["bad"]) < 10:
            rep["bad"].append(r)
    return rep


def near_tie_rows(ref: dict, tie: float = 1e-4) -> int:
    """Number of (request, position) rows on which a decision the oracle took
    had a relative margin <= tie: the accept test of position j (every j <= n
    that was evaluated) and the race at position n.  The denominator of the
    near-tie fraction is B * (G + 1) rows."""
    if "accept_margin" not in ref:
        return 0
    am, rm, n = ref["accept_margin"], ref["race_margin"], ref["num_accepted"]
    G = am.shape[1]
    rows = 0
    for r in range(n.shape[0]):
        ev = min(int(n[r]) + 1, G)
        tied = set(np.nonzero(am[r, :ev] <= tie)[0].tolist())
        if rm[r] <= tie:
            tied.add(int(n[r]))
        rows += len(tied)
    return rows


def assert_parity(entry: str, got: dict, ref: dict, prob_tol: float = 1e-5, tie: float = 1e-4,
                  max_exempt_fraction: float | None = 1e-4) -> dict:
    """compare() and the bar: no difference outside near-ties, probabilities
    within prob_tol, and at most max_exempt_fraction of the rows (rounded
    down) spent on near-tie exemptions."""
    rep = compare(entry, got, ref, prob_tol, tie)
    assert rep["mismatch_non_tie"] == 0, f"token/length mismatch outside near-ties: {rep}"
    if entry == "greedy":
        assert rep.get("argmax_mismatch", 0) == 0, rep
    else:
        assert rep["max_dp"] <= prob_tol, rep
        assert rep["max_dq"] <= prob_tol, rep
    assert rep["mismatch_tie"] <= _exempt_bound(rep["rows"], max_exempt_fraction), \
        f"near-tie exemptions used beyond the bound: {rep}"
    return rep


def compare_batch(got: dict, ref: dict, prob_tol: float = 1e-5, tie: float = 1e-4, cut_tol: float = 1e-9) -> dict:
    """Per-request comparison of a batch call (per-request settings).

    Invalid requests: nothing emitted (tokens -1, n 0, p = q = 0), exactly.
    Temperature-0 requests: tokens, n and the 0/1 law p(x_j), q = 1, exactly.
    Sampled requests: the bar of ``compare``; a request whose oracle top-p
    stop had a margin below ``cut_tol`` is counted in ``near_cut_requests``,
    compared like the others, and a difference on it is counted in
    ``mismatch_cut`` (an exemption used).
    """
    out_g, out_r = np.asarray(got["out_tokens"]), ref["out_tokens"]
    n_g, n_r = np.asarray(got["num_accepted"]), ref["num_accepted"]
    pd_g, qd_g = np.asarray(got["p_draft"], np.float64), np.asarray(got["q_draft"], np.float64)
    nreq, G1 = out_r.shape
    pos = near_tie_position(ref, tie)
    rep = {"requests": int(nreq), "rows": int(nreq * G1), "max_dp": 0.0, "max_dq": 0.0, "near_tie_requests": 0,
           "near_tie_rows": near_tie_rows(ref, tie), "near_cut_requests": 0, "mismatch_non_tie": 0,
           "mismatch_tie": 0, "mismatch_cut": 0, "greedy_requests": 0, "invalid_requests": 0, "bad": []}

    def fail(r):
        rep["mismatch_non_tie"] += 1
        if len(rep["bad"]) < 10:
            rep["bad"].append(r)

    for r in range(nreq):
        same = (n_g[r] == n_r[r]) and bool((out_g[r] == out_r[r]).all())
        g = int(ref["lengths"][r]) if "lengths" in ref else pd_g.shape[1]
        if ref["bad_param"][r]:
            rep["invalid_requests"] += 1
            if not same or (pd_g[r, :g] != 0).any() or (qd_g[r, :g] != 0).any():
                fail(r)
            continue
        if ref["greedy"][r]:
            rep["greedy_requests"] += 1
            if not same or (pd_g[r, :g] != ref["p_draft"][r, :g]).any() or (qd_g[r, :g] != ref["q_draft"][r, :g]).any():
                fail(r)
            continue
        near_cut = ref["cut_margin"][r] < cut_tol
        rep["near_cut_requests"] += int(near_cut)
        if g:
            rep["max_dp"] = max(rep["max_dp"], float(np.max(np.abs(pd_g[r, :g] - ref["p_draft"][r, :g]))))
            rep["max_dq"] = max(rep["max_dq"], float(np.max(np.abs(qd_g[r, :g] - ref["q_draft"][r, :g]))))
        if pos[r] >= 0:
            rep["near_tie_requests"] += 1
        if same:
            continue
        if pos[r] >= 0:
            j0 = int(pos[r])
            if (out_g[r, :j0] == out_r[r, :j0]).all() and n_g[r] >= j0:
                rep["mismatch_tie"] += 1
                continue
        if near_cut:
            rep["mismatch_cut"] += 1
            continue
        fail(r)
    return rep


def assert_parity_batch(got: dict, ref: dict, prob_tol: float = 1e-5, tie: float = 1e-4, cut_tol: float = 1e-9,
                        max_exempt_fraction: float | None = 1e-4) -> dict:
    rep = compare_batch(got, ref, prob_tol, tie, cut_tol)
    assert rep["mismatch_non_tie"] == 0, f"mismatch outside near-ties: {rep}"
    assert rep["max_dp"] <= prob_tol and rep["max_dq"] <= prob_tol, rep
    assert rep["mismatch_tie"] + rep["mismatch_cut"] <= _exempt_bound(rep["rows"], max_exempt_fraction), \
        f"exemptions used beyond the bound: {rep}"
    return rep
