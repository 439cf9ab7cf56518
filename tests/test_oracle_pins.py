"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with itself: each checks a printed
value, a closed form, an exact identity, an independent implementation that
is run (not copied), or a brute-force enumeration.  A plausible slip in the
oracle (a dropped max(0, .), a swapped p and q, a resample from p instead of
the residual, a wrong counter word, a flipped tie rule) fails at least one.
"""

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.parity import compare_batch, near_tie_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HELPERS = os.path.join(os.path.dirname(__file__), "helpers")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _f32_logits(probs):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(probs, dtype=np.float64)).astype(np.float32)


# ---------------------------------------------------------------------------
# Philox4x32-10 and the uniform mapping
# ---------------------------------------------------------------------------

def test_philox_known_answers():
    for r in _read_golden("philox4x32_10_kat.txt"):
        vals = [int(v, 16) for v in r]
        ctr, key, want = vals[0:4], vals[4:6], vals[6:10]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_philox_matches_aten_engine_runs():
    """Bit-equality with ATen's independent header-only Philox engine, run on
    1000 random counter/key blocks."""
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not shutil.which("g++") or not os.path.isdir(inc):
        pytest.skip("g++ or torch headers unavailable")
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "aten_philox")
        subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, os.path.join(HELPERS, "aten_philox.cpp"),
                        "-o", exe], check=True)
        rng = np.random.default_rng(1234)
        blocks = rng.integers(0, 2**32, size=(1000, 6), dtype=np.uint64)
        blocks[:10, :4] = 0  # include tiny counters
        stdin = "\n".join(" ".join(f"{int(v):08x}" for v in row) for row in blocks) + "\n"
        out = subprocess.run([exe], input=stdin, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(blocks, out):
        want = [int(v, 16) for v in line.split()]
        got = list(oracle.philox4x32_10(row[:4], row[4:6]))
        assert got == want


def _unit_from_words(lo, hi):
    k53 = ((int(hi) << 32) | int(lo)) >> 11
    return (k53 + 1) / 2.0**53


def test_uniform_streams_use_documented_counters():
    seed = 0x0123456789ABCDEF
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for b, j in [(0, 0), (5, 3), (1023, 8), (2**31 - 1, 7)]:
        w = oracle.philox4x32_10([0, j, b, 0], key)
        assert oracle.uniform_accept(seed, b, j) == _unit_from_words(w[0], w[1])
        for y in [0, 1, 2, 3, 255998, 255999]:
            w = oracle.philox4x32_10([y >> 1, j, b, 1], key)
            want = _unit_from_words(w[0], w[1]) if y % 2 == 0 else _unit_from_words(w[2], w[3])
            assert oracle.uniform_race(seed, b, j, y) == want


def test_uniforms_in_half_open_unit_interval_and_uniform():
    u = np.array([oracle.uniform_accept(42, b, j) for b in range(2000) for j in range(8)])
    assert np.all(u > 0.0) and np.all(u <= 1.0)
    assert np.all(np.floor(u * 2.0**53) == u * 2.0**53)  # multiples of 2^-53
    assert stats.kstest(u, "uniform").pvalue > 1e-4


# ---------------------------------------------------------------------------
# Adjusted distribution of one position: temperature, top-k, softmax
# ---------------------------------------------------------------------------

def test_temperature_closed_form():
    # l = T * ln(w)  =>  softmax(l / T) = w / sum(w).
    w = np.array([1.0, 2.0, 3.0, 4.0])
    for T in [0.5, 0.7, 1.0, 2.0]:
        l = (T * np.log(w)).astype(np.float32)
        want = np.exp(l.astype(np.float64) / T)
        want /= want.sum()
        got = oracle.row_probs(l, T)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
        np.testing.assert_allclose(got, w / w.sum(), rtol=1e-6)


def test_temperature_peaks_the_law():
    rng = np.random.default_rng(0)
    l = (rng.standard_normal(64) * 3).astype(np.float32)
    p1, p07, p2 = (oracle.row_probs(l, T) for T in (1.0, 0.7, 2.0))
    top = int(np.argmax(l))
    assert p07[top] > p1[top] > p2[top]
    for p in (p1, p07, p2):
        assert abs(p.sum() - 1.0) < 1e-12


def test_topk_keeps_k_largest_with_lowest_index_ties():
    # All equal: the first k indices are kept.
    l = np.zeros(10, dtype=np.float32)
    p = oracle.row_probs(l, 1.0, top_k=3)
    np.testing.assert_array_equal(p, [1 / 3, 1 / 3, 1 / 3] + [0.0] * 7)
    # A tie straddling the k-th place: ranks by (value desc, index asc).
    l = np.array([1, 5, 3, 5, 3, 3, 0], dtype=np.float32)
    p = oracle.row_probs(l, 1.0, top_k=4)
    kept = np.nonzero(p)[0].tolist()
    assert kept == [1, 2, 3, 4]
    r = np.exp(5.0 - 3.0)
    np.testing.assert_allclose(p[[1, 3]], r / (2 * r + 2), rtol=1e-14)
    np.testing.assert_allclose(p[[2, 4]], 1 / (2 * r + 2), rtol=1e-14)


def test_topk_random_rows_against_sorted_reference():
    rng = np.random.default_rng(7)
    for V, k in [(50, 1), (50, 7), (300, 64), (1000, 64)]:
        l = np.round(rng.standard_normal(V) * 4, 1).astype(np.float32)  # many ties
        order = sorted(range(V), key=lambda y: (-float(l[y]), y))
        kept = sorted(order[:k])
        p = oracle.row_probs(l, 0.7, top_k=k)
        assert np.nonzero(p)[0].tolist() == kept
        # Ratios inside the kept set follow exp((l_a - l_b) / T).
        a, c = kept[0], kept[-1]
        assert math.isclose(p[a] / p[c], math.exp((float(l[a]) - float(l[c])) / 0.7), rel_tol=1e-12)
        assert abs(p.sum() - 1.0) < 1e-12


def test_topk_at_or_above_vocab_is_off():
    l = np.random.default_rng(1).standard_normal(33).astype(np.float32)
    base = oracle.row_probs(l, 0.8, 0)
    for k in (33, 34, 1000):
        np.testing.assert_array_equal(oracle.row_probs(l, 0.8, k), base)


def test_neg_inf_logits_have_zero_mass_and_bf16_decoding():
    # bf16 bit patterns: 0x3F80 = 1.0, 0x4000 = 2.0, 0xFF80 = -inf, 0x0000 = 0.
    bits = np.array([0x3F80, 0x4000, 0xFF80, 0x0000], dtype=np.uint16)
    p = oracle.row_probs(bits, 1.0)
    e = np.exp([1.0, 2.0, 0.0])
    np.testing.assert_allclose(p[[0, 1, 3]], e / e.sum(), rtol=1e-14)
    assert p[2] == 0.0
    assert oracle.row_argmax(bits) == 1
    assert oracle.row_argmax(np.array([0xC000, 0x3F80, 0x3F80], dtype=np.uint16)) == 1  # tie -> lowest


# ---------------------------------------------------------------------------
# The Exp(1) race
# ---------------------------------------------------------------------------

def test_race_law_chi_square():
    w = np.array([0.1, 0.0, 0.5, 0.2, 0.2, 0.0, 1e-3])
    n = 200_000
    counts = np.zeros(w.size)
    for b in range(n):
        tok, _ = oracle.race(w, 99, b, 3)
        counts[tok] += 1
    assert counts[1] == 0 and counts[5] == 0  # zero weight never wins
    pos = w > 0
    chi = stats.chisquare(counts[pos], n * w[pos] / w.sum())
    assert chi.pvalue > 1e-6


def test_zero_residual_fallback_law():
    """Equal target and draft laws at a position rejected only because its
    draft token is out of range: max(p - q, 0) is 0 everywhere, and the
    token drawn there must follow p itself (the zero-mass reading).  Over
    40,000 requests its frequencies match p (chi-square); emitting nothing
    (-1) or racing on the masked or uniform law would fail."""
    p = np.array([0.5, 0.3, 0.15, 0.05])
    n = 40_000
    row = np.log(p).astype(np.float32)
    lt = np.ascontiguousarray(np.broadcast_to(row, (n, 2, 4)))
    ld = np.ascontiguousarray(np.broadcast_to(row, (n, 1, 4)))
    x = np.full((n, 1), 4, np.int32)  # out of range: rejected at position 0
    ref = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.0, seed=17)
    assert (ref["num_accepted"] == 0).all() and ref["bad_token"].all()
    tok = ref["out_tokens"][:, 0]
    assert (tok >= 0).all() and (ref["out_tokens"][:, 1] == -1).all()
    counts = np.bincount(tok, minlength=4)
    assert stats.chisquare(counts, n * p).pvalue > 1e-6
    assert stats.chisquare(counts, n * np.full(4, 0.25)).pvalue < 1e-12


def test_race_wrong_law_is_detected():
    """Power check: a plausible slip (racing on p instead of the residual)
    is far outside the chi-square acceptance region used above."""
    w = np.array([0.1, 0.5, 0.2, 0.2])
    wrong = np.array([0.25, 0.25, 0.25, 0.25])
    n = 50_000
    counts = np.zeros(4)
    for b in range(n):
        counts[oracle.race(wrong, 5, b, 0)[0]] += 1
    assert stats.chisquare(counts, n * w / w.sum()).pvalue < 1e-12


# ---------------------------------------------------------------------------
# The worked 5-token example and its Monte Carlo table
# ---------------------------------------------------------------------------

def _worked():
    g = {r[0]: r[1:] for r in _read_golden("worked_example_5tok.txt")}
    p = np.array([float(v) for v in g["p"]])
    q = np.array([float(v) for v in g["q"]])
    return p, q, g


def _single_position_batch(p, q, n, rng, onehot=False):
    """n requests with gamma = 1: position 0 carries the draft, row 1 is the
    bonus position.  Draft tokens are drawn from q (or argmax q)."""
    lp, lq = _f32_logits(p), _f32_logits(q)
    lt = np.broadcast_to(np.stack([lp, lp]), (n, 2, p.size)).copy()
    ld = np.broadcast_to(lq[None], (n, 1, q.size)).copy()
    if onehot:
        x = np.full((n, 1), int(np.argmax(q)), dtype=np.int32)
    else:
        x = rng.choice(p.size, size=(n, 1), p=q).astype(np.int32)
    return lt, ld, x


def test_worked_example_acceptance_identities():
    p, q, g = _worked()
    lt, ld, x = _single_position_batch(p, q, 1, np.random.default_rng(0))
    res = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.0, diagnostics=True)
    assert abs(res["beta"][0, 0] - float(g["sum_min_pq"][0])) < 1e-6
    res = oracle.verify(oracle.MODE_ONEHOT, lt, None, np.array([[int(np.argmax(q))]], np.int32),
                        diagnostics=True)
    assert abs(res["p_draft"][0, 0] - float(g["p_at_argmax_q"][0])) < 1e-6
    assert res["q_draft"][0, 0] == 1.0


@pytest.mark.parametrize("method", ["prob", "greedy", "naive"])
def test_worked_example_monte_carlo_table(method):
    """Reruns the page's 2e6-trial table: acceptance rate, output law, L1."""
    p, q, g = _worked()
    n = int(g["trials"][0])
    printed = {r[0]: [float(v) for v in r[1:]] for r in _read_golden("worked_example_5tok.txt")
               if r[0] in ("prob", "greedy", "naive")}[method]
    rng = np.random.default_rng({"prob": 11, "greedy": 12, "naive": 13}[method])
    lt, ld, x = _single_position_batch(p, q, n, rng, onehot=(method == "greedy"))
    mode = {"prob": oracle.MODE_PROB, "greedy": oracle.MODE_ONEHOT, "naive": oracle.MODE_NAIVE}[method]
    res = oracle.verify(mode, lt, ld if method != "greedy" else None, x, temperature=1.0, seed=42)
    acc = res["num_accepted"].mean()
    freq = np.bincount(res["out_tokens"][:, 0], minlength=5) / n
    l1 = np.abs(freq - p).sum()
    sd_acc = math.sqrt(printed[0] * (1 - printed[0]) / n)
    assert abs(acc - printed[0]) < 6 * sd_acc + 1e-4          # printed to 4 decimals
    if method == "naive":
        # Exact naive law min(p, q) + (1 - beta) p; first token 0.425.
        beta = np.minimum(p, q).sum()
        law = np.minimum(p, q) + (1 - beta) * p
        assert abs(law[0] - float(g["naive_first_token"][0])) < 1e-12
        assert abs(freq[0] - 0.425) < 5 * math.sqrt(0.425 * 0.575 / n)
        assert abs(l1 - printed[6]) < 0.003
        assert stats.chisquare(freq * n, law * n).pvalue > 1e-6
    else:
        assert l1 < 0.003
        assert stats.chisquare(freq * n, p * n).pvalue > 1e-6
    np.testing.assert_allclose(freq, printed[1:6], atol=6 * math.sqrt(0.25 / n) + 1e-4)


# ---------------------------------------------------------------------------
# Eq. 1 and the law of the accepted length
# ---------------------------------------------------------------------------

def _eq1(alpha, gamma):
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


def test_eq1_printed_values():
    for r in _read_golden("eq1_expected_tokens.txt"):
        if r[0] == "compute":
            a, gm, val, dec = float(r[1]), int(r[2]), float(r[3]), int(r[4])
            assert round((gm + 1) / _eq1(a, gm), dec) == val
        else:
            a, gm, val, dec = float(r[0]), int(r[1]), float(r[2]), int(r[3])
            assert round(_eq1(a, gm), dec) == val


def _iid_onehot_rows(alpha, gamma, n):
    """One-hot rows whose draft token has target probability alpha at every
    position: each position accepts independently with probability alpha."""
    l = _f32_logits([alpha, 1 - alpha])
    lt = np.broadcast_to(l[None, None], (n, gamma + 1, 2)).copy()
    x = np.zeros((n, gamma), dtype=np.int32)
    return lt, x


@pytest.mark.parametrize("alpha,gamma", [(0.8, 5), (0.901, 3), (0.75, 7), (0.9, 7)])
def test_mean_tokens_per_round_matches_eq1(alpha, gamma):
    n = 200_000
    lt, x = _iid_onehot_rows(alpha, gamma, n)
    res = oracle.verify(oracle.MODE_ONEHOT, lt, None, x, temperature=1.0, seed=7, diagnostics=True)
    a_eff = float(res["beta"][0, 0])  # p(x) after fp32 rounding of the logits
    assert abs(a_eff - alpha) < 1e-6
    tokens = res["num_accepted"] + 1
    se = tokens.std() / math.sqrt(n)
    assert abs(tokens.mean() - _eq1(a_eff, gamma)) < 5 * se
    # Law of n: P(n = k) = alpha^k (1 - alpha) for k < gamma, alpha^gamma at gamma.
    k = np.arange(gamma + 1)
    law = np.where(k < gamma, a_eff ** k * (1 - a_eff), a_eff ** gamma)
    counts = np.bincount(res["num_accepted"], minlength=gamma + 1)
    assert stats.chisquare(counts, law * n).pvalue > 1e-6


def test_greedy_iid_matches_and_invariants():
    """Greedy rows where each draft equals the target argmax with prob 0.8."""
    rng = np.random.default_rng(3)
    n, G, V = 20_000, 5, 17
    lt = rng.standard_normal((n, G + 1, V)).astype(np.float32)
    amax = np.argmax(lt, axis=-1)
    match = rng.random((n, G)) < 0.8
    other = (amax[:, :G] + 1 + rng.integers(0, V - 1, (n, G))) % V
    x = np.where(match, amax[:, :G], other).astype(np.int32)
    res = oracle.verify(oracle.MODE_GREEDY, lt, None, x)
    nacc, out = res["num_accepted"], res["out_tokens"]
    np.testing.assert_array_equal(res["target_argmax"], amax)
    for r in range(200):
        k = nacc[r]
        assert (out[r, :k] == x[r, :k]).all() and (x[r, :k] == amax[r, :k]).all()
        assert out[r, k] == amax[r, k] and (k == G or x[r, k] != amax[r, k])
        assert (out[r, k + 1:] == -1).all()
    tokens = nacc + 1
    assert abs(tokens.mean() - _eq1(0.8, G)) < 5 * tokens.std() / math.sqrt(n)


# ---------------------------------------------------------------------------
# Brute-force enumeration at V <= 4
# ---------------------------------------------------------------------------

def _exact_outcome_law(p, q, mode):
    """Exact law of (n, emitted tokens) by enumerating every draft sequence.
    p: [G+1][V], q: [G][V] (rows of the adjusted laws)."""
    G, V = q.shape if mode == "prob" else (p.shape[0] - 1, p.shape[1])
    law = {}
    import itertools

    if mode == "prob":
        seqs = itertools.product(range(V), repeat=G)
    else:  # onehot: the draft is the fixed q-argmax sequence
        seqs = [tuple(int(np.argmax(q[j])) for j in range(G))]
    for xs in seqs:
        w = np.prod([q[j][xs[j]] for j in range(G)]) if mode == "prob" else 1.0
        if w == 0:
            continue
        reach = w
        for j in range(G + 1):
            if j == G:
                for y in range(V):
                    if p[G][y] > 0:
                        key = (G, xs + (y,))
                        law[key] = law.get(key, 0.0) + reach * p[G][y]
                break
            x = xs[j]
            qx = q[j][x] if mode == "prob" else 1.0
            a = min(1.0, p[j][x] / qx) if qx > 0 else 0.0
            rej = reach * (1 - a)
            if rej > 0:
                if mode == "prob":
                    r = np.maximum(p[j] - q[j], 0)
                else:
                    r = p[j].copy()
                    r[x] = 0
                r = r / r.sum()
                for y in range(V):
                    if r[y] > 0:
                        key = (j, xs[:j] + (y,))
                        law[key] = law.get(key, 0.0) + rej * r[y]
            reach *= a
            if reach == 0:
                break
    return law


def _check_brute_force(lt, ld, mode, n_runs, seed, top_k=0, T=1.0):
    G = lt.shape[0] - 1
    V = lt.shape[1]
    p = np.stack([oracle.row_probs(lt[j], T, top_k) for j in range(G + 1)])
    if mode == "prob":
        q = np.stack([oracle.row_probs(ld[j], T, top_k) for j in range(G)])
    else:
        q = np.zeros((G, V))
        q[np.arange(G), np.argmax(ld, axis=-1)] = 1.0
    law = _exact_outcome_law(p, q, mode)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    # Losslessness: the token emitted at each reached position follows p_j,
    # and the accepted length follows prod(beta_i) (1 - beta_k).
    beta = [np.minimum(p[j], q[j]).sum() for j in range(G)]
    for j in range(G + 1):
        reach = np.prod(beta[:j])
        marg = np.zeros(V)
        for (k, toks), pr in law.items():
            if k >= j:
                marg[toks[j]] += pr
        np.testing.assert_allclose(marg, reach * p[j], atol=1e-12)
    for k in range(G + 1):
        pk = sum(pr for (kk, _), pr in law.items() if kk == k)
        want = np.prod(beta[:k]) * ((1 - beta[k]) if k < G else 1.0)
        assert abs(pk - want) < 1e-12
    # Empirical law of the oracle over n_runs independent requests.
    rng = np.random.default_rng(seed)
    ltb = np.broadcast_to(lt[None], (n_runs,) + lt.shape).copy()
    if mode == "prob":
        ldb = np.broadcast_to(ld[None], (n_runs,) + ld.shape).copy()
        x = np.stack([rng.choice(V, size=n_runs, p=q[j]) for j in range(G)], axis=1).astype(np.int32)
        res = oracle.verify(oracle.MODE_PROB, ltb, ldb, x, temperature=T, top_k=top_k, seed=seed)
    else:
        x = np.broadcast_to(np.argmax(ld, axis=-1)[None].astype(np.int32), (n_runs, G)).copy()
        res = oracle.verify(oracle.MODE_ONEHOT, ltb, None, x, temperature=T, top_k=top_k, seed=seed)
    keys = list(law)
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for r in range(n_runs):
        k = int(res["num_accepted"][r])
        toks = tuple(int(t) for t in res["out_tokens"][r, :k + 1])
        assert (k, toks) in index, f"impossible outcome {(k, toks)}"
        counts[index[(k, toks)]] += 1
    expected = np.array([law[k] for k in keys]) * n_runs
    big = expected >= 5
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(expected[big], expected[~big].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    if len(exp) > 1:
        assert stats.chisquare(obs, exp).pvalue > 1e-6


def _logits(rows):
    return _f32_logits(rows)


@pytest.mark.parametrize("case", ["generic", "zeros", "equal", "v1", "topk1"])
def test_brute_force_prob(case):
    rng = np.random.default_rng(hash(case) % 2**32)
    if case == "generic":
        lt = (rng.standard_normal((3, 3)) * 1.5).astype(np.float32)
        ld = (rng.standard_normal((2, 3)) * 1.5).astype(np.float32)
        _check_brute_force(lt, ld, "prob", 200_000, 1)
    elif case == "zeros":  # zeros in p and in q
        lt = _logits([[0.5, 0.0, 0.3, 0.2], [0.0, 0.6, 0.4, 0.0], [0.1, 0.2, 0.3, 0.4]])
        ld = _logits([[0.2, 0.4, 0.0, 0.4], [0.3, 0.3, 0.4, 0.0]])
        _check_brute_force(lt, ld, "prob", 200_000, 2)
    elif case == "equal":  # q == p: never rejected, n = G always
        lt = (rng.standard_normal((4, 4))).astype(np.float32)
        _check_brute_force(lt, lt[:3].copy(), "prob", 100_000, 3)
    elif case == "v1":
        lt = np.zeros((3, 1), dtype=np.float32)
        _check_brute_force(lt, np.zeros((2, 1), dtype=np.float32), "prob", 1000, 4)
    elif case == "topk1":
        lt = (rng.standard_normal((3, 4)) * 2).astype(np.float32)
        ld = (rng.standard_normal((2, 4)) * 2).astype(np.float32)
        _check_brute_force(lt, ld, "prob", 20_000, 5, top_k=1)


def test_brute_force_onehot():
    rng = np.random.default_rng(9)
    lt = (rng.standard_normal((4, 4)) * 1.2).astype(np.float32)
    ld = (rng.standard_normal((3, 4)) * 1.2).astype(np.float32)
    _check_brute_force(lt, ld, "onehot", 200_000, 6, T=0.8)


def test_brute_force_detects_naive_resampling():
    """Power check: the deliberately wrong naive mode (resample from p after a
    rejection) fails the same chi-square that the real rule passes."""
    lt = _logits([[0.5, 0.25, 0.15, 0.1], [0.25, 0.25, 0.25, 0.25]])
    ld = _logits([[0.3, 0.4, 0.1, 0.2]])
    p = np.stack([oracle.row_probs(lt[j], 1.0) for j in range(2)])
    q = oracle.row_probs(ld[0], 1.0)[None]
    law = _exact_outcome_law(p, q, "prob")
    n = 100_000
    rng = np.random.default_rng(8)
    x = rng.choice(4, size=(n, 1), p=q[0]).astype(np.int32)
    res = oracle.verify(oracle.MODE_NAIVE, np.broadcast_to(lt[None], (n, 2, 4)).copy(),
                        np.broadcast_to(ld[None], (n, 1, 4)).copy(), x, seed=1)
    first = np.bincount(res["out_tokens"][:, 0], minlength=4)
    want = np.zeros(4)
    for (k, toks), pr in law.items():
        want[toks[0]] += pr
    assert stats.chisquare(first, want * n).pvalue < 1e-12


# ---------------------------------------------------------------------------
# Exact reductions between the modes, and special cases
# ---------------------------------------------------------------------------

def test_topk1_prob_equals_greedy():
    rng = np.random.default_rng(21)
    n, G, V = 300, 4, 50
    lt = (rng.standard_normal((n, G + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :G] + rng.standard_normal((n, G, V))).astype(np.float32)
    x = np.argmax(ld, axis=-1).astype(np.int32)
    a = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=0.9, top_k=1, seed=5)
    g = oracle.verify(oracle.MODE_GREEDY, lt, None, x)
    np.testing.assert_array_equal(a["num_accepted"], g["num_accepted"])
    np.testing.assert_array_equal(a["out_tokens"], g["out_tokens"])
    assert 0 < g["num_accepted"].mean() < G  # both outcomes present


def test_onehot_by_logits_prob_equals_onehot():
    rng = np.random.default_rng(22)
    n, G, V = 400, 3, 40
    lt = (rng.standard_normal((n, G + 1, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, (n, G)).astype(np.int32)
    ld = np.full((n, G, V), -np.inf, dtype=np.float32)
    np.put_along_axis(ld, x[..., None], 0.0, axis=-1)
    a = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.3, seed=77)
    o = oracle.verify(oracle.MODE_ONEHOT, lt, None, x, temperature=1.3, seed=77)
    np.testing.assert_array_equal(a["out_tokens"], o["out_tokens"])
    np.testing.assert_array_equal(a["num_accepted"], o["num_accepted"])
    np.testing.assert_array_equal(a["p_draft"], o["p_draft"])


def test_p_zero_always_rejected_and_q_equal_p_never():
    rng = np.random.default_rng(23)
    n, G, V = 500, 3, 30
    lt = (rng.standard_normal((n, G + 1, V))).astype(np.float32)
    # Draft tokens outside the target's top-5: p(x) = 0 after top-k.
    order = np.argsort(-lt[:, :G], axis=-1, kind="stable")
    x = order[..., 10].astype(np.int32)
    ld = lt[:, :G].copy()
    r = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.0, top_k=5)
    assert (r["num_accepted"] == 0).all()
    assert (r["p_draft"][:, 0] == 0).all()
    # q = p: every draft accepted, the bonus follows.
    x2 = rng.integers(0, V, (n, G)).astype(np.int32)
    r2 = oracle.verify(oracle.MODE_PROB, lt, ld, x2, temperature=1.0)
    assert (r2["num_accepted"] == G).all()


def test_accounting_and_padding():
    rng = np.random.default_rng(24)
    n, G, V = 1000, 6, 20
    lt = (rng.standard_normal((n, G + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :G] + rng.standard_normal((n, G, V))).astype(np.float32)
    x = rng.integers(0, V, (n, G)).astype(np.int32)
    r = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.0, seed=3)
    emitted = (r["out_tokens"] >= 0).sum(axis=1)
    np.testing.assert_array_equal(emitted, r["num_accepted"] + 1)
    for k in range(n):
        m = r["num_accepted"][k]
        assert (r["out_tokens"][k, :m] == x[k, :m]).all()


def test_out_of_range_draft_token_is_rejected_and_flagged():
    lt = np.zeros((2, 3, 4), dtype=np.float32)
    ld = np.zeros((2, 2, 4), dtype=np.float32)
    x = np.array([[1, 7], [-1, 0]], dtype=np.int32)
    r = oracle.verify(oracle.MODE_PROB, lt, ld, x, temperature=1.0)
    assert r["num_accepted"][0] == 1 and r["num_accepted"][1] == 0
    assert r["bad_token"].tolist() == [1, 1]
    assert r["p_draft"][0, 1] == 0.0 and r["q_draft"][1, 0] == 0.0
    g = oracle.verify(oracle.MODE_GREEDY, lt, None, x)
    assert g["num_accepted"].tolist() == [0, 0]  # argmax of all-zero rows is 0


def test_argument_validation():
    lt = np.zeros((1, 2, 4), dtype=np.float32)
    x = np.zeros((1, 1), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.verify(oracle.MODE_ONEHOT, lt, None, x, temperature=0.0)
    with pytest.raises(ValueError):
        oracle.verify(oracle.MODE_PROB, lt, None, x, temperature=1.0)
    with pytest.raises(ValueError):
        oracle.verify(oracle.MODE_ONEHOT, lt, None, x, temperature=1.0, top_k=-1)


# ---------------------------------------------------------------------------
# Top-p (nucleus) after temperature and top-k; per-request settings
# ---------------------------------------------------------------------------

def test_top_p_closed_forms():
    """Law (0.5, 0.3, 0.15, 0.05): the nucleus is the shortest rank prefix
    whose mass reaches top_p, renormalised (hand-computed values)."""
    lt = _f32_logits([0.5, 0.3, 0.15, 0.05])
    cases = {
        1e-30: [1.0, 0, 0, 0],
        0.45: [1.0, 0, 0, 0],
        0.5 - 1e-6: [1.0, 0, 0, 0],
        0.55: [0.625, 0.375, 0, 0],
        0.79: [0.625, 0.375, 0, 0],
        0.81: [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0],
        0.96: [0.5, 0.3, 0.15, 0.05],
    }
    for top_p, want in cases.items():
        got, margin = oracle.row_probs(lt, 1.0, 0, top_p, return_margin=True)
        np.testing.assert_allclose(got, want, atol=2e-7, err_msg=f"top_p={top_p}")
    # Margins: distance of top_p to the nearest cumulative mass.
    assert abs(oracle.row_probs(lt, 1.0, 0, 0.55, return_margin=True)[1] - 0.05) < 1e-7
    assert abs(oracle.row_probs(lt, 1.0, 0, 0.79, return_margin=True)[1] - 0.01) < 1e-7
    # top_p = 1 is off, identical to the law without it.
    np.testing.assert_array_equal(oracle.row_probs(lt, 0.7, 0, 1.0), oracle.row_probs(lt, 0.7, 0))


def test_top_p_ties_go_to_the_lowest_index():
    # Flat row: every token 1/10; 0.45 needs five tokens, 0.55 six.
    flat = np.zeros(10, dtype=np.float32)
    np.testing.assert_allclose(oracle.row_probs(flat, 1.0, 0, 0.45), [0.2] * 5 + [0] * 5, atol=1e-15)
    np.testing.assert_allclose(oracle.row_probs(flat, 1.0, 0, 0.55), [1 / 6] * 6 + [0] * 4, atol=1e-15)
    # Three tied maxima at 1, 3, 5 (mass e^2 / (3 e^2 + 4) = 0.2823 each):
    # top_p 0.5 takes two of them, the two lowest indices.
    row = np.array([0, 2, 0, 2, 0, 2, 0], dtype=np.float32)
    np.testing.assert_allclose(oracle.row_probs(row, 1.0, 0, 0.5), [0, 0.5, 0, 0.5, 0, 0, 0], atol=1e-15)
    # Mass that equals top_p exactly reaches it: 0.25 + 0.25 = 0.5 keeps two.
    np.testing.assert_allclose(oracle.row_probs(np.zeros(4, np.float32), 1.0, 0, 0.5), [0.5, 0.5, 0, 0],
                               atol=1e-15)
    # The largest fp32 below 1 keeps every token of a flat row.
    top = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    np.testing.assert_allclose(oracle.row_probs(flat, 1.0, 0, top), [0.1] * 10, atol=1e-15)


def test_top_p_applies_after_temperature():
    """Logits (2, 1, 0), top_p 0.8: at T = 1 the law (e^2, e, 1) / 11.107 needs
    two tokens (0.665 < 0.8 <= 0.910); at T = 0.5 the law (e^4, e^2, 1) / 62.99
    needs one (0.867).  Cutting at T = 1 and then sharpening would keep two."""
    row = np.array([2, 1, 0], dtype=np.float32)
    e = math.e
    np.testing.assert_allclose(oracle.row_probs(row, 1.0, 0, 0.8), [e / (e + 1), 1 / (e + 1), 0], atol=1e-7)
    np.testing.assert_allclose(oracle.row_probs(row, 0.5, 0, 0.8), [1, 0, 0], atol=1e-15)


def test_top_p_applies_to_the_top_k_law():
    """Logits (3, 2, 1, 0): after top-2 the law is (e^3, e^2) / (e^3 + e^2),
    0.731 >= 0.72, so top_p 0.72 keeps one token; on the untruncated law
    (0.644 < 0.72) it would keep two.  After top-3, top_p 0.9 keeps two
    (0.6652 + 0.2447 = 0.9100)."""
    row = np.array([3, 2, 1, 0], dtype=np.float32)
    e = math.e
    np.testing.assert_allclose(oracle.row_probs(row, 1.0, 2, 0.72), [1, 0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(oracle.row_probs(row, 1.0, 0, 0.72), [e / (e + 1), 1 / (e + 1), 0, 0], atol=1e-7)
    np.testing.assert_allclose(oracle.row_probs(row, 1.0, 3, 0.9), [e / (e + 1), 1 / (e + 1), 0, 0], atol=1e-7)


@pytest.mark.parametrize("top_k", [0, 7, 40])
def test_top_p_invariants_on_random_rows(top_k):
    """On random rows: the nucleus is a rank prefix of the top-k set; its mass
    under the top-k law reaches top_p and falls short of it without its last
    token; on it the law is proportional to exp(l / T) and sums to 1."""
    rng = np.random.default_rng(17 + top_k)
    for it in range(40):
        V = int(rng.integers(2, 300))
        row = (rng.standard_normal(V) * rng.uniform(0.3, 4)).astype(np.float32)
        if it % 5 == 0:
            row = np.round(row).astype(np.float32)  # many ties
        T = float(rng.uniform(0.3, 2.0))
        top_p = float(rng.uniform(0.05, 0.99))
        p = oracle.row_probs(row, T, top_k, top_p)
        base = oracle.row_probs(row, T, top_k)
        rank = sorted(range(V), key=lambda y: (-float(row[y]), y))
        kept = [y for y in rank if p[y] > 0]
        assert kept == rank[:len(kept)], "nucleus is not a rank prefix"
        mass = sum(base[y] for y in kept)
        assert mass >= top_p - 1e-12
        assert mass - base[kept[-1]] < top_p + 1e-12
        z = row[kept].astype(np.float64) / T
        w = np.exp(z - z.max())
        np.testing.assert_allclose(p[kept], w / w.sum(), rtol=1e-12)
        assert abs(p.sum() - 1.0) < 1e-12


def test_brute_force_top_p():
    """Losslessness with the nucleus law: the exact outcome law of the
    verification, and the oracle's empirical one, with top-p on p and q."""
    rng = np.random.default_rng(23)
    lt = (rng.standard_normal((3, 4)) * 1.5).astype(np.float32)
    ld = (rng.standard_normal((2, 4)) * 1.5).astype(np.float32)
    G, V, n_runs, T, top_p = 2, 4, 100_000, 0.9, 0.8
    p = np.stack([oracle.row_probs(lt[j], T, 0, top_p) for j in range(G + 1)])
    q = np.stack([oracle.row_probs(ld[j], T, 0, top_p) for j in range(G)])
    assert (p == 0).any() and (q == 0).any()  # the cut removes tokens here
    law = _exact_outcome_law(p, q, "prob")
    beta = [np.minimum(p[j], q[j]).sum() for j in range(G)]
    for j in range(G + 1):
        marg = np.zeros(V)
        for (k, toks), pr in law.items():
            if k >= j:
                marg[toks[j]] += pr
        np.testing.assert_allclose(marg, np.prod(beta[:j]) * p[j], atol=1e-12)
    ltb = np.broadcast_to(lt[None], (n_runs,) + lt.shape).copy()
    ldb = np.broadcast_to(ld[None], (n_runs,) + ld.shape).copy()
    x = np.stack([rng.choice(V, size=n_runs, p=q[j]) for j in range(G)], axis=1).astype(np.int32)
    res = oracle.verify_batch(ltb, ldb, x, np.full(n_runs, T, np.float32), np.zeros(n_runs, np.int32),
                              np.full(n_runs, top_p, np.float32), seed=11)
    keys = list(law)
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for r in range(n_runs):
        k = int(res["num_accepted"][r])
        toks = tuple(int(t) for t in res["out_tokens"][r, :k + 1])
        assert (k, toks) in index, f"impossible outcome {(k, toks)}"
        counts[index[(k, toks)]] += 1
    expected = np.array([law[k] for k in keys]) * n_runs
    big = expected >= 5
    assert stats.chisquare(counts[big], expected[big] * counts[big].sum() / expected[big].sum()).pvalue > 1e-6


def _mixed_case(rng, n, G, V, dtype=np.float32):
    lt = (rng.standard_normal((n, G + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :G] + rng.standard_normal((n, G, V)).astype(np.float32)).astype(np.float32)
    x = rng.integers(0, V, size=(n, G)).astype(np.int32)
    # Make some drafts the target argmax so greedy requests accept some.
    am = np.argmax(lt[:, :G], axis=-1).astype(np.int32)
    sel = rng.random((n, G)) < 0.6
    x[sel] = am[sel]
    T = rng.choice(np.array([0.0, 0.5, 0.8, 1.0, 1.3], np.float32), size=n)
    K = rng.choice(np.array([0, 1, 5, 20, V + 3], np.int32), size=n)
    P = rng.choice(np.array([1.0, 0.3, 0.9, 0.95], np.float32), size=n)
    return lt, ld, x, T, K, P


@pytest.mark.parametrize("draft", ["prob", "onehot"])
def test_batch_reduces_to_single_setting_calls(draft):
    """Each request of a mixed batch gives exactly what a call with its own
    settings alone gives: the sampled path of verify() (top-p off) or, at
    temperature 0, the greedy rule."""
    rng = np.random.default_rng(31 if draft == "prob" else 32)
    n, G, V = 40, 4, 50
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    P[:] = 1.0
    res = oracle.verify_batch(lt, ld if draft == "prob" else None, x, T, K, P, seed=77)
    mode = oracle.MODE_PROB if draft == "prob" else oracle.MODE_ONEHOT
    for r in range(n):
        if T[r] == 0:
            one = oracle.verify(oracle.MODE_GREEDY, lt[r:r + 1], None, x[r:r + 1], seed=77, req_ids=[r])
        else:
            one = oracle.verify(mode, lt[r:r + 1], ld[r:r + 1] if draft == "prob" else None, x[r:r + 1],
                                temperature=float(T[r]), top_k=int(K[r]), seed=77, req_ids=[r])
            np.testing.assert_array_equal(res["p_draft"][r], one["p_draft"][0])
        np.testing.assert_array_equal(res["out_tokens"][r], one["out_tokens"][0])
        assert res["num_accepted"][r] == one["num_accepted"][0]


def test_batch_greedy_requests_follow_numpy_argmax():
    rng = np.random.default_rng(41)
    n, G, V = 30, 5, 64
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    T[:] = 0.0
    res = oracle.verify_batch(lt, ld, x, T, K, P, seed=5)
    a = np.argmax(lt, axis=-1)
    for r in range(n):
        mism = np.nonzero(x[r] != a[r, :G])[0]
        nn = int(mism[0]) if mism.size else G
        want = np.full(G + 1, -1)
        want[:nn] = x[r, :nn]
        want[nn] = a[r, nn]
        np.testing.assert_array_equal(res["out_tokens"][r], want)
        assert res["num_accepted"][r] == nn
        np.testing.assert_array_equal(res["p_draft"][r], (x[r] == a[r, :G]).astype(np.float64))
        np.testing.assert_array_equal(res["q_draft"][r], np.ones(G))


def test_batch_top_p_tiny_is_greedy_acceptance_and_bonus():
    """With top_p tiny every law is one-hot on its row's argmax: a draft that
    is the argmax of both rows is always accepted, any other always rejected,
    and the emitted token at n is the target argmax."""
    rng = np.random.default_rng(43)
    n, G, V = 30, 4, 40
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    ld = lt[:, :G].copy()
    T[:] = 0.9
    K[:] = 0
    P[:] = 1e-30
    res = oracle.verify_batch(lt, ld, x, T, K, P, seed=6)
    a = np.argmax(lt, axis=-1)
    for r in range(n):
        mism = np.nonzero(x[r] != a[r, :G])[0]
        nn = int(mism[0]) if mism.size else G
        assert res["num_accepted"][r] == nn
        assert res["out_tokens"][r, nn] == a[r, nn]


def test_batch_invalid_settings_emit_nothing():
    rng = np.random.default_rng(47)
    n, G, V = 6, 3, 30
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    T[:] = 0.8
    K[:] = 0
    P[:] = 1.0
    T[0] = -1.0
    T[1] = np.inf
    K[2] = -1
    K[3] = 25  # above max_top_k = 20 and below V
    P[4] = 0.0
    P[5] = 1.5
    res = oracle.verify_batch(lt, ld, x, T, K, P, max_top_k=20, seed=1)
    assert res["bad_param"].tolist() == [1] * 6
    assert (res["out_tokens"] == -1).all() and (res["num_accepted"] == 0).all()
    K[3] = 20
    T[:2] = 0.8
    K[2] = 0
    P[4:] = 1.0
    res = oracle.verify_batch(lt, ld, x, T, K, P, max_top_k=20, seed=1)
    assert res["bad_param"].tolist() == [0] * 6


# ---------------------------------------------------------------------------
# Draft given as probabilities; ragged draft lengths
# ---------------------------------------------------------------------------

def test_brute_force_draft_probabilities():
    """q given as probabilities (zeros included, not a softmax of anything):
    the exact outcome law, its losslessness identities, and the oracle's
    empirical law."""
    lt = _logits([[0.5, 0.0, 0.3, 0.2], [0.1, 0.6, 0.3, 0.0], [0.25, 0.25, 0.25, 0.25]])
    q = np.array([[0.0, 0.5, 0.25, 0.25], [0.5, 0.25, 0.0, 0.25]], dtype=np.float32)
    G, V, n_runs = 2, 4, 100_000
    p = np.stack([oracle.row_probs(lt[j], 1.0) for j in range(G + 1)])
    law = _exact_outcome_law(p, q.astype(np.float64), "prob")
    beta = [np.minimum(p[j], q[j]).sum() for j in range(G)]
    for j in range(G + 1):
        marg = np.zeros(V)
        for (k, toks), pr in law.items():
            if k >= j:
                marg[toks[j]] += pr
        np.testing.assert_allclose(marg, np.prod(beta[:j]) * p[j], atol=1e-12)
    rng = np.random.default_rng(29)
    x = np.stack([rng.choice(V, size=n_runs, p=q[j].astype(np.float64)) for j in range(G)], axis=1).astype(np.int32)
    res = oracle.verify_batch(np.broadcast_to(lt[None], (n_runs,) + lt.shape).copy(), None, x,
                              np.ones(n_runs, np.float32), np.zeros(n_runs, np.int32), np.ones(n_runs, np.float32),
                              draft_probs=np.broadcast_to(q[None], (n_runs, G, V)).copy(), seed=13)
    np.testing.assert_array_equal(res["q_draft"], q[np.arange(G)[None, :], x])
    keys = list(law)
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for r in range(n_runs):
        k = int(res["num_accepted"][r])
        counts[index[(k, tuple(int(t) for t in res["out_tokens"][r, :k + 1]))]] += 1
    expected = np.array([law[k] for k in keys]) * n_runs
    big = expected >= 5
    assert stats.chisquare(counts[big], expected[big] * counts[big].sum() / expected[big].sum()).pvalue > 1e-6


def test_one_hot_probabilities_equal_onehot_drafts():
    """q = 1 at the draft token, 0 elsewhere, given as probabilities, is the
    one-hot rule exactly: accept iff u <= p(x), residual p with x masked."""
    rng = np.random.default_rng(37)
    n, G, V = 40, 4, 30
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    T[T == 0] = 0.9
    q = np.zeros((n, G, V), np.float32)
    q[np.arange(n)[:, None], np.arange(G)[None, :], x] = 1.0
    a = oracle.verify_batch(lt, None, x, T, K, P, draft_probs=q, seed=3)
    b = oracle.verify_batch(lt, None, x, T, K, P, seed=3)
    for key in ("out_tokens", "num_accepted", "p_draft", "q_draft"):
        np.testing.assert_array_equal(a[key], b[key])


def test_ragged_lengths_reduce_to_single_requests():
    """A request with g of gamma draft positions gives exactly what a call
    with gamma = g gives (its own uniforms); padding after it is -1."""
    rng = np.random.default_rng(53)
    n, G, V = 24, 5, 40
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    g = rng.integers(0, G + 1, size=n).astype(np.int32)
    g[:3] = [0, G, 1]
    for draft in ("logits", "onehot"):
        res = oracle.verify_batch(lt, ld if draft == "logits" else None, x, T, K, P, lengths=g, seed=21)
        for r in range(n):
            one = oracle.verify_batch(lt[r:r + 1, :g[r] + 1], ld[r:r + 1, :g[r]] if draft == "logits" else None,
                                      x[r:r + 1, :g[r]], T[r:r + 1], K[r:r + 1], P[r:r + 1], seed=21, req_ids=[r])
            assert res["num_accepted"][r] == one["num_accepted"][0]
            np.testing.assert_array_equal(res["out_tokens"][r, :g[r] + 1], one["out_tokens"][0])
            assert (res["out_tokens"][r, g[r] + 1:] == -1).all()
            np.testing.assert_array_equal(res["p_draft"][r, :g[r]], one["p_draft"][0])
            assert np.isnan(res["p_draft"][r, g[r]:]).all()


def test_zero_draft_positions_emit_a_draw_from_p0():
    """g = 0: nothing to verify, the one emitted token is the bonus draw from
    p_0 (chi-square over many requests of one row)."""
    lt = _logits([[0.5, 0.3, 0.15, 0.05], [0.25, 0.25, 0.25, 0.25]])
    n = 50_000
    res = oracle.verify_batch(np.broadcast_to(lt[None], (n, 2, 4)).copy(), None, np.zeros((n, 1), np.int32),
                              np.ones(n, np.float32), np.zeros(n, np.int32), np.ones(n, np.float32),
                              lengths=np.zeros(n, np.int32), seed=8)
    assert (res["num_accepted"] == 0).all() and (res["out_tokens"][:, 1] == -1).all()
    counts = np.bincount(res["out_tokens"][:, 0], minlength=4)
    assert stats.chisquare(counts, np.array([0.5, 0.3, 0.15, 0.05]) * n).pvalue > 1e-6


# ---------------------------------------------------------------------------
# Per-position acceptance probability beta through the batch path
# ---------------------------------------------------------------------------

def test_beta_worked_example_with_draft_probabilities():
    """The 5-token example with q handed over as probabilities: beta =
    sum min(p, q) = 0.75 as printed; with one-hot drafts beta = p(x)."""
    p, q, g = _worked()
    lt = _f32_logits(p)[None, None, :].repeat(2, axis=1)
    one = np.ones(1, np.float32)
    res = oracle.verify_batch(lt, None, np.zeros((1, 1), np.int32), one, np.zeros(1, np.int32), one,
                              draft_probs=np.asarray(q, np.float32)[None, None, :], diagnostics=True)
    assert abs(res["beta"][0, 0] - float(g["sum_min_pq"][0])) < 1e-6
    res = oracle.verify_batch(lt, None, np.array([[int(np.argmax(q))]], np.int32), one, np.zeros(1, np.int32), one,
                              diagnostics=True)
    assert abs(res["beta"][0, 0] - float(g["p_at_argmax_q"][0])) < 1e-6


def test_beta_closed_forms():
    rng = np.random.default_rng(61)
    n, G, V = 12, 3, 50
    lt = (rng.standard_normal((n, G + 1, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, (n, G)).astype(np.int32)
    T = np.full(n, 0.8, np.float32)
    K = np.zeros(n, np.int32)
    P = np.ones(n, np.float32)
    p = np.stack([np.stack([oracle.row_probs(lt[r, j], 0.8) for j in range(G)]) for r in range(n)])
    # q = p (up to fp32 rounding): beta = 1.
    res = oracle.verify_batch(lt, None, x, T, K, P, draft_probs=p.astype(np.float32), diagnostics=True)
    np.testing.assert_allclose(res["beta"], 1.0, atol=1e-6)
    # q only where a top-5 target has no mass: beta = 0.
    K5 = np.full(n, 5, np.int32)
    p5 = np.stack([np.stack([oracle.row_probs(lt[r, j], 0.8, 5) for j in range(G)]) for r in range(n)])
    q0 = (p5 == 0).astype(np.float32)
    q0 /= q0.sum(-1, keepdims=True)
    res = oracle.verify_batch(lt, None, x, T, K5, P, draft_probs=q0, diagnostics=True, max_top_k=5)
    np.testing.assert_array_equal(res["beta"], 0.0)
    # Temperature 0: beta is the argmax indicator.
    res = oracle.verify_batch(lt, None, x, np.zeros(n, np.float32), K, P, diagnostics=True)
    np.testing.assert_array_equal(res["beta"], (x == np.argmax(lt[:, :G], axis=-1)).astype(np.float64))


def test_decay_sigmas_give_the_pages_rates():
    """The draft-noise levels of the decaying-acceptance workload give mean
    beta = sum min(p, q) of 0.951, 0.889, 0.852 at positions 0, 1, 2 (the
    Gemma run's per-position rates on the draft-model page), on rows other
    than the ones they were solved on."""
    import workloads
    wl = workloads.ROUNDS_WORKLOADS["rounds_decay_bf16_b512_g3_v128256"].scaled(B=32, data_seed=11)
    inp = workloads.generate(wl)
    h = workloads.to_host_arrays
    res = oracle.verify(oracle.MODE_PROB, h(inp["target_logits"]), h(inp["draft_logits"]), h(inp["draft_tokens"]),
                        temperature=wl.temperature, seed=1, diagnostics=True)
    np.testing.assert_allclose(res["beta"].mean(axis=0), workloads.DECAY_ALPHAS, atol=0.01)


# ---------------------------------------------------------------------------
# Sampler-match acceptance over chains and trees
# ---------------------------------------------------------------------------

def _match_runs(lt, x, parents, n_runs, seed, T=1.0):
    G = x.shape[-1]
    ltb = np.broadcast_to(lt[None], (n_runs,) + lt.shape).copy()
    xb = np.broadcast_to(x[None], (n_runs, G)).copy()
    pb = None if parents is None else np.broadcast_to(np.asarray(parents, np.int32)[None], (n_runs, G)).copy()
    one = np.full(n_runs, T, np.float32)
    return oracle.verify_batch(ltb, None, xb, one, np.zeros(n_runs, np.int32), np.ones(n_runs, np.float32),
                               seed=seed, match=True, parents=pb, diagnostics=True)


def test_sampler_match_chain_law():
    """Chain x_0, x_1: the walk accepts x_j iff the fresh sample equals it;
    P(n = d, out) = prod_{j<d} p_j(x_j) * p_d(out_d) with out_d != x_d for
    d < G.  Checked exactly and against the oracle's empirical law."""
    lt = _logits([[0.5, 0.25, 0.15, 0.1], [0.3, 0.3, 0.2, 0.2], [0.1, 0.2, 0.3, 0.4]])
    x = np.array([0, 2], np.int32)
    p = np.stack([oracle.row_probs(lt[j], 1.0) for j in range(3)])
    law = {}
    for d in range(3):
        pre = np.prod([p[j][x[j]] for j in range(d)])
        for y in range(4):
            if d < 2 and y == x[d]:
                continue
            law[(d, tuple(x[:d]) + (y,))] = pre * p[d][y]
    assert abs(sum(law.values()) - 1.0) < 1e-12
    n_runs = 60_000
    res = _match_runs(lt, x, None, n_runs, 3)
    np.testing.assert_allclose(res["p_draft"][0], [p[0][0], p[1][2]], rtol=1e-12)
    keys = list(law)
    idx = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for r in range(n_runs):
        d = int(res["num_accepted"][r])
        counts[idx[(d, tuple(int(t) for t in res["out_tokens"][r, :d + 1]))]] += 1
        assert list(res["path_nodes"][r, :d]) == list(range(1, d + 1))
    expected = np.array([law[k] for k in keys]) * n_runs
    assert stats.chisquare(counts, expected).pvalue > 1e-6


def test_sampler_match_tree_branches():
    """Root with children a = 1 (node 1) and b = 2 (node 2), node 3 a child of
    node 1 with token 0: the walk follows a with probability p_0(a), b with
    p_0(b), stops at the root otherwise; the root's emitted token is ~p_0."""
    lt = _logits([[0.4, 0.3, 0.2, 0.1], [0.6, 0.1, 0.1, 0.2], [0.25, 0.25, 0.25, 0.25], [0.1, 0.1, 0.1, 0.7]])
    x = np.array([1, 2, 0], np.int32)
    parents = np.array([0, 0, 1], np.int32)
    n_runs = 60_000
    res = _match_runs(lt, x, parents, n_runs, 9)
    p0, p1 = oracle.row_probs(lt[0], 1.0), oracle.row_probs(lt[1], 1.0)
    np.testing.assert_allclose(res["p_draft"][0], [p0[1], p0[2], p1[0]], rtol=1e-12)
    first = res["out_tokens"][:, 0]
    assert stats.chisquare(np.bincount(first, minlength=4), p0 * n_runs).pvalue > 1e-6
    path1 = res["path_nodes"][:, 0]
    via = np.array([(path1 == -1).sum(), (path1 == 1).sum(), (path1 == 2).sum()])
    assert stats.chisquare(via, np.array([1 - p0[1] - p0[2], p0[1], p0[2]]) * n_runs).pvalue > 1e-6
    # Through node 1, node 3 (token 0) is accepted with probability p_1(0).
    thru = path1 == 1
    deep = (res["path_nodes"][thru, 1] == 3).mean()
    assert abs(deep - p1[0]) < 4 * np.sqrt(p1[0] * (1 - p1[0]) / thru.sum())


def test_sampler_match_reductions():
    rng = np.random.default_rng(71)
    n, G, V = 30, 4, 40
    lt, ld, x, T, K, P = _mixed_case(rng, n, G, V)
    chain = np.tile(np.arange(G, dtype=np.int32), (n, 1))  # node j + 1's parent is node j
    a = oracle.verify_batch(lt, None, x, T, K, P, seed=4, match=True)
    b = oracle.verify_batch(lt, None, x, T, K, P, seed=4, match=True, parents=chain)
    for key in ("out_tokens", "num_accepted", "p_draft", "path_nodes"):
        np.testing.assert_array_equal(a[key], b[key])
    # Temperature 0: the sampler is the argmax, and a chain is the greedy rule.
    T0 = np.zeros(n, np.float32)
    m = oracle.verify_batch(lt, None, x, T0, K, P, seed=4, match=True)
    gr = oracle.verify_batch(lt, None, x, T0, K, P, seed=4)
    np.testing.assert_array_equal(m["out_tokens"], gr["out_tokens"])
    np.testing.assert_array_equal(m["num_accepted"], gr["num_accepted"])
    np.testing.assert_array_equal(m["p_draft"], gr["p_draft"])
    # Two children with the same token: the lower-indexed one is followed.
    lt2 = _logits([[0.0, 1.0, 0.0, 0.0], [0.25] * 4, [0.25] * 4])
    r = _match_runs(lt2, np.array([1, 1], np.int32), np.array([0, 0], np.int32), 20, 5)
    assert (r["path_nodes"][:, 0] == 1).all()
    # A parent that is not an earlier node makes the request invalid.
    bad = chain.copy()
    bad[2, 1] = 2
    c = oracle.verify_batch(lt, None, x, T, K, P, seed=4, match=True, parents=bad)
    assert c["bad_param"][2] == 1 and (c["out_tokens"][2] == -1).all() and c["bad_param"].sum() == 1


def test_sampler_match_sample_is_the_race_on_the_node_law():
    """The fresh sample of a node is the one Exp(1) race over its adjusted
    law on the race stream of (request, node), for every size of law (a
    top-k of 64, 1024 or 1025 tokens, the whole vocabulary): the emitted
    token of a walk that ends at the root equals that race."""
    rng = np.random.default_rng(13)
    V = 3000
    for trial in range(6):
        lt = rng.normal(0.0, 2.0, size=(1, 2, V)).astype(np.float32)
        x = np.array([[-1]], np.int32)  # no child can match: the root's sample is emitted
        for k in (64, 1024, 1025, 0):
            p = oracle.row_probs(lt[0, 0], 1.0, k)
            res = oracle.verify_batch(lt, None, x, np.ones(1, np.float32), np.full(1, k, np.int32),
                                      np.ones(1, np.float32), max_top_k=max(k, 1), seed=17 + trial, match=True)
            assert int(res["out_tokens"][0, 0]) == oracle.race(p, 17 + trial, 0, 0)[0]


def test_sampler_match_full_law_frequencies():
    """Sampler-match over the whole vocabulary: a root with no matching child
    emits its sample, whose law over 40k requests is the row's p (chi-square;
    the full-vocabulary path draws every token's own variate)."""
    V = 40
    rng = np.random.default_rng(2)
    row = rng.normal(0.0, 1.5, V).astype(np.float32)
    n = 40_000
    lt = np.broadcast_to(row, (n, 2, V)).copy()
    x = np.full((n, 1), -1, np.int32)
    res = oracle.verify_batch(lt, None, x, np.ones(n, np.float32), np.zeros(n, np.int32), np.ones(n, np.float32),
                              seed=3, match=True)
    p = oracle.row_probs(row, 1.0)
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert (p * n >= 5).all()
    assert stats.chisquare(counts, p * n).pvalue > 1e-6


# ---------------------------------------------------------------------------
# Decision margins: they decide which results a comparison may exempt
# ---------------------------------------------------------------------------

def test_nucleus_margin_hand_computed():
    """Top-p on (0.5, 0.3, 0.15, 0.05): the stop at rank s has the sides
    C_s - top_p and top_p - C_(s-1); at s = 1 only the first exists."""
    logits = np.log(np.array([0.5, 0.3, 0.15, 0.05])).astype(np.float32)
    # (top_p, kept tokens, margin)
    for top_p, kept, margin in ((1e-30, 1, 0.5), (0.45, 1, 0.05), (0.5, 1, 0.0), (0.6, 2, 0.1), (0.79, 2, 0.01),
                                (0.81, 3, 0.01), (0.9, 3, 0.05), (0.97, 4, 0.02)):
        p, m = oracle.row_probs(logits, 1.0, 0, top_p, return_margin=True)
        assert int((p > 0).sum()) == kept, top_p
        assert m == pytest.approx(margin, abs=1e-7), (top_p, m)
    # The function itself, on exact values.
    assert oracle.nucleus_margin(1, 0.5, 0.0, 1e-30) == 0.5 - 1e-30
    assert oracle.nucleus_margin(1, 0.5, 0.0, 0.45) == 0.5 - 0.45
    assert oracle.nucleus_margin(2, 0.75, 0.5, 0.625) == 0.125
    assert oracle.nucleus_margin(2, 0.75, 0.5, 0.5625) == 0.0625
    assert oracle.nucleus_margin(3, 1.0, 0.75, 0.75) == 0.0
    # Top-p off: margin 1.
    assert oracle.row_probs(logits, 1.0, 0, 1.0, return_margin=True)[1] == 1.0


def test_accept_margin_hand_computed():
    """|u q(x) - p(x)| / max(u q(x), p(x)); no boundary (margin 1) for an
    invalid token or q(x) = 0."""
    assert oracle.accept_margin(0.5, 0.25, 0.5) == 0.0          # u q = p exactly
    assert oracle.accept_margin(0.5, 0.3, 0.5) == pytest.approx(0.05 / 0.3)
    assert oracle.accept_margin(0.8, 0.2, 0.5) == pytest.approx(0.2 / 0.4)
    assert oracle.accept_margin(0.25, 0.5, 1.0) == 0.5           # one-hot q: |u - p| / max(u, p)
    assert oracle.accept_margin(0.7, 0.0, 0.5) == 1.0            # p = 0: rejected by any u
    assert oracle.accept_margin(0.7, 0.4, 0.0) == 1.0            # q = 0: rejected
    assert oracle.accept_margin(0.7, 0.4, 0.5, valid=False) == 1.0
    # The denominator is the larger side (a slip to min() would give 1/3 here).
    assert oracle.accept_margin(1.0, 0.75, 1.0) == pytest.approx(0.25)


def test_race_margin_hand_computed():
    """(s1 - s2) / s1 over the two best scores; one candidate: 1; an infinite
    winner is flipped only by another."""
    assert oracle.race_margin(2, 2.0, 2.0) == 0.0
    assert oracle.race_margin(3, 2.0, 1.0) == 0.5                # a slip to / s2 would give 1
    assert oracle.race_margin(1, 2.0, float("-inf")) == 1.0
    assert oracle.race_margin(2, float("inf"), 3.0) == 1.0
    assert oracle.race_margin(2, float("inf"), float("inf")) == 0.0


def _race_e(seed, b, j, y):
    return -math.log(oracle.uniform_race(seed, b, j, y))


def test_race_margin_in_the_race():
    """Weights set to the race's own exponentials make every score exactly 1:
    the margin is 0 and the lowest index wins; a relative gap of 5e-5 planted
    on one weight is flagged (<= 1e-4), one of 2e-4 is not; a single
    candidate has margin 1."""
    seed, b, j = 11, 3, 2
    e = np.array([_race_e(seed, b, j, y) for y in range(6)])
    tok, m = oracle.race(e, seed, b, j)
    assert tok == 0 and m == 0.0
    w = e.copy()
    w[4] *= 1 + 5e-5
    tok, m = oracle.race(w, seed, b, j)
    assert tok == 4 and 0 < m <= 1e-4 and m == pytest.approx(5e-5 / (1 + 5e-5), rel=1e-6)
    w = e.copy()
    w[4] *= 1 + 2e-4
    tok, m = oracle.race(w, seed, b, j)
    assert tok == 4 and m > 1e-4
    w = np.zeros(6)
    w[3] = 0.2
    assert oracle.race(w, seed, b, j) == (3, 1.0)


def _onehot_row_for(p_target):
    """Two logits whose softmax gives token 0 the probability p_target."""
    d = math.log(p_target / (1 - p_target))
    return np.array([d, 0.0])


def test_near_tie_planted_in_a_verifier_call():
    """One-hot drafts on V = 2 with p(x_j) planted next to the accept
    uniform u_j: at position 1, p(x) = u (1 - 2e-5) is a near tie (flagged,
    position 1, one row); p(x) = u (1 - 1e-3) is not.  Position 0 accepts
    surely (p(x) = 1 - 1e-12) and takes no near tie."""
    seed, G = 5, 3
    for b in range(4):
        u1 = oracle.uniform_accept(seed, b, 1)
        for gap, flagged in ((2e-5, True), (1e-3, False)):
            lt = np.zeros((1, G + 1, 2))
            lt[0, 0] = _onehot_row_for(1 - 1e-12)
            lt[0, 1] = _onehot_row_for(u1 * (1 - gap))
            lt[0, 2] = _onehot_row_for(0.5)
            lt[0, 3] = _onehot_row_for(0.5)
            x = np.zeros((1, G), np.int32)
            res = oracle.verify(oracle.MODE_ONEHOT, lt.astype(np.float64).astype(np.float32), None, x,
                                temperature=1.0, seed=seed, req_ids=np.array([b], np.int32), diagnostics=True)
            # fp32 rounding of the logits moves p(x) by ~1e-7 relative: the gap stays on its side.
            assert res["num_accepted"][0] == 1
            am = res["accept_margin"][0]
            assert (am[1] <= 1e-4) == flagged, am
            pos = oracle.near_tie_position(res)
            assert pos[0] == (1 if flagged else -1)
            assert near_tie_rows(res) == (1 if flagged else 0)


def test_near_tie_position_and_rows_hand_built():
    """On hand-built diagnostics: only decisions actually taken count (accept
    tests j <= n, the race at n); margins past n are ignored; NaN margins
    (greedy requests, unused positions) never flag; under sampler-match a
    flagged race leaves no position fixed (0)."""
    nan = float("nan")
    res = {"num_accepted": np.array([1, 1, 3, 2, 0]),
           "accept_margin": np.array([[0.5, 1e-5, 0.3],    # rejected at 1 with a near tie: position 1
                                      [0.5, 0.5, 1e-6],    # margin past n = 1: ignored
                                      [0.5, 0.5, 0.5],     # all accepted, race near tie at n = G = 3
                                      [nan, nan, nan],     # greedy: never flagged
                                      [0.2, 0.5, 0.5]]),
           "race_margin": np.array([0.5, 0.5, 5e-5, nan, 1e-4])}
    pos = oracle.near_tie_position(res)
    np.testing.assert_array_equal(pos, [1, -1, 3, -1, 0])
    # Rows: request 0 row 1; request 2 row 3 (its race); request 4 row 0
    # (race at n = 0, margin exactly 1e-4 counts).
    assert near_tie_rows(res) == 3
    # Accept near tie and race near tie on the same row count once.
    res2 = {"num_accepted": np.array([1]), "accept_margin": np.array([[0.5, 1e-6]]),
            "race_margin": np.array([1e-6])}
    assert near_tie_rows(res2) == 1
    assert oracle.near_tie_position(res2)[0] == 1
    res3 = dict(res2, match=True)
    assert oracle.near_tie_position(dict(res3, accept_margin=np.ones((1, 2))))[0] == 0


def test_near_cut_requests_compared_not_skipped():
    """A top-p of 1e-30 keeps one token on every row with a margin of about
    the top token's mass (not 1e-30): no request is near-cut, so every
    request of such a batch is compared."""
    rng = np.random.default_rng(4)
    n, G, V = 6, 3, 50
    lt = rng.normal(0, 2, size=(n, G + 1, V)).astype(np.float32)
    x = rng.integers(0, V, size=(n, G)).astype(np.int32)
    res = oracle.verify_batch(lt, None, x, np.ones(n, np.float32), np.zeros(n, np.int32),
                              np.full(n, 1e-30, np.float32), seed=1, diagnostics=True)
    assert (res["cut_margin"] > 1e-3).all()
    rep = compare_batch(res, res)
    assert rep["near_cut_requests"] == 0 and rep["mismatch_non_tie"] == 0
