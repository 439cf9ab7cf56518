"""Plain fp64 CPU oracle of the speculative-sampling verifier (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or calls
anything in this directory; only the test suite, the smoke check and the
benchmark's CPU-baseline leg may.  The arithmetic lives in
``spec_oracle.cpp``; this module only compiles it (with g++) and marshals
numpy arrays.

Pinned functions and their pins (see tests/test_oracle_pins.py):
  philox4x32_10, uniform_accept, uniform_race -- Random123 known-answer
      values and runs of ATen's independent Philox engine;
  row_probs -- closed forms (temperature, top-k ties, -inf logits; top-p
      nucleus sets on hand-computed laws, index ties on flat rows, the
      temperature-before-top-p and top-k-before-top-p orders);
  race -- chi-square against w / sum(w);
  accept_margin, race_margin, nucleus_margin, near_tie_position and
      oracle.parity.near_tie_rows -- hand-computed values (equal scores give
      0, one candidate 1, a planted relative gap of 5e-5 is flagged, a top-p
      stop at the first token has only the C_1 - top_p side), and planted
      near-ties in whole verifier calls;
  verify (prob / onehot / greedy / naive) -- the worked 5-token example and
      Monte Carlo table of the vLLM rejection-resampling page, Eq. 1 of the
      draft-model page, brute-force enumeration at V <= 4, and exact
      reductions between the three modes;
  verify_batch -- per-request settings reduce exactly to single-setting
      calls; temperature-0 requests follow numpy's argmax.
  The zero-mass fallback (equal laws at a forced rejection) is pinned by its
  law: the token drawn there follows p.
Parity unpinned by the pages (pinned only by this oracle's own definition):
  the tie rules, the Philox keying and bit mapping.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libspec_oracle.so")

MODE_PROB, MODE_ONEHOT, MODE_GREEDY, MODE_NAIVE = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle into oracle/libspec_oracle.so (g++, fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = build()
    lib = ctypes.CDLL(path)
    c_u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.sv_ref_philox4x32_10.argtypes = [c_u32p, c_u32p, c_u32p]
    lib.sv_ref_philox4x32_10.restype = None
    lib.sv_ref_uniform_accept.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
    lib.sv_ref_uniform_accept.restype = ctypes.c_double
    lib.sv_ref_uniform_race.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.sv_ref_uniform_race.restype = ctypes.c_double
    lib.sv_ref_row_probs.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_int, ctypes.c_void_p]
    lib.sv_ref_row_probs.restype = ctypes.c_int
    lib.sv_ref_row_probs_p.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                       ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_double)]
    lib.sv_ref_row_probs_p.restype = ctypes.c_int
    lib.sv_ref_verify_ex.argtypes = ([ctypes.c_int] * 5 + [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_uint64]
                                     + [ctypes.c_void_p] * 18 + [ctypes.c_int])
    lib.sv_ref_verify_ex.restype = ctypes.c_int
    lib.sv_ref_row_argmax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    lib.sv_ref_row_argmax.restype = ctypes.c_int
    lib.sv_ref_race.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                ctypes.c_uint32, ctypes.POINTER(ctypes.c_double)]
    lib.sv_ref_race.restype = ctypes.c_int
    lib.sv_ref_accept_margin.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int]
    lib.sv_ref_accept_margin.restype = ctypes.c_double
    lib.sv_ref_race_margin.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    lib.sv_ref_race_margin.restype = ctypes.c_double
    lib.sv_ref_nucleus_margin.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.sv_ref_nucleus_margin.restype = ctypes.c_double
    lib.sv_ref_verify.argtypes = ([ctypes.c_int] * 5 + [ctypes.c_double, ctypes.c_int, ctypes.c_uint64]
                                  + [ctypes.c_void_p] * 13 + [ctypes.c_int])
    lib.sv_ref_verify.restype = ctypes.c_int
    lib.sv_ref_max_threads.argtypes = []
    lib.sv_ref_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits_bytes(a) -> tuple[np.ndarray, int]:
    """Accept float32 arrays or bfloat16 bit patterns held as uint16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, DTYPE_F32
    if a.dtype == np.uint16:
        return a, DTYPE_BF16
    raise TypeError(f"logits must be float32 or uint16 (bfloat16 bits), got {a.dtype}")


def philox4x32_10(ctr, key) -> np.ndarray:
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.sv_ref_philox4x32_10(c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                             k.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
    return out


def uniform_accept(seed: int, b: int, j: int) -> float:
    return _load().sv_ref_uniform_accept(seed, b, j)


def uniform_race(seed: int, b: int, j: int, y: int) -> float:
    return _load().sv_ref_uniform_race(seed, b, j, y)


def row_probs(row, temperature: float, top_k: int = 0, top_p: float = 1.0, return_margin: bool = False):
    """Adjusted law of one row: temperature, top-k, top-p (>= 1: off)."""
    r, dt = _logits_bytes(row)
    V = r.shape[-1]
    out = np.zeros(V, dtype=np.float64)
    m = ctypes.c_double(1.0)
    if top_p >= 1.0:
        _load().sv_ref_row_probs(_ptr(r), dt, V, float(temperature), int(top_k), _ptr(out))
    else:
        _load().sv_ref_row_probs_p(_ptr(r), dt, V, float(temperature), int(top_k), float(top_p), _ptr(out),
                                   ctypes.byref(m))
    return (out, m.value) if return_margin else out


def row_argmax(row) -> int:
    r, dt = _logits_bytes(row)
    return _load().sv_ref_row_argmax(_ptr(r), dt, r.shape[-1])


def race(w, seed: int, b: int, j: int) -> tuple[int, float]:
    wv = np.ascontiguousarray(w, dtype=np.float64)
    m = ctypes.c_double(0.0)
    tok = _load().sv_ref_race(_ptr(wv), wv.shape[0], seed, b, j, ctypes.byref(m))
    return tok, m.value


def accept_margin(u: float, px: float, qx: float, valid: bool = True) -> float:
    """Relative distance of the accept test u q(x) <= p(x) from its boundary."""
    return _load().sv_ref_accept_margin(float(u), float(px), float(qx), int(bool(valid)))


def race_margin(ncand: int, s1: float, s2: float) -> float:
    """Relative gap of a race winner's score s1 over the runner-up's s2."""
    return _load().sv_ref_race_margin(int(ncand), float(s1), float(s2))


def nucleus_margin(s: int, C: float, Cprev: float, top_p: float) -> float:
    """Distance of top_p from the nucleus decision that stops at rank s with
    running masses C (through rank s) and Cprev (through rank s - 1)."""
    return _load().sv_ref_nucleus_margin(int(s), float(C), float(Cprev), float(top_p))


def max_threads() -> int:
    return _load().sv_ref_max_threads()


def verify(mode: int, target_logits, draft_logits, draft_tokens, *, temperature: float = 1.0,
           top_k: int = 0, seed: int = 0, req_ids=None, diagnostics: bool = False,
           nthreads: int = 0) -> dict:
    """Run the oracle on host arrays.

    target_logits: [n, G+1, V] float32 or uint16 (bfloat16 bits)
    draft_logits:  [n, G, V] same dtype (prob / naive modes), else None
    draft_tokens:  [n, G] int32
    req_ids:       [n] request indices for the Philox streams (default 0..n-1)
    """
    lib = _load()
    lt, dt = _logits_bytes(target_logits)
    n, G1, V = lt.shape
    G = G1 - 1
    ld = None
    if draft_logits is not None:
        ld, dt2 = _logits_bytes(draft_logits)
        if dt2 != dt or ld.shape != (n, G, V):
            raise ValueError("draft logits must match target dtype and be [n, G, V]")
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if x.shape != (n, G):
        raise ValueError("draft tokens must be [n, G]")
    rid = None if req_ids is None else np.ascontiguousarray(req_ids, dtype=np.int32)
    out = np.empty((n, G + 1), dtype=np.int32)
    nacc = np.empty(n, dtype=np.int32)
    res = {"out_tokens": out, "num_accepted": nacc}
    bad = np.zeros(n, dtype=np.int32)
    res["bad_token"] = bad
    pd = qd = targ = beta = am = rm = None
    if mode == MODE_GREEDY:
        targ = np.empty((n, G + 1), dtype=np.int32)
        res["target_argmax"] = targ
    else:
        pd = np.empty((n, G), dtype=np.float64)
        qd = np.empty((n, G), dtype=np.float64)
        res["p_draft"], res["q_draft"] = pd, qd
        if diagnostics:
            beta = np.empty((n, G), dtype=np.float64)
            am = np.empty((n, G), dtype=np.float64)
            rm = np.empty(n, dtype=np.float64)
            res["beta"], res["accept_margin"], res["race_margin"] = beta, am, rm
    rc = lib.sv_ref_verify(mode, n, G, V, dt, float(temperature), int(top_k), int(seed),
                           _ptr(lt), _ptr(ld), _ptr(x), _ptr(rid), _ptr(out), _ptr(nacc), _ptr(pd), _ptr(qd),
                           _ptr(targ), _ptr(beta), _ptr(am), _ptr(rm), _ptr(bad), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return res


def verify_batch(target_logits, draft_logits, draft_tokens, temperature, top_k, top_p, *, max_top_k: int = 1024,
                 seed: int = 0, req_ids=None, diagnostics: bool = False, nthreads: int = 0, draft_probs=None,
                 lengths=None, match: bool = False, parents=None) -> dict:
    """Run the oracle with per-request settings.

    Arrays are padded: target_logits [n, G+1, V], draft_logits [n, G, V]
    (None: one-hot drafts), draft_probs [n, G, V] float32 (the drafter's
    probabilities, used as given; replaces draft_logits), draft_tokens
    [n, G]; lengths [n] (draft positions per request, 0..G; None: all G)
    selects the rows and positions that exist.  temperature [n] float32 (0 =
    greedy request), top_k [n] int32, top_p [n] float32, taken at the
    caller's fp32 / int32 precision.  Per-position outputs are [n, G], NaN
    after a request's length.

    match: token-only drafts verified by sampler-match; draft position j is
    node j + 1 of a tree whose root (node 0) has target row 0; parents [n, G]
    gives each draft node's parent node (0..j), None for chains.  Returns
    path_nodes [n, G+1] (accepted nodes in order, -1 after).
    """
    lib = _load()
    lt, dt = _logits_bytes(target_logits)
    n, G1, V = lt.shape
    G = G1 - 1
    kind = 1
    ld = qp = None
    if match:
        kind = 3
    elif draft_probs is not None:
        kind = 2
        qp = np.ascontiguousarray(draft_probs, dtype=np.float32)
        if qp.shape != (n, G, V):
            raise ValueError("draft probabilities must be [n, G, V]")
    elif draft_logits is not None:
        kind = 0
        ld, dt2 = _logits_bytes(draft_logits)
        if dt2 != dt or ld.shape != (n, G, V):
            raise ValueError("draft logits must match target dtype and be [n, G, V]")
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if x.shape != (n, G):
        raise ValueError("draft tokens must be [n, G]")
    g = np.full(n, G, dtype=np.int32) if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    if g.shape != (n,) or (g < 0).any() or (g > G).any():
        raise ValueError("lengths must be [n] in 0..G")
    # Pack: request r keeps target rows 0..g_r and draft rows / tokens 0..g_r-1.
    lt_p = np.ascontiguousarray(np.concatenate([lt[r, :g[r] + 1] for r in range(n)])) if n else lt.reshape(0, V)
    ld_p = (np.ascontiguousarray(np.concatenate([ld[r, :g[r]] for r in range(n)])) if ld is not None else None)
    qp_p = (np.ascontiguousarray(np.concatenate([qp[r, :g[r]] for r in range(n)])) if qp is not None else None)
    x_p = np.ascontiguousarray(np.concatenate([x[r, :g[r]] for r in range(n)])) if n else x.reshape(0)
    par_p = None
    if parents is not None:
        par = np.ascontiguousarray(parents, dtype=np.int32)
        par_p = np.ascontiguousarray(np.concatenate([par[r, :g[r]] for r in range(n)])) if n else par.reshape(0)
    path = np.full((n, G + 1), -1, dtype=np.int32)
    tot = int(g.sum())
    t = np.ascontiguousarray(temperature, dtype=np.float32).reshape(n)
    k = np.ascontiguousarray(top_k, dtype=np.int32).reshape(n)
    p = np.ascontiguousarray(top_p, dtype=np.float32).reshape(n)
    rid = None if req_ids is None else np.ascontiguousarray(req_ids, dtype=np.int32)
    out = np.empty((n, G + 1), dtype=np.int32)
    nacc = np.empty(n, dtype=np.int32)
    pd, qd = np.empty(tot, np.float64), np.empty(tot, np.float64)
    bad, badp, cm = np.zeros(n, np.int32), np.zeros(n, np.int32), np.empty(n, np.float64)
    beta = am = rm = None
    if diagnostics:
        beta, am, rm = np.empty(tot, np.float64), np.empty(tot, np.float64), np.empty(n, np.float64)
    rc = lib.sv_ref_verify_ex(kind, n, G, V, dt, _ptr(t), _ptr(k), _ptr(p), int(max_top_k), int(seed), _ptr(lt_p),
                              _ptr(ld_p), _ptr(qp_p), _ptr(x_p), _ptr(g), _ptr(rid), _ptr(out), _ptr(nacc), _ptr(pd),
                              _ptr(qd), _ptr(beta), _ptr(am), _ptr(rm), _ptr(cm), _ptr(bad), _ptr(badp),
                              _ptr(par_p), _ptr(path), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")

    def pad(v):
        o = np.full((n, G), np.nan)
        off = 0
        for r in range(n):
            o[r, :g[r]] = v[off:off + g[r]]
            off += g[r]
        return o

    res = {"out_tokens": out, "num_accepted": nacc, "p_draft": pad(pd), "q_draft": pad(qd), "bad_token": bad,
           "bad_param": badp, "cut_margin": cm, "greedy": t == 0.0, "lengths": g, "path_nodes": path,
           "match": bool(match)}
    if diagnostics:
        res["beta"], res["accept_margin"], res["race_margin"] = pad(beta), pad(am), rm
    return res


def near_tie_position(res: dict, threshold: float = 1e-4) -> np.ndarray:
    """First position whose decision had a margin <= threshold, else -1.

    The accept decision at j (j <= n) and the race at n are the decisions of
    a request; the greedy path takes none that can tie numerically.  Under
    sampler-match the races of every node the walk visited decide the path:
    a near-tie among them leaves no position fixed (0).
    """
    nacc = res["num_accepted"]
    n_req = nacc.shape[0]
    pos = np.full(n_req, -1, dtype=np.int64)
    if "accept_margin" not in res:
        return pos
    am, rm = res["accept_margin"], res["race_margin"]
    G = am.shape[1]
    for r in range(n_req):
        n = int(nacc[r])
        for j in range(min(n + 1, G)):
            if am[r, j] <= threshold:
                pos[r] = j
                break
        if pos[r] < 0 and rm[r] <= threshold:
            pos[r] = 0 if res.get("match") else n
    return pos
