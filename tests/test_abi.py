"""CPU checks of the C-ABI library: it loads, exports every symbol that
include/specverify.h declares, sizes workspaces, and rejects bad arguments
before touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_rejection_amd as sv
    from speculative_decoding_rejection_amd import build as b
    if b.is_stale():
        b.build()
    sv.load_library()
    return sv


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_exports_every_declared_symbol(sv):
    names = _declared_functions()
    assert "spec_verify_prob" in names and "spec_verify_greedy" in names and "sv_workspace_bytes" in names
    lib = sv.load_library()
    for n in names:
        assert hasattr(lib, n), f"symbol {n} declared in include/ but not exported"


def test_workspace_sizing(sv):
    p = sv.make_params(1024, 8, 256000, sv.SV_BF16, 0.7, 64, 42)
    n = sv.sv_workspace_bytes(p)
    # Candidates: 17408 rows x 64 keys x 8 bytes, plus small per-request state.
    assert 17408 * 64 * 8 <= n < 17408 * 64 * 8 + 4 * 2**20
    assert sv.sv_workspace_bytes(sv.make_params(0, 8, 100, sv.SV_F32)) == 0
    assert sv.sv_workspace_bytes(sv.make_params(4, 2, 100, sv.SV_F32, 0.0)) > 0  # greedy parameters


@pytest.mark.parametrize("B,G,V,bf16", [(8, 4, 32000, False), (64, 5, 128256, True), (256, 7, 151936, False),
                                        (512, 3, 262144, True), (1024, 8, 256000, True)])
def test_one_workspace_size_for_every_entry(sv, B, G, V, bf16):
    """spec_verify_greedy ignores temperature and top_k, so a workspace
    sized from sampled parameters must also fit a greedy call of the same
    shape: never smaller than the size for temperature 0 (the greedy plan)."""
    dt = sv.SV_BF16 if bf16 else sv.SV_F32
    greedy = sv.sv_workspace_bytes(sv.make_params(B, G, V, dt, 0.0, 0, 1))
    assert greedy > 0
    for T, k in ((1.0, 0), (0.7, 64), (1.0, 1000), (1.0, 2000)):
        assert sv.sv_workspace_bytes(sv.make_params(B, G, V, dt, T, k, 1)) >= greedy, (T, k)


def _call_prob(sv, params, ws_bytes=1 << 20, null=None):
    lib = sv.load_library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    args = [fake] * 5
    if null is not None:
        args[null] = None
    return lib.spec_verify_prob(ctypes.byref(params), args[0], args[1], args[2], args[3], args[4], None, None,
                                fake, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(gamma=0), 1), (dict(vocab=0), 1), (dict(dtype=7), 2),
    (dict(temperature=0.0), 1), (dict(temperature=-1.0), 1), (dict(temperature=float("inf")), 1),
    (dict(top_k=-1), 1), (dict(gamma=16385), 5),
])
def test_argument_errors(sv, kw, status):
    base = dict(batch=4, gamma=3, vocab=5000, dtype=sv.SV_BF16, temperature=1.0, top_k=0, seed=1)
    base.update(kw)
    assert _call_prob(sv, sv.make_params(**base)) == status


def test_null_pointers_and_workspace(sv):
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 1.0, 0, 1)
    for i in range(5):
        assert _call_prob(sv, p, null=i) == sv.SV_ERR_INVALID_ARG
    assert _call_prob(sv, p, ws_bytes=16) == sv.SV_ERR_WORKSPACE
    lib = sv.load_library()
    assert lib.sv_read_device_error(None, None, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_kernel_timing_read(9, None, None) == sv.SV_ERR_INVALID_ARG


def test_top_k_at_or_above_vocab_is_accepted(sv):
    # top_k >= V is "off", never unsupported.
    p = sv.make_params(4, 3, 500, sv.SV_BF16, 1.0, 5000, 1)
    assert _call_prob(sv, p, ws_bytes=16) == sv.SV_ERR_WORKSPACE  # reaches the workspace check


def test_large_top_k_is_accepted(sv):
    # 1024 < top_k < V: a cut over each full row (one RowCut per row).
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 1.0, 2000, 1)
    assert _call_prob(sv, p, ws_bytes=16) == sv.SV_ERR_WORKSPACE  # reaches the workspace check
    assert _call_prob(sv, sv.make_params(4, 3, 5000, sv.SV_BF16, 0.0, 2000, 1), ws_bytes=16) == \
        sv.SV_ERR_INVALID_ARG  # temperature 0 is the greedy entry's
    rows = 4 * 7
    small = sv.sv_workspace_bytes(sv.make_params(4, 3, 5000, sv.SV_BF16, 1.0, 1000, 1))
    large = sv.sv_workspace_bytes(p)
    assert small >= rows * 1000 * 8                  # 1000 candidate keys per row
    assert rows * 16 <= large < small                # one cut per row, no candidates


def test_status_strings(sv):
    for s in range(6):
        assert sv.sv_status_string(s)


def _call_batch(sv, params, sampling, ws_bytes=1 << 20, null=None, layout=None, draft=None):
    lib = sv.load_library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    args = [fake] * 5
    if null is not None:
        args[null] = None
    sp = ctypes.byref(sampling) if sampling is not None else None
    lp = ctypes.byref(layout) if layout is not None else None
    outs = sv.SvOutputs(args[2], args[3], None, None, None, None)
    return lib.spec_verify_batch(ctypes.byref(params), sp, lp, args[0], draft, args[1], ctypes.byref(outs), args[4],
                                 ws_bytes, None)


def test_batch_argument_errors(sv):
    fake = 1 << 21
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 1.0, 0, 1)
    ok = sv.SvSampling(fake, fake, fake, 64, 0)
    assert _call_batch(sv, p, ok, ws_bytes=16) == sv.SV_ERR_WORKSPACE  # everything else valid
    assert _call_batch(sv, p, sv.SvSampling(None, fake, fake, 64, 0)) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, sv.SvSampling(fake, fake, fake, -1, 0)) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, sv.SvSampling(fake, fake, fake, 1025, 0), ws_bytes=16) == sv.SV_ERR_WORKSPACE
    for i in range(4):
        assert _call_batch(sv, p, ok, null=i) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, ok, null=4) == sv.SV_ERR_WORKSPACE
    # params->temperature and ->top_k are not used by the batch entry.
    p2 = sv.make_params(4, 3, 5000, sv.SV_BF16, -5.0, 99999, 1)
    assert _call_batch(sv, p2, ok, ws_bytes=16) == sv.SV_ERR_WORKSPACE


def test_batch_workspace_sizing(sv):
    fake = 1 << 21
    p = sv.make_params(256, 7, 151936, sv.SV_F32, 1.0, 0, 1)
    plain = sv.sv_workspace_bytes_batch(p, sv.SvSampling(fake, None, None, 0, 0))
    topk = sv.sv_workspace_bytes_batch(p, sv.SvSampling(fake, fake, None, 64, 0))
    nuc = sv.sv_workspace_bytes_batch(p, sv.SvSampling(fake, fake, fake, 64, 0))
    rows = 256 * 15
    assert topk - plain >= rows * 64 * 8           # candidate keys of every row
    assert nuc - topk >= rows * 16                  # one nucleus cut per row
    assert plain >= sv.sv_workspace_bytes(sv.make_params(256, 7, 151936, sv.SV_F32, 1.0, 0, 1))
    assert sv.sv_workspace_bytes_batch(sv.make_params(0, 7, 100, sv.SV_F32), sv.SvSampling(fake, None, None, 0, 0)) == 0


def test_batch_single_setting_and_layout_errors(sv):
    fake = 1 << 21
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 0.7, 64, 1)
    # No per-request settings: params' temperature / top_k apply to every request.
    assert _call_batch(sv, p, None, ws_bytes=16) == sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, sv.make_params(4, 3, 5000, sv.SV_BF16, 0.0, 0, 1), None, ws_bytes=16) == sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, sv.make_params(4, 3, 5000, sv.SV_BF16, -1.0, 0, 1), None) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, sv.make_params(4, 3, 5000, sv.SV_BF16, 1.0, 2000, 1), None, ws_bytes=16) == \
        sv.SV_ERR_WORKSPACE
    ok = sv.SvSampling(fake, None, None, 0, 0)
    L = sv.SvLayout
    d = ctypes.c_void_p(fake)
    assert _call_batch(sv, p, ok, ws_bytes=16, layout=L(sv.SV_DRAFT_PROBS, 0, 0, 0, None), draft=d) == \
        sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, p, ok, layout=L(7, 0, 0, 0, None), draft=d) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, ok, layout=L(sv.SV_DRAFT_PROBS, 0, 0, 0, None)) == sv.SV_ERR_INVALID_ARG  # no draft
    assert _call_batch(sv, p, ok, layout=L(sv.SV_DRAFT_LOGITS, 0, 4999, 0, None), draft=d) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, ok, layout=L(sv.SV_DRAFT_LOGITS, 0, 0, 4000, None), draft=d) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, ok, ws_bytes=16, layout=L(sv.SV_DRAFT_LOGITS, 0, 5120, 5008, fake), draft=d) == \
        sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, p, ok, layout=L(sv.SV_DRAFT_LOGITS, 0, 0, 0, fake + 2), draft=d) == sv.SV_ERR_INVALID_ARG


def test_batch_outputs_checks(sv):
    lib = sv.load_library()
    fake = ctypes.c_void_p(1 << 20)
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 0.7, 0, 1)
    assert lib.spec_verify_batch(ctypes.byref(p), None, None, fake, None, fake, None, fake, 1 << 20, None) == \
        sv.SV_ERR_INVALID_ARG
    outs = sv.SvOutputs(1 << 20, 1 << 20, None, None, None, (1 << 20) + 4)  # counters must be 8-byte aligned
    assert lib.spec_verify_batch(ctypes.byref(p), None, None, fake, None, fake, ctypes.byref(outs), fake, 1 << 20,
                                 None) == sv.SV_ERR_INVALID_ARG


def test_batch_match_layout_errors(sv):
    """Sampler-match: no draft rows are read; parents only with this kind and
    4-byte aligned; path_nodes 4-byte aligned."""
    fake = 1 << 21
    p = sv.make_params(4, 3, 5000, sv.SV_BF16, 0.7, 0, 1)
    ok = sv.SvSampling(fake, None, None, 0, 0)
    L = sv.SvLayout
    d = ctypes.c_void_p(fake)
    M = sv.SV_DRAFT_MATCH
    assert _call_batch(sv, p, ok, ws_bytes=16, layout=L(M, 0, 0, 0, None, None)) == sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, p, ok, ws_bytes=16, layout=L(M, 0, 0, 0, None, fake)) == sv.SV_ERR_WORKSPACE
    assert _call_batch(sv, p, ok, layout=L(M, 0, 0, 0, None, fake + 2)) == sv.SV_ERR_INVALID_ARG
    assert _call_batch(sv, p, ok, layout=L(sv.SV_DRAFT_LOGITS, 0, 0, 0, None, fake), draft=d) == \
        sv.SV_ERR_INVALID_ARG  # parents with another kind
    assert _call_batch(sv, p, ok, layout=L(4, 0, 0, 0, None, None)) == sv.SV_ERR_INVALID_ARG
    lib = sv.load_library()
    outs = sv.SvOutputs(1 << 20, 1 << 20, None, None, None, None, (1 << 20) + 2)
    assert lib.spec_verify_batch(ctypes.byref(p), ctypes.byref(ok), ctypes.byref(L(M, 0, 0, 0, None, None)),
                                 d, None, d, ctypes.byref(outs), d, 1 << 20, None) == sv.SV_ERR_INVALID_ARG


@pytest.mark.parametrize("B,G", [(1, 1), (3, 2), (256, 7)])
def test_batch_workspace_holds_the_split_nucleus(sv, B, G):
    """With top-p settings the workspace also holds the split nucleus passes'
    buffers: the row list, chunk histograms for min(1024, 16 x rows) chunks
    (4104 doubles each: a window of 4096 bins and its record; rows capped at 512), and a 2048-key buffer per split
    row; calls without top-p carry none of it."""
    fake = 1 << 21
    p = sv.make_params(B, G, 5003, sv.SV_F32, 1.0, 0, 1)
    topk = sv.sv_workspace_bytes_batch(p, sv.SvSampling(fake, fake, None, 64, 0))
    nuc = sv.sv_workspace_bytes_batch(p, sv.SvSampling(fake, fake, fake, 64, 0))
    rows = B * (2 * G + 1)
    split_rows = min(rows, 512)
    items = min(1024, 16 * split_rows)
    need = rows * 16 + rows * 4 + items * 4104 * 8 + split_rows * 2048 * 8
    assert nuc - topk >= need
    assert nuc - topk <= need + split_rows * 64 + 16 * 4096  # state records and alignment


def test_noalloc_limits_before_any_gpu_call(sv):
    """spec_verify_prob_noalloc checks its parameters and its scratch limit
    before any HIP call: an oversized call, a top-k above 1024 and bad sizes
    are refused on a machine without a GPU."""
    lib = sv.load_library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced

    def call(p):
        return lib.spec_verify_prob_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, None, None)

    big = sv.make_params(4096, 8, 256000, sv.SV_BF16, 0.7, 1024, 1)
    assert sv.sv_workspace_bytes(big) > sv.SV_NOALLOC_SCRATCH_BYTES
    assert call(big) == sv.SV_ERR_SCRATCH
    assert call(sv.make_params(4, 2, 5000, sv.SV_BF16, 0.7, 2000, 1)) == sv.SV_ERR_UNSUPPORTED
    assert call(sv.make_params(0, 2, 5000, sv.SV_BF16, 0.7, 0, 1)) == sv.SV_ERR_INVALID_ARG
    assert call(sv.make_params(4, 2, 5000, sv.SV_BF16, 0.0, 0, 1)) == sv.SV_ERR_INVALID_ARG
    # The headline call fits.
    head = sv.make_params(1024, 8, 256000, sv.SV_BF16, 0.7, 64, 42)
    assert sv.sv_workspace_bytes(head) <= sv.SV_NOALLOC_SCRATCH_BYTES
    assert "16 MiB" in sv.sv_status_string(sv.SV_ERR_SCRATCH)


def test_stream_read_rejects_bad_arguments(sv):
    """The read-ceiling measurement hook validates before enqueueing."""
    lib = sv.load_library()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert lib.sv_stream_read(None, 1 << 20, fake, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_stream_read(fake, 1 << 20, None, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_stream_read(fake, 24, fake, None) == sv.SV_ERR_INVALID_ARG   # not a multiple of 16
    assert lib.sv_stream_read(odd, 1 << 20, fake, None) == sv.SV_ERR_INVALID_ARG  # not 16-byte aligned
    assert lib.sv_stream_read(fake, 0, fake, None) == sv.SV_ERR_INVALID_ARG
