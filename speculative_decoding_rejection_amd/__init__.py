"""Python binding of libspecverify (ctypes): argument marshalling only.

Every step of the verifier runs in the HIP kernels of libspecverify.so; this
module passes device pointers, sizes and the current HIP stream through the C
ABI declared in include/specverify.h, and uses PyTorch only to allocate device
memory.  There is no fallback: if the library is not built, importing a
function raises.

Same names as the C ABI: sv_workspace_bytes, sv_workspace_bytes_batch,
sv_status_string, spec_verify_prob, spec_verify_prob_noalloc,
spec_verify_onehot, spec_verify_greedy, spec_verify_batch,
sv_read_device_error, sv_kernel_timing_enable / _reset / _read,
sv_stream_read.  ``verify`` and ``verify_batch`` are convenience wrappers that
allocate the outputs and the workspace.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB may point at another build of the library (measurement of
# build variants); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_UNSUPPORTED, SV_ERR_SCRATCH = range(7)
SV_NOALLOC_SCRATCH_BYTES = 16 << 20
SV_F32, SV_BF16 = 0, 1
SV_DRAFT_LOGITS, SV_DRAFT_ONEHOT, SV_DRAFT_PROBS, SV_DRAFT_MATCH = 0, 1, 2, 3
FAMILY_ROWS, FAMILY_ACCEPT, FAMILY_RACE = 0, 1, 2


class SvParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("gamma", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("temperature", ctypes.c_float),
        ("top_k", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


class SvSampling(ctypes.Structure):
    _fields_ = [
        ("temperature", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
        ("max_top_k", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class SvLayout(ctypes.Structure):
    _fields_ = [
        ("draft_kind", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("target_stride", ctypes.c_int64),
        ("draft_stride", ctypes.c_int64),
        ("cu_draft", ctypes.c_void_p),
        ("parents", ctypes.c_void_p),
    ]


class SvOutputs(ctypes.Structure):
    _fields_ = [
        ("out_tokens", ctypes.c_void_p),
        ("num_accepted", ctypes.c_void_p),
        ("p_draft", ctypes.c_void_p),
        ("q_draft", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("counters", ctypes.c_void_p),
        ("path_nodes", ctypes.c_void_p),
    ]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sv_status_string(status)} (status {status})")


_lib = None


def load_library():
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                           f"g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(SvParams)
    lib.sv_workspace_bytes.argtypes = [pp]
    lib.sv_workspace_bytes.restype = sz
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.spec_verify_prob.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_prob.restype = ctypes.c_int
    lib.spec_verify_prob_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_verify_prob_noalloc.restype = ctypes.c_int
    lib.spec_verify_onehot.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_onehot.restype = ctypes.c_int
    lib.spec_verify_greedy.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.restype = ctypes.c_int
    ps = ctypes.POINTER(SvSampling)
    lib.sv_workspace_bytes_batch.argtypes = [pp, ps]
    lib.sv_workspace_bytes_batch.restype = sz
    pl_ = ctypes.POINTER(SvLayout)
    po = ctypes.POINTER(SvOutputs)
    lib.spec_verify_batch.argtypes = [pp, ps, pl_, vp, vp, vp, po, vp, sz, vp]
    lib.spec_verify_batch.restype = ctypes.c_int
    lib.sv_read_device_error.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
    lib.sv_read_device_error.restype = ctypes.c_int
    lib.sv_kernel_timing_enable.argtypes = [ctypes.c_int]
    lib.sv_kernel_timing_enable.restype = ctypes.c_int
    lib.sv_kernel_timing_reset.argtypes = []
    lib.sv_kernel_timing_reset.restype = ctypes.c_int
    lib.sv_kernel_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.sv_kernel_timing_read.restype = ctypes.c_int
    lib.sv_stream_read.argtypes = [vp, sz, vp, vp]
    lib.sv_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib


def make_params(batch, gamma, vocab, dtype, temperature=1.0, top_k=0, seed=0) -> SvParams:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}[dtype]
    return SvParams(int(batch), int(gamma), int(vocab), int(dtype), float(temperature), int(top_k),
                    int(seed) & 0xFFFFFFFFFFFFFFFF)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libspecverify takes device tensors")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status, where):
    if status != SV_OK:
        raise SpecVerifyError(status, where)


def sv_status_string(status: int) -> str:
    return load_library().sv_status_string(int(status)).decode()


def sv_workspace_bytes(params: SvParams) -> int:
    return int(load_library().sv_workspace_bytes(ctypes.byref(params)))


def spec_verify_prob(params, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted, p_draft,
                     q_draft, workspace, stream=None):
    st = load_library().spec_verify_prob(ctypes.byref(params), _ptr(target_logits), _ptr(draft_logits),
                                         _ptr(draft_tokens), _ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft),
                                         _ptr(q_draft), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "spec_verify_prob")


def spec_verify_prob_noalloc(params, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted, p_draft,
                             q_draft, error_word=None, stream=None):
    st = load_library().spec_verify_prob_noalloc(ctypes.byref(params), _ptr(target_logits), _ptr(draft_logits),
                                                 _ptr(draft_tokens), _ptr(out_tokens), _ptr(num_accepted),
                                                 _ptr(p_draft), _ptr(q_draft), _ptr(error_word), _stream(stream))
    _check(st, "spec_verify_prob_noalloc")


def spec_verify_onehot(params, target_logits, draft_tokens, out_tokens, num_accepted, p_draft, workspace,
                       stream=None):
    st = load_library().spec_verify_onehot(ctypes.byref(params), _ptr(target_logits), _ptr(draft_tokens),
                                           _ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft), _ptr(workspace),
                                           workspace.numel(), _stream(stream))
    _check(st, "spec_verify_onehot")


def spec_verify_greedy(params, target_logits, draft_tokens, out_tokens, num_accepted, target_argmax, workspace,
                       stream=None):
    st = load_library().spec_verify_greedy(ctypes.byref(params), _ptr(target_logits), _ptr(draft_tokens),
                                           _ptr(out_tokens), _ptr(num_accepted), _ptr(target_argmax),
                                           _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "spec_verify_greedy")


def make_sampling(temperature, top_k=None, top_p=None, max_top_k: int = 0) -> SvSampling:
    """Per-request settings from device tensors: temperature [B] float32,
    top_k [B] int32 or None, top_p [B] float32 or None.  The returned struct
    holds raw pointers: keep the tensors alive while it is used."""
    def chk(t, dt):
        if t is None:
            return None
        if t.dtype != dt:
            raise ValueError(f"expected {dt}, got {t.dtype}")
        return _ptr(t)
    return SvSampling(chk(temperature, torch.float32), chk(top_k, torch.int32), chk(top_p, torch.float32),
                      int(max_top_k), 0)


def sv_workspace_bytes_batch(params: SvParams, sampling) -> int:
    return int(load_library().sv_workspace_bytes_batch(ctypes.byref(params),
                                                       ctypes.byref(sampling) if sampling else None))


def make_outputs(out_tokens, num_accepted, p_draft=None, q_draft=None, beta=None, counters=None,
                 path_nodes=None) -> SvOutputs:
    """Output pointers of spec_verify_batch (device tensors; counters int64
    [B, 3], accumulated across calls; path_nodes int32 [B, G+1] for
    sampler-match).  Keep the tensors alive while the struct is used."""
    if counters is not None and counters.dtype != torch.int64:
        raise ValueError("counters must be int64")
    if path_nodes is not None and path_nodes.dtype != torch.int32:
        raise ValueError("path_nodes must be int32")
    return SvOutputs(_ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft), _ptr(q_draft), _ptr(beta),
                     _ptr(counters), _ptr(path_nodes))


def spec_verify_batch(params, sampling, layout, target_logits, draft, draft_tokens, outputs, workspace,
                      stream=None):
    """sampling (SvSampling) and layout (SvLayout) may be None; outputs is an
    SvOutputs (make_outputs)."""
    st = load_library().spec_verify_batch(ctypes.byref(params), ctypes.byref(sampling) if sampling else None,
                                          ctypes.byref(layout) if layout else None, _ptr(target_logits),
                                          _ptr(draft), _ptr(draft_tokens), ctypes.byref(outputs), _ptr(workspace),
                                          workspace.numel(), _stream(stream))
    _check(st, "spec_verify_batch")


def sv_read_device_error(workspace, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(load_library().sv_read_device_error(_ptr(workspace), ctypes.byref(code), _stream(stream)),
           "sv_read_device_error")
    return int(code.value)


def sv_kernel_timing_enable(enable: bool) -> None:
    _check(load_library().sv_kernel_timing_enable(1 if enable else 0), "sv_kernel_timing_enable")


def sv_kernel_timing_reset() -> None:
    _check(load_library().sv_kernel_timing_reset(), "sv_kernel_timing_reset")


def sv_kernel_timing_read(family: int) -> tuple[float, int]:
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(load_library().sv_kernel_timing_read(int(family), ctypes.byref(ms), ctypes.byref(n)),
           "sv_kernel_timing_read")
    return float(ms.value), int(n.value)


def sv_stream_read(buf, sink, stream=None) -> None:
    """One streaming read of the whole device tensor `buf` (measurement)."""
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().sv_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "sv_stream_read")


def alloc_workspace(params: SvParams, device) -> torch.Tensor:
    nbytes = sv_workspace_bytes(params)
    if nbytes == 0:
        raise SpecVerifyError(SV_ERR_INVALID_ARG, "sv_workspace_bytes")
    # torch's caching allocator returns 256-byte-aligned blocks.
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def verify(entry: str, target_logits, draft_tokens, draft_logits=None, *, temperature=1.0, top_k=0, seed=0,
           workspace=None, stream=None) -> dict:
    """Allocates outputs (and a workspace if none is given) and runs one entry
    point.  target_logits [B, G+1, V] fp32/bf16 on the GPU; draft_tokens
    [B, G] int32; draft_logits [B, G, V] for the "prob" entry."""
    B, G1, V = target_logits.shape
    G = G1 - 1
    dev = target_logits.device
    params = make_params(B, G, V, target_logits.dtype, temperature, top_k, seed)
    ws = workspace if workspace is not None else alloc_workspace(params, dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    res = {"out_tokens": out, "num_accepted": nacc, "workspace": ws}
    if entry == "prob":
        pd = torch.empty((B, G), dtype=torch.float32, device=dev)
        qd = torch.empty((B, G), dtype=torch.float32, device=dev)
        spec_verify_prob(params, target_logits, draft_logits, draft_tokens, out, nacc, pd, qd, ws, stream)
        res.update(p_draft=pd, q_draft=qd)
    elif entry == "onehot":
        pd = torch.empty((B, G), dtype=torch.float32, device=dev)
        spec_verify_onehot(params, target_logits, draft_tokens, out, nacc, pd, ws, stream)
        res.update(p_draft=pd)
    elif entry == "greedy":
        ta = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
        spec_verify_greedy(params, target_logits, draft_tokens, out, nacc, ta, ws, stream)
        res.update(target_argmax=ta)
    else:
        raise ValueError(entry)
    return res


def verify_batch(target_logits, draft_tokens, draft=None, *, temperature=None, top_k=None, top_p=None,
                 max_top_k=None, seed=0, draft_kind=None, cu_draft=None, gamma=None, vocab=None,
                 single_temperature=1.0, single_top_k=0, beta=False, counters=None, parents=None, workspace=None,
                 stream=None) -> dict:
    """Allocates outputs (and a workspace if none is given) and runs
    spec_verify_batch.

    Dense: target_logits [B, G+1, W], draft [B, G, W] (logits, or float32
    probabilities with draft_kind SV_DRAFT_PROBS; None: one-hot drafts),
    draft_tokens [B, G].  Ragged (cu_draft [B+1] int32 given, gamma = the
    largest draft length): target_logits [sum(g_b + 1), W], draft
    [sum(g_b), W], draft_tokens [sum(g_b)].  W is the row stride; vocab
    (default W) the number of valid logits per row.  temperature / top_k /
    top_p: [B] device tensors (float32 / int32 / float32), or temperature
    None for one setting for every request (single_temperature,
    single_top_k).  max_top_k (the bound on every top_k below vocab) defaults
    to 1024 when top_k is given; pass it for top_k above 1024 (a request whose
    top_k exceeds max_top_k and is below vocab is invalid).  beta:
    also return the per-position acceptance probability; counters: an int64
    [B, 3] device tensor the call adds its round to.  draft_kind
    SV_DRAFT_MATCH: sampler-match over chains, or over trees with parents
    (int32, laid out like draft_tokens); also returns path_nodes [B, G+1]."""
    dev = target_logits.device
    W = target_logits.shape[-1]
    V = int(vocab) if vocab is not None else W
    if cu_draft is not None:
        B = cu_draft.shape[0] - 1
        G = int(gamma)
        tok_shape = draft_tokens.shape
    else:
        B, G1, _ = target_logits.shape
        G = G1 - 1
        tok_shape = (B, G)
    if draft_kind is None:
        draft_kind = SV_DRAFT_ONEHOT if draft is None else SV_DRAFT_LOGITS
    dW = draft.shape[-1] if draft is not None else 0
    layout = SvLayout(int(draft_kind), 0, W, dW, _ptr(cu_draft), _ptr(parents))
    sampling = None
    if temperature is not None:
        if max_top_k is None:
            max_top_k = 1024 if top_k is not None else 0
        sampling = make_sampling(temperature, top_k, top_p, max_top_k)
    params = make_params(B, G, V, target_logits.dtype, single_temperature, single_top_k, seed)
    nbytes = sv_workspace_bytes_batch(params, sampling)
    if nbytes == 0:
        raise SpecVerifyError(SV_ERR_INVALID_ARG, "sv_workspace_bytes_batch")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    pd = torch.empty(tok_shape, dtype=torch.float32, device=dev)
    qd = torch.empty(tok_shape, dtype=torch.float32, device=dev)
    bt = torch.empty(tok_shape, dtype=torch.float32, device=dev) if beta else None
    pn = torch.empty((B, G + 1), dtype=torch.int32, device=dev) if draft_kind == SV_DRAFT_MATCH else None
    outputs = make_outputs(out, nacc, pd, qd, bt, counters, pn)
    spec_verify_batch(params, sampling, layout, target_logits, draft, draft_tokens, outputs, ws, stream)
    res = {"out_tokens": out, "num_accepted": nacc, "p_draft": pd, "q_draft": qd, "workspace": ws}
    if pn is not None:
        res["path_nodes"] = pn
    if beta:
        res["beta"] = bt
    return res
