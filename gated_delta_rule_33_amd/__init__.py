"""Python binding for libkda, the gfx950 Kimi Delta Attention library.

Argument marshalling only: every step of the operator runs in the HIP
kernels of ``libkda.so`` behind the C ABI declared in ``include/kda.h``.
PyTorch supplies device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library is missing, or a tensor is not on a GPU,
these functions raise.

    o, S_T = prefill(q, k, v, log_alpha, beta, cu_seqlens, S0=None)
    o      = decode_step(q, k, v, log_alpha, beta, S)      # S updated in place
    prefill_recovered(...)   # did the last overlapped call fall back?
    g = prefill_backward(q, k, v, log_alpha, beta, cu_seqlens, S0, dO, dS_T)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_DEVICE = 4
KDA_F32 = 0
KDA_BF16 = 1
KDA_PREFILL_ONE_STREAM = 1
KDA_PREFILL_BOUNDED = 2
KDA_GATE_CHANNEL = 0
KDA_GATE_SCALAR = 1
KDA_GATE_NONE = 2

EXPORTED = ("kda_prefill", "kda_prefill_workspace_size", "kda_prefill_noalloc", "kda_prefill_recovered",
            "kda_prefill_set_wait_limit", "kda_decode_step", "kda_prefill_backward_workspace_size",
            "kda_prefill_backward", "kda_status_string", "kda_version")
NOALLOC_SCRATCH_BYTES = 256 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


class Stages(ctypes.Structure):
    """kda_stages: input and output stages around the recurrence."""
    _fields_ = [
        ("l2norm_qk", ctypes.c_int32),
        ("l2norm_eps", ctypes.c_float),
        ("gate_softplus", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("out_gate", ctypes.c_void_p),
    ]


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("io_dtype", ctypes.c_int),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("flags", ctypes.c_uint32),
        ("gate", ctypes.c_int),
        ("stages", ctypes.POINTER(Stages)),
    ]


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libkda.so and declare its C signatures.  Works without a GPU
    (validation-only calls and symbol checks need no device)."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libkda.so not built: run `python -m gated_delta_rule_33_amd.build` (%s)" % path)
        lib = ctypes.CDLL(path)
        vp, fp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_version.restype = ctypes.c_int32
        lib.kda_version.argtypes = []
        lib.kda_prefill_workspace_size.restype = ctypes.c_size_t
        lib.kda_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc)]
        lib.kda_prefill.restype = ctypes.c_int
        lib.kda_prefill.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]
        lib.kda_prefill_noalloc.restype = ctypes.c_int
        lib.kda_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_prefill_recovered.restype = ctypes.c_int
        lib.kda_prefill_recovered.argtypes = [ctypes.POINTER(PrefillDesc), vp, ctypes.POINTER(ctypes.c_int32), vp]
        lib.kda_prefill_set_wait_limit.restype = ctypes.c_int32
        lib.kda_prefill_set_wait_limit.argtypes = [ctypes.c_int32]
        lib.kda_prefill_backward_workspace_size.restype = ctypes.c_size_t
        lib.kda_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc)]
        lib.kda_prefill_backward.restype = ctypes.c_int
        lib.kda_prefill_backward.argtypes = [ctypes.POINTER(PrefillDesc)] + [vp] * 16 + [ctypes.c_size_t, vp]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                        ctypes.c_int, ctypes.POINTER(Stages), vp, vp, vp, vp, vp, vp, vp, vp]
        if path == LIB_PATH:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().kda_version())


def make_desc(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int, chunk: int, io_dtype: int,
              cu_seqlens_host: Optional[Sequence[int]] = None, flags: int = 0, gate: int = 0, stages=None):
    """Build a kda_prefill_desc.  Returns (desc, keepalive) -- keep the second
    value alive while the desc is used (it owns the host offsets)."""
    keep = None
    ptr = ctypes.POINTER(ctypes.c_int32)()
    if cu_seqlens_host is not None:
        keep = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
        ptr = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    d = PrefillDesc(int(num_seqs), int(total_tokens), int(num_heads), int(dk), int(dv), int(chunk), int(io_dtype),
                    ptr, int(flags), int(gate), ctypes.pointer(stages) if stages is not None else None)
    return d, (keep, stages)


def prefill_workspace_size(desc: PrefillDesc) -> int:
    return int(load_library().kda_prefill_workspace_size(ctypes.byref(desc)))


# ---------------------------------------------------------------------------
# torch-facing helpers (torch supplies memory and streams only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _dev_ptr(t, name: str, dtype=None, shape=None, device=None) -> int:
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    return t.data_ptr()


def _gate(log_alpha, lead) -> int:
    """Gate form from log_alpha: None -> no gate; [*lead] -> one rate per
    head; [*lead, dk] -> one rate per key channel."""
    if log_alpha is None:
        return KDA_GATE_NONE
    if log_alpha.dim() == len(lead):
        return KDA_GATE_SCALAR
    return KDA_GATE_CHANNEL


def _la_shape(gate: int, lead, dk: int):
    return None if gate == KDA_GATE_NONE else (tuple(lead) if gate == KDA_GATE_SCALAR else tuple(lead) + (dk,))


def _stages(shape_o, dtype, device, l2norm_qk=False, gate_softplus=False, out_gate=None, norm_weight=None,
            l2norm_eps=1e-6, norm_eps=1e-6):
    """A kda_stages struct for the keyword arguments (None when no stage is
    selected).  out_gate: tensor shaped like o in its dtype; norm_weight: [dv]
    fp32 tensor."""
    torch = _torch()
    if not (l2norm_qk or gate_softplus or out_gate is not None or norm_weight is not None):
        return None
    return Stages(int(bool(l2norm_qk)), float(l2norm_eps), int(bool(gate_softplus)),
                  _dev_ptr(norm_weight, "norm_weight", torch.float32, (shape_o[-1],), device),
                  float(norm_eps), _dev_ptr(out_gate, "out_gate", dtype, shape_o, device))


def _stream(stream):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


# One prefill workspace per (device, stream), grown on demand.  A workspace
# is allocated on the stream that uses it, so when it is replaced the caching
# allocator reuses its memory only after that stream's pending work.
_ws_cache = {}
_ws_lock = threading.Lock()


def _workspace(device, stream, need: int, kind: str = "prefill"):
    torch = _torch()
    key = (device, stream.cuda_stream) if kind == "prefill" else (device, stream.cuda_stream, kind)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < need:
            _ws_cache.pop(key, None)
            del ws
            with torch.cuda.stream(stream):
                ws = torch.empty(need, dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def clear_workspace_cache():
    """Drop the cached prefill workspaces (their memory returns to torch's
    caching allocator once the streams that used them reach this point)."""
    with _ws_lock:
        _ws_cache.clear()


def prefill(q, k, v, log_alpha, beta, cu_seqlens, S0=None, *, chunk: int = 64, o=None, S_T=None,
            cu_seqlens_host: Optional[Sequence[int]] = None, workspace=None, stream=None, want_state: bool = True,
            one_stream: bool = False, max_workspace_bytes: Optional[int] = None, **stage_kw):
    """KDA chunked prefill over a packed batch.

    q, k: [T, H, dk]; v: [T, H, dv] (bf16 or fp32, same dtype); log_alpha: [T, H, dk]
    fp32; beta: [T, H] fp32; cu_seqlens: [N+1] int32 (GPU); S0: [N, H, dk, dv] fp32 or
    None.  Returns (o, S_T); S_T is None when ``want_state`` is False.
    ``S_T`` may be passed as ``S0`` to update the state in place.
    ``one_stream`` selects the schedule that never leaves the caller's stream.
    ``max_workspace_bytes`` selects the bounded schedule (KDA_PREFILL_BOUNDED):
    the library uses at most that many workspace bytes, whatever the token
    count, taking the chunks in segments that fit.
    ``log_alpha`` may also be [T, H] (one rate per head: Gated DeltaNet) or
    None (no forget gate: DeltaNet).  Stage keywords (kda_stages):
    ``l2norm_qk``, ``gate_softplus`` (log_alpha then holds the gate
    projection's output), ``norm_weight`` ([dv] fp32), ``out_gate`` (like o),
    ``l2norm_eps``, ``norm_eps``.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3 or cu_seqlens.dim() != 1:
        raise ValueError("q, k, v must be [T, H, d] and cu_seqlens [N+1]")
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    dt = _dtype_code(q)
    dev = q.device
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    s = _stream(stream)
    gate = _gate(log_alpha, (T, H))
    stg = _stages((T, H, dv), q.dtype, dev, **stage_kw)
    flags = (KDA_PREFILL_ONE_STREAM if one_stream else 0) | (KDA_PREFILL_BOUNDED if max_workspace_bytes else 0)
    desc, keep = make_desc(N, T, H, dk, dv, chunk, dt, cu_seqlens_host, flags, gate, stg)
    need = int(lib.kda_prefill_workspace_size(ctypes.byref(desc)))
    if need == 0:
        st = lib.kda_prefill(ctypes.byref(desc), *([None] * 10), 0, None)
        raise KdaError(st if st != KDA_OK else KDA_ERR_INVALID_ARGUMENT, "kda_prefill_workspace_size")
    if max_workspace_bytes:
        if need > max_workspace_bytes:
            raise KdaError(KDA_ERR_WORKSPACE_TOO_SMALL, "kda_prefill (bounded: %d bytes at least)" % need)
        # beyond the one-stream schedule's workspace (plus the carried
        # states) a longer segment gains nothing
        one, keep1 = make_desc(N, T, H, dk, dv, chunk, dt, cu_seqlens_host, KDA_PREFILL_ONE_STREAM, gate, stg)
        full = int(lib.kda_prefill_workspace_size(ctypes.byref(one))) + N * H * dk * dv * 4 + 256
        need = min(int(max_workspace_bytes) // 256 * 256, full)
    ptrs = (_dev_ptr(q, "q", None, (T, H, dk), dev), _dev_ptr(k, "k", None, (T, H, dk), dev),
            _dev_ptr(v, "v", None, (T, H, dv), dev),
            _dev_ptr(log_alpha, "log_alpha", torch.float32, _la_shape(gate, (T, H), dk), dev),
            _dev_ptr(beta, "beta", torch.float32, (T, H), dev),
            _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev),
            _dev_ptr(S0, "S0", torch.float32, (N, H, dk, dv), dev),
            _dev_ptr(o, "o", q.dtype, (T, H, dv), dev),
            _dev_ptr(S_T, "S_T", torch.float32, (N, H, dk, dv), dev))
    if workspace is None:
        workspace = _workspace(dev, s, need)
    wptr = _dev_ptr(workspace, "workspace", None, None, dev)
    wbytes = workspace.numel() * workspace.element_size()
    if max_workspace_bytes:
        wbytes = min(wbytes, need)
    st = lib.kda_prefill(ctypes.byref(desc), *ptrs, wptr, wbytes, s.cuda_stream)
    del keep
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill")
    return o, S_T


def prefill_noalloc(q, k, v, log_alpha, beta, cu_seqlens, S0=None, *, chunk: int = 64, o=None, S_T=None,
                    cu_seqlens_host: Optional[Sequence[int]] = None, stream=None, want_state: bool = True,
                    **stage_kw):
    """kda_prefill_noalloc: the prefill with the library's static per-GPU
    scratch as its workspace (no device allocation inside the call; the
    binding still allocates o and S_T unless they are passed in).  Same
    arguments and results as ``prefill``; problems whose workspace exceeds
    NOALLOC_SCRATCH_BYTES raise KdaError(KDA_ERR_WORKSPACE_TOO_SMALL)."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3 or cu_seqlens.dim() != 1:
        raise ValueError("q, k, v must be [T, H, d] and cu_seqlens [N+1]")
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    dt = _dtype_code(q)
    dev = q.device
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    gate = _gate(log_alpha, (T, H))
    desc, keep = make_desc(N, T, H, dk, dv, chunk, dt, cu_seqlens_host, 0, gate,
                           _stages((T, H, dv), q.dtype, dev, **stage_kw))
    st = lib.kda_prefill_noalloc(ctypes.byref(desc),
                                 _dev_ptr(q, "q", None, (T, H, dk), dev), _dev_ptr(k, "k", None, (T, H, dk), dev),
                                 _dev_ptr(v, "v", None, (T, H, dv), dev),
                                 _dev_ptr(log_alpha, "log_alpha", torch.float32, _la_shape(gate, (T, H), dk), dev),
                                 _dev_ptr(beta, "beta", torch.float32, (T, H), dev),
                                 _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev),
                                 _dev_ptr(S0, "S0", torch.float32, (N, H, dk, dv), dev),
                                 _dev_ptr(o, "o", q.dtype, (T, H, dv), dev),
                                 _dev_ptr(S_T, "S_T", torch.float32, (N, H, dk, dv), dev),
                                 _stream(stream).cuda_stream)
    del keep
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill_noalloc")
    return o, S_T


def prefill_recovered(q, v, cu_seqlens, *, chunk: int = 64, cu_seqlens_host=None, workspace=None, stream=None,
                      one_stream: bool = False, max_workspace_bytes: Optional[int] = None) -> bool:
    """Whether the last prefill call with these shapes on ``stream`` (using
    ``workspace``, or the binding's cached one for that stream) stopped
    waiting in its overlapped schedule and recomputed its outputs on the
    caller's stream.  Synchronises the stream.  Pass the call's
    ``one_stream`` and ``max_workspace_bytes``: those schedules never wait
    (False without a look at the workspace)."""
    if max_workspace_bytes:
        return False
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    s = _stream(stream)
    desc, keep = make_desc(N, T, H, dk, dv, chunk, _dtype_code(q), cu_seqlens_host,
                           KDA_PREFILL_ONE_STREAM if one_stream else 0)
    if workspace is None:
        with _ws_lock:
            workspace = _ws_cache.get((q.device, s.cuda_stream))
    if workspace is None:
        raise RuntimeError("no prefill workspace for this stream")
    out = ctypes.c_int32(0)
    st = lib.kda_prefill_recovered(ctypes.byref(desc), workspace.data_ptr(), ctypes.byref(out), s.cuda_stream)
    del keep
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill_recovered")
    return bool(out.value)


def prefill_backward(q, k, v, log_alpha, beta, cu_seqlens, S0, dO, dS_T=None, *, want_dS0: bool = True,
                     cu_seqlens_host: Optional[Sequence[int]] = None, workspace=None, stream=None):
    """Gradients of sum <dO, o> + <dS_T, S_T> through ``prefill`` (64-token
    chunks, no stages).  Arguments as for ``prefill``; dO like o, dS_T like
    S_T (or None).  Returns a dict: dq, dk, dv (the io dtype), dlog_alpha
    (fp32, shaped like log_alpha; None without a gate), dbeta (fp32) and dS0
    (fp32, None when ``want_dS0`` is False).  The backward workspace is
    cached per (device, stream) like the prefill's."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3 or cu_seqlens.dim() != 1:
        raise ValueError("q, k, v must be [T, H, d] and cu_seqlens [N+1]")
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    dt = _dtype_code(q)
    dev = q.device
    if k.dtype != q.dtype or v.dtype != q.dtype or dO.dtype != q.dtype:
        raise TypeError("q, k, v and dO must share a dtype")
    gate = _gate(log_alpha, (T, H))
    la_shape = _la_shape(gate, (T, H), dk)
    s = _stream(stream)
    desc, keep = make_desc(N, T, H, dk, dv, 64, dt, cu_seqlens_host, 0, gate)
    need = int(lib.kda_prefill_backward_workspace_size(ctypes.byref(desc)))
    if need == 0:
        st = lib.kda_prefill_backward(ctypes.byref(desc), *([None] * 16), 0, None)
        raise KdaError(st if st != KDA_OK else KDA_ERR_INVALID_ARGUMENT, "kda_prefill_backward_workspace_size")
    out = {"dq": torch.empty((T, H, dk), dtype=q.dtype, device=dev),
           "dk": torch.empty((T, H, dk), dtype=q.dtype, device=dev),
           "dv": torch.empty((T, H, dv), dtype=q.dtype, device=dev),
           "dlog_alpha": None if la_shape is None else torch.empty(la_shape, dtype=torch.float32, device=dev),
           "dbeta": torch.empty((T, H), dtype=torch.float32, device=dev),
           "dS0": torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None}
    ptrs = (_dev_ptr(q, "q", None, (T, H, dk), dev), _dev_ptr(k, "k", None, (T, H, dk), dev),
            _dev_ptr(v, "v", None, (T, H, dv), dev),
            _dev_ptr(log_alpha, "log_alpha", torch.float32, la_shape, dev),
            _dev_ptr(beta, "beta", torch.float32, (T, H), dev),
            _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev),
            _dev_ptr(S0, "S0", torch.float32, (N, H, dk, dv), dev),
            _dev_ptr(dO, "dO", q.dtype, (T, H, dv), dev),
            _dev_ptr(dS_T, "dS_T", torch.float32, (N, H, dk, dv), dev),
            _dev_ptr(out["dq"], "dq"), _dev_ptr(out["dk"], "dk"), _dev_ptr(out["dv"], "dv"),
            _dev_ptr(out["dlog_alpha"], "dlog_alpha"), _dev_ptr(out["dbeta"], "dbeta"),
            _dev_ptr(out["dS0"], "dS0"))
    if workspace is None:
        workspace = _workspace(dev, s, need, "backward")
    wptr = _dev_ptr(workspace, "workspace", None, None, dev)
    st = lib.kda_prefill_backward(ctypes.byref(desc), *ptrs, wptr, workspace.numel() * workspace.element_size(),
                                  s.cuda_stream)
    del keep
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill_backward")
    return out


def set_wait_limit(polls: int) -> int:
    """Test hook: see kda_prefill_set_wait_limit in include/kda.h."""
    return int(load_library().kda_prefill_set_wait_limit(int(polls)))


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, stream=None, **stage_kw):
    """One KDA step for B requests: q, k [B, H, dk]; v [B, H, dv]; log_alpha
    [B, H, dk] fp32 ([B, H] for one rate per head, None without a gate);
    beta [B, H] fp32; S [B, H, dk, dv] fp32 updated in place.  Returns o
    [B, H, dv].  Stage keywords as for ``prefill`` (out_gate [B, H, dv])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    gate = _gate(log_alpha, (B, H))
    stg = _stages((B, H, dv), q.dtype, dev, **stage_kw)
    st = lib.kda_decode_step(B, H, dk, dv, dt, gate, ctypes.pointer(stg) if stg is not None else None,
                             _dev_ptr(q, "q", None, (B, H, dk), dev),
                             _dev_ptr(k, "k", None, (B, H, dk), dev), _dev_ptr(v, "v", None, (B, H, dv), dev),
                             _dev_ptr(log_alpha, "log_alpha", torch.float32, _la_shape(gate, (B, H), dk), dev),
                             _dev_ptr(beta, "beta", torch.float32, (B, H), dev),
                             _dev_ptr(S, "S", torch.float32, (B, H, dk, dv), dev),
                             _dev_ptr(o, "o", q.dtype, (B, H, dv), dev), _stream(stream).cuda_stream)
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o
