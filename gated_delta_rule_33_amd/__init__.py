"""Python binding for libkda, the gfx950 Kimi Delta Attention library.

Argument marshalling only: every step of the operator runs in the HIP
kernels of ``libkda.so`` behind the C ABI declared in ``include/kda.h``.
PyTorch supplies device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library is missing, or a tensor is not on a GPU,
these functions raise.

    o, S_T = prefill(q, k, v, log_alpha, beta, cu_seqlens, S0=None)
    o      = decode_step(q, k, v, log_alpha, beta, S)      # S updated in place
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

EXPORTED = ("kda_prefill", "kda_prefill_workspace_size", "kda_decode_step", "kda_status_string", "kda_version")


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


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
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                        vp, vp, vp, vp, vp, vp, vp, vp]
        if path == LIB_PATH:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().kda_version())


def make_desc(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int, chunk: int, io_dtype: int,
              cu_seqlens_host: Optional[Sequence[int]] = None):
    """Build a kda_prefill_desc.  Returns (desc, keepalive) -- keep the second
    value alive while the desc is used (it owns the host offsets)."""
    keep = None
    ptr = ctypes.POINTER(ctypes.c_int32)()
    if cu_seqlens_host is not None:
        keep = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
        ptr = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    d = PrefillDesc(int(num_seqs), int(total_tokens), int(num_heads), int(dk), int(dv), int(chunk), int(io_dtype),
                    ptr)
    return d, keep


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


def _dev_ptr(t, name: str, dtype=None) -> int:
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_ws_cache = {}


def prefill(q, k, v, log_alpha, beta, cu_seqlens, S0=None, *, chunk: int = 64, o=None, S_T=None,
            cu_seqlens_host: Optional[Sequence[int]] = None, workspace=None, stream=None, want_state: bool = True):
    """KDA chunked prefill over a packed batch.

    q, k: [T, H, dk]; v: [T, H, dv] (bf16 or fp32, same dtype); log_alpha: [T, H, dk]
    fp32; beta: [T, H] fp32; cu_seqlens: [N+1] int32 (GPU); S0: [N, H, dk, dv] fp32 or
    None.  Returns (o, S_T); S_T is None when ``want_state`` is False.
    ``S_T`` may be passed as ``S0`` to update the state in place.
    """
    torch = _torch()
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    desc, keep = make_desc(N, T, H, dk, dv, chunk, dt, cu_seqlens_host)
    need = int(lib.kda_prefill_workspace_size(ctypes.byref(desc)))
    if need == 0:
        st = lib.kda_prefill(ctypes.byref(desc), *([None] * 10), 0, None)
        raise KdaError(st if st != KDA_OK else KDA_ERR_INVALID_ARGUMENT, "kda_prefill_workspace_size")
    if workspace is None:
        key = (q.device, need)
        workspace = _ws_cache.get(key)
        if workspace is None:
            _ws_cache.clear()
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _ws_cache[key] = workspace
    st = lib.kda_prefill(ctypes.byref(desc),
                         _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                         _dev_ptr(log_alpha, "log_alpha", torch.float32), _dev_ptr(beta, "beta", torch.float32),
                         _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32),
                         _dev_ptr(S0, "S0", torch.float32) if S0 is not None else None,
                         _dev_ptr(o, "o", q.dtype),
                         _dev_ptr(S_T, "S_T", torch.float32) if S_T is not None else None,
                         _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                         _stream_ptr(stream))
    del keep
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill")
    return o, S_T


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, stream=None):
    """One KDA step for B requests: q, k [B, H, dk]; v [B, H, dv]; log_alpha
    [B, H, dk] fp32; beta [B, H] fp32; S [B, H, dk, dv] fp32 updated in place.
    Returns o [B, H, dv]."""
    torch = _torch()
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    st = lib.kda_decode_step(B, H, dk, dv, dt, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                             _dev_ptr(log_alpha, "log_alpha", torch.float32), _dev_ptr(beta, "beta", torch.float32),
                             _dev_ptr(S, "S", torch.float32), _dev_ptr(o, "o", q.dtype), _stream_ptr(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o
