"""fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it,
and it imports nothing from the product path.

Two independent definitions live here:

* ``prefill`` / ``decode_step`` -- the sequential recurrence, in plain C
  (``kda_oracle.c``), all arithmetic in double precision.  It follows the KDA
  update of the "Kimi Linear" deep-read report (zako-mio knowledge base),
  section 2.3 (per-channel diagonal forget gate; forget, erase along k, write
  beta k v^T, in that order) and the zhaixingw.cn explainer's KDA section
  (one forget rate per key channel).
* ``backward`` -- the reverse-mode derivative of that recurrence (same C
  file), for the loss sum_t <dO_t, o_t> + <dS_T, S_T>: the chain rule taken
  through the forward loop's lines in reverse order, token by token.
* ``brute.unified_form`` -- the unified recurrent form of the report's
  section 2.4 / 6.1 (o_t as a sum over j of q_t^T times the product of the
  transition matrices A_i times k_j v_j^T), evaluated with explicit dk x dk
  matrices in numpy.  It is a different computation used to pin the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/_build/libkda_oracle.so``."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """ctypes handle for a compiled copy of ``kda_oracle.c`` at ``path``."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [
        ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_decode_step.restype = ctypes.c_int
    lib.kda_oracle_decode_step.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_backward.restype = ctypes.c_int
    lib.kda_oracle_backward.argtypes = [
        ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = load_library(_LIB_PATH)
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, log_alpha, beta, cu_seqlens, S0=None, threads: int = 0, return_threads: bool = False,
            lib=None):
    """Sequential fp64 recurrence over a packed batch.

    q, k, log_alpha: [T_tot, H, dk]; v: [T_tot, H, dv]; beta: [T_tot, H];
    cu_seqlens: [N+1] int offsets; S0: [N, H, dk, dv] or None (zero).
    Returns (o [T_tot, H, dv], S_T [N, H, dk, dv]) as float64 arrays.
    """
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T_tot, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T_tot, H, dk) and la.shape == (T_tot, H, dk)
    assert v.shape == (T_tot, H, dv) and b.shape == (T_tot, H)
    assert int(cu[-1]) == T_tot
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((T_tot, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    lib = lib or _load()
    used = lib.kda_oracle_prefill(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), H, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b),
        _ptr(s0) if s0 is not None else ctypes.POINTER(ctypes.c_double)(),
        _ptr(o), _ptr(ST), int(threads))
    if used < 0:
        raise ValueError("oracle rejected its arguments")
    return (o, ST, used) if return_threads else (o, ST)


def decode_step(q, k, v, log_alpha, beta, S, threads: int = 0, lib=None, inplace: bool = False):
    """One recurrence step for B independent states.

    q, k, log_alpha: [B, H, dk]; v: [B, H, dv]; beta: [B, H]; S: [B, H, dk, dv].
    Returns (o [B, H, dv], S_new [B, H, dk, dv]); the input S is not modified,
    unless ``inplace`` is set and S is a C-contiguous float64 array, which is
    then updated and returned as S_new.
    """
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    if not (inplace and isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]):
        S = np.array(S, dtype=np.float64, copy=True, order="C")
    B, H, dk = q.shape
    dv = v.shape[2]
    assert S.shape == (B, H, dk, dv)
    o = np.zeros((B, H, dv), dtype=np.float64)
    used = (lib or _load()).kda_oracle_decode_step(B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b),
                                          _ptr(S), _ptr(o), int(threads))
    if used < 0:
        raise ValueError("oracle rejected its arguments")
    return o, S


def backward(q, k, v, log_alpha, beta, cu_seqlens, S0, dO, dS_T=None, threads: int = 0, lib=None):
    """Gradients of L = sum <dO, o> + <dS_T, S_T> through the recurrence.

    Shapes as for ``prefill`` (log_alpha per channel, [T_tot, H, dk]); dO like
    o, dS_T like S_T (None = zero).  Returns a dict with dq, dk, dv,
    dlog_alpha, dbeta ([T_tot, H]) and dS0 ([N, H, dk, dv]), float64.
    """
    q, k, v, la, b, dO = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta), _f64(dO)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T_tot, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T_tot, H, dk) and la.shape == (T_tot, H, dk)
    assert v.shape == (T_tot, H, dv) and b.shape == (T_tot, H) and dO.shape == (T_tot, H, dv)
    assert int(cu[-1]) == T_tot
    s0 = None if S0 is None else _f64(S0)
    dst = None if dS_T is None else _f64(dS_T)
    for x in (s0, dst):
        if x is not None:
            assert x.shape == (N, H, dk, dv)
    out = {"dq": np.zeros((T_tot, H, dk)), "dk": np.zeros((T_tot, H, dk)), "dv": np.zeros((T_tot, H, dv)),
           "dlog_alpha": np.zeros((T_tot, H, dk)), "dbeta": np.zeros((T_tot, H)),
           "dS0": np.zeros((N, H, dk, dv))}
    null = ctypes.POINTER(ctypes.c_double)()
    used = (lib or _load()).kda_oracle_backward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), H, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(s0) if s0 is not None else null,
        _ptr(dO), _ptr(dst) if dst is not None else null,
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
        _ptr(out["dS0"]), int(threads))
    if used < 0:
        raise ValueError("oracle rejected its arguments")
    return out
