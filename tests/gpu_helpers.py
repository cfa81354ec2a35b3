"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI binding, run the oracle on the same values, compare."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import synth

TOL = {"bf16": 1e-2, "f32": 1e-4}


def torch_mod():
    import torch
    return torch


def have_gpu() -> bool:
    try:
        return torch_mod().cuda.is_available()
    except Exception:
        return False


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str = "f32"):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def gpu_prefill(w: synth.PrefillInputs, chunk: int = None, S0=None, in_place: bool = False, host_offsets=True,
                one_stream: bool = False, want_state: bool = True, report: dict = None, max_workspace_bytes=None,
                **stage_kw):
    """Run libkda prefill on the inputs; returns (o, S_T) as float64 numpy
    (S_T None when want_state is False).  When ``report`` is a dict, its key
    "recovered" is set to whether the call's overlapped schedule recovered."""
    import gated_delta_rule_33_amd as kda
    torch = torch_mod()
    dt = w.io_dtype
    q, k, v = dev(w.q, dt), dev(w.k, dt), dev(w.v, dt)
    la = dev(w.log_alpha) if w.log_alpha is not None else None
    b = dev(w.beta)
    cu = dev(w.cu_seqlens)
    s0 = S0 if S0 is not None else w.S0
    s0d = dev(s0) if s0 is not None else None
    kw = {}
    if in_place:
        assert s0d is not None
        kw["S_T"] = s0d
    host_cu = w.cu_seqlens.tolist() if host_offsets else None
    o, ST = kda.prefill(q, k, v, la, b, cu, s0d, chunk=chunk or w.chunk, cu_seqlens_host=host_cu,
                        one_stream=one_stream, want_state=want_state, max_workspace_bytes=max_workspace_bytes,
                        **kw, **stage_kw)
    torch.cuda.synchronize()
    if report is not None:
        report["recovered"] = kda.prefill_recovered(q, v, cu, chunk=chunk or w.chunk, cu_seqlens_host=host_cu,
                                                    one_stream=one_stream, max_workspace_bytes=max_workspace_bytes)
    return host(o), (host(ST) if ST is not None else None)


def oracle_prefill(w: synth.PrefillInputs, S0=None, heads=None, threads: int = 0):
    """fp64 oracle on the same values; optionally on a subset of heads."""
    s0 = S0 if S0 is not None else w.S0
    la = w.log_alpha_channels()
    if heads is None:
        return oracle.prefill(w.q, w.k, w.v, la, w.beta, w.cu_seqlens, s0, threads=threads)
    hs = list(heads)
    return oracle.prefill(w.q[:, hs], w.k[:, hs], w.v[:, hs], la[:, hs], w.beta[:, hs], w.cu_seqlens,
                          None if s0 is None else s0[:, hs], threads=threads)


def check(name: str, got: np.ndarray, ref: np.ndarray, tol: float):
    e = rel_err(got, ref)
    log("  %-28s rel_err %.3e (tol %.0e) max|ref| %.3e" % (name, e, tol, float(np.max(np.abs(ref))) if ref.size else 0))
    assert np.all(np.isfinite(got)), name + ": non-finite output"
    assert e <= tol, "%s: rel err %.3e > %.0e" % (name, e, tol)
    return e


def assert_not_recovered(report: dict):
    """The call's overlapped schedule ran to the end without falling back to
    its recovery launches (the two streams ran side by side)."""
    log("  overlapped schedule recovered: %s" % report["recovered"])
    assert report["recovered"] is False, "the state pass stopped waiting for a prep segment"
