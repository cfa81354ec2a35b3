"""fp64 definitions of the input and output stages around the KDA recurrence.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests, the
package smoke check and the benchmark's CPU-baseline leg use it.

The "Kimi Linear" deep-read report (zako-mio knowledge base), section 3.2,
places the recurrence between an input side -- q, k and v pass a short
convolution with Swish, q and k are then L2-normalised (to keep the
transition's eigenvalues stable), and the forget gate comes out of a
low-rank projection -- and an output side -- a head-wise RMSNorm and a
low-rank, data-dependent sigmoid output gate.  The projections (and the
short convolution) produce the inputs of these stages and are outside them.
Readings where the page is silent:

* L2 normalisation is over the key dimension of each (token, head) vector:
  x / max(||x||, eps).
* The gate activation is log alpha = -softplus(z) of the projection output
  z, the form the synthetic workloads already use for their gates.
* RMSNorm is over the value dimension of each (token, head) output, with one
  weight per value channel shared by the heads: o / sqrt(mean(o^2) + eps) * w.
* The output gate multiplies after the norm: y = RMSNorm(o) * sigmoid(z_o).
"""
from __future__ import annotations

import numpy as np

import oracle


def l2norm(x, eps: float):
    """x / max(||x||_2, eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def gate_log_alpha(z):
    """log alpha = -softplus(z) = -log(1 + e^z), written without overflow as
    -(max(z, 0) + log1p(e^{-|z|}))."""
    z = np.asarray(z, dtype=np.float64)
    return -(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))


def output_stage(o, out_gate=None, norm_weight=None, eps: float = 1e-6):
    """Head-wise RMSNorm over the last axis (when a weight is given), then
    the sigmoid output gate (when its pre-activation is given)."""
    y = np.asarray(o, dtype=np.float64)
    if norm_weight is not None:
        ms = np.mean(y * y, axis=-1, keepdims=True)
        y = y / np.sqrt(ms + eps) * np.asarray(norm_weight, dtype=np.float64)
    if out_gate is not None:
        y = y * sigmoid(out_gate)
    return y


def _gate_channels(la, shape):
    """Per-key-channel log alpha from a per-channel, per-head or absent gate."""
    T, H, dk = shape
    if la is None:
        return np.zeros((T, H, dk))
    la = np.asarray(la, dtype=np.float64)
    return la if la.ndim == 3 else np.broadcast_to(la[:, :, None], (T, H, dk))


def prefill_staged(q, k, v, gate, beta, cu_seqlens, S0=None, *, l2norm_qk=False, l2norm_eps=1e-6,
                   gate_softplus=False, out_gate=None, norm_weight=None, norm_eps=1e-6, threads: int = 0):
    """Input stage, the recurrence (the C oracle), output stage.  ``gate`` is
    log alpha, or the projection output z when ``gate_softplus``; it may be
    [T, H, dk], [T, H] (one rate per head) or None (no gate)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if l2norm_qk:
        q, k = l2norm(q, l2norm_eps), l2norm(k, l2norm_eps)
    if gate is not None and gate_softplus:
        gate = gate_log_alpha(gate)
    la = _gate_channels(gate, q.shape)
    o, ST = oracle.prefill(q, k, v, la, beta, cu_seqlens, S0, threads=threads)
    return output_stage(o, out_gate, norm_weight, norm_eps), ST


def decode_staged(q, k, v, gate, beta, S, *, l2norm_qk=False, l2norm_eps=1e-6, gate_softplus=False,
                  out_gate=None, norm_weight=None, norm_eps=1e-6, inplace: bool = False):
    """One decode step with the same stages; returns (y, S_new)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if l2norm_qk:
        q, k = l2norm(q, l2norm_eps), l2norm(k, l2norm_eps)
    if gate is not None and gate_softplus:
        gate = gate_log_alpha(gate)
    la = _gate_channels(gate, q.shape)
    o, S = oracle.decode_step(q, k, v, la, beta, S, inplace=inplace)
    return output_stage(o, out_gate, norm_weight, norm_eps), S
