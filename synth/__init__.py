"""Seeded synthetic inputs for the KDA operator.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and shapes them into operator inputs; it contains none
of the operator's own arithmetic (no recurrence, no gate cumsum, no chunk
math), so both the oracle and the HIP path can consume what it produces.

Recipe (numpy ``Generator(PCG64(...))``, every draw float32):

* tokens are drawn in blocks of 4096; block ``j`` of a workload with seed
  ``s`` uses its own stream ``PCG64([s, j])`` and draws, in this order, q, k,
  v ([4096, H, d] each), z_beta ([4096, H]) and z_alpha ([4096, H, dk]).
  Blocks are independent, so they are generated on several threads and the
  result does not depend on the thread count;
* sequence lengths (packed-varlen workload) come first, from ``PCG64([s])``;
  the long-memory channel mask from ``PCG64([s, 2**20])``; S0 from
  ``PCG64([s, 2**21])``;
* q and k are L2-normalised per (token, head) over the key dimension in
  float32: x / max(||x||, 1e-6);
* beta = sigmoid(z_beta);
* log_alpha = -softplus(z_alpha) = -(max(z, 0) + log1p(exp(-|z|))), float32;
* bf16 tensors are rounded from float32 to nearest-even once, here, and both
  sides read those same rounded values.

The five standard workloads (``WORKLOADS``) mirror the operator's five
reference shapes: a tiny fp32 case, a 4 x 4096 batch, one 131072-token
sequence with 5% long-memory channels, a 64-sequence packed batch with
log-uniform lengths and a random initial state, and a batched decode.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BLOCK = 4096
_MASK_STREAM = 1 << 20
_S0_STREAM = 1 << 21
_COT_STREAM = 1 << 22


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# bf16 helpers (bit-level; numpy has no bfloat16)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest-even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Expand bfloat16 bit patterns to the float32 values they denote."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (returned as float32)."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# element-wise input shaping
# --------------------------------------------------------------------------

def l2norm_f32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def sigmoid_f32(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32, copy=False)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-z))).astype(np.float32)


def neg_softplus_f32(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32, copy=False)
    return (-(np.maximum(z, np.float32(0.0)) + np.log1p(np.exp(-np.abs(z))))).astype(np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillInputs:
    """Host-side prefill inputs.  Float arrays hold the exact values both sides
    use (bf16-rounded where ``io_dtype == 'bf16'``)."""
    q: np.ndarray            # [T_tot, H, dk] float32
    k: np.ndarray            # [T_tot, H, dk] float32
    v: np.ndarray            # [T_tot, H, dv] float32
    log_alpha: Optional[np.ndarray]  # [T_tot, H, dk] (gate "channel"), [T_tot, H] ("scalar") or None ("none")
    beta: np.ndarray         # [T_tot, H]     float32
    cu_seqlens: np.ndarray   # [N + 1]        int32
    S0: Optional[np.ndarray]  # [N, H, dk, dv] float32 or None
    io_dtype: str            # 'f32' or 'bf16'
    chunk: int = 64
    gate: str = "channel"    # forget-gate form: 'channel' (KDA), 'scalar' (GDN) or 'none' (DeltaNet)

    def log_alpha_channels(self) -> np.ndarray:
        """log_alpha as one rate per key channel [T_tot, H, dk] (the scalar
        gate repeated over the channels, zeros without a gate)."""
        T, H, dk = self.q.shape
        if self.gate == "channel":
            return self.log_alpha
        if self.gate == "scalar":
            return np.ascontiguousarray(np.broadcast_to(self.log_alpha[:, :, None], (T, H, dk)))
        return np.zeros((T, H, dk), np.float32)

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])


def make_prefill(lengths, H: int, dk: int, dv: int, io_dtype: str, seed: int,
                 S0_std: Optional[float] = None, long_memory_frac: float = 0.0,
                 chunk: int = 64, lengths_from_rng=None, gate: str = "channel") -> PrefillInputs:
    """Generic seeded prefill inputs.

    ``gate`` selects the forget-gate form: "channel" draws z_alpha per key
    channel [.., H, dk], "scalar" one per head [.., H] (the last draw of a
    block, so the other tensors are the same as for "channel"), "none" draws
    no gate (log_alpha is None).

    lengths: list of sequence lengths, or None when ``lengths_from_rng`` (a
    callable taking the Generator) draws them first.  ``long_memory_frac``
    picks round(frac * dk) key channels per head whose forget gate stays
    near 1: log_alpha = -1e-5 * softplus(z) on those channels for every token.
    """
    if lengths_from_rng is not None:
        lengths = lengths_from_rng(np.random.Generator(np.random.PCG64([seed])))
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = np.empty((T, H, dk), np.float32)
    k = np.empty((T, H, dk), np.float32)
    v = np.empty((T, H, dv), np.float32)
    beta = np.empty((T, H), np.float32)
    if gate not in ("channel", "scalar", "none"):
        raise ValueError(gate)
    la = {"channel": lambda: np.empty((T, H, dk), np.float32), "scalar": lambda: np.empty((T, H), np.float32),
          "none": lambda: None}[gate]()

    def fill(j: int):
        a, b = j * BLOCK, min(T, (j + 1) * BLOCK)
        n = b - a
        rng = np.random.Generator(np.random.PCG64([seed, j]))
        qb = rng.standard_normal((BLOCK, H, dk), dtype=np.float32)[:n]
        kb = rng.standard_normal((BLOCK, H, dk), dtype=np.float32)[:n]
        vb = rng.standard_normal((BLOCK, H, dv), dtype=np.float32)[:n]
        zb = rng.standard_normal((BLOCK, H), dtype=np.float32)[:n]
        if gate != "none":
            za = rng.standard_normal((BLOCK, H, dk) if gate == "channel" else (BLOCK, H), dtype=np.float32)[:n]
            la[a:b] = neg_softplus_f32(za)
        qb, kb = l2norm_f32(qb), l2norm_f32(kb)
        if io_dtype == "bf16":
            qb, kb, vb = bf16_round(qb), bf16_round(kb), bf16_round(vb)
        q[a:b], k[a:b], v[a:b] = qb, kb, vb
        beta[a:b] = sigmoid_f32(zb)

    if io_dtype not in ("bf16", "f32"):
        raise ValueError(io_dtype)
    nblk = (T + BLOCK - 1) // BLOCK
    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(nblk)))
    if long_memory_frac > 0.0 and gate == "channel":
        nlm = int(round(long_memory_frac * dk))
        mrng = np.random.Generator(np.random.PCG64([seed, _MASK_STREAM]))
        for h in range(H):
            ch = mrng.choice(dk, size=nlm, replace=False)
            la[:, h, ch] = (np.float32(1e-5) * la[:, h, ch]).astype(np.float32)
    S0 = None
    if S0_std is not None:
        srng = np.random.Generator(np.random.PCG64([seed, _S0_STREAM]))
        S0 = (srng.standard_normal((len(lengths), H, dk, dv), dtype=np.float32) * np.float32(S0_std)).astype(np.float32)
    return PrefillInputs(q=q, k=k, v=v, log_alpha=la, beta=beta, cu_seqlens=cu, S0=S0,
                         io_dtype=io_dtype, chunk=chunk, gate=gate)


@dataclasses.dataclass
class StageInputs:
    """Inputs of the input and output stages: raw q and k (the workload's
    unit vectors scaled per (token, head) by a factor in [0.25, 4), then
    rounded to the io dtype), the gate projection's output z (the standard
    normal draw whose -softplus the workload's log_alpha is; same shape as
    the gate), the output gate's pre-activation z_o ~ N(0, 1) shaped like o
    (rounded to the io dtype) and an RMSNorm weight ~ U[0.5, 1.5) per value
    channel."""
    q_raw: np.ndarray
    k_raw: np.ndarray
    z_gate: Optional[np.ndarray]
    z_out: np.ndarray
    norm_weight: np.ndarray


def make_stage_inputs(w: "PrefillInputs", seed: int, z_gate=None) -> StageInputs:
    """Stage inputs for a prefill (or decode step) input set ``w``; ``z_gate``
    is the gate projection output when already known (else drawn)."""
    rng = np.random.Generator(np.random.PCG64([seed, _S0_STREAM + 1]))
    T, H, dk = w.q.shape
    dv = w.v.shape[-1]
    rnd = bf16_round if w.io_dtype == "bf16" else (lambda x: x.astype(np.float32))
    sq = rng.uniform(0.25, 4.0, size=(T, H, 1)).astype(np.float32)
    sk = rng.uniform(0.25, 4.0, size=(T, H, 1)).astype(np.float32)
    q_raw, k_raw = rnd(w.q * sq), rnd(w.k * sk)
    if z_gate is None and w.log_alpha is not None:
        z_gate = rng.standard_normal(w.log_alpha.shape, dtype=np.float32)
    z_out = rnd(rng.standard_normal((T, H, dv), dtype=np.float32))
    nw = rng.uniform(0.5, 1.5, size=dv).astype(np.float32)
    return StageInputs(q_raw, k_raw, z_gate, z_out, nw)


@dataclasses.dataclass
class Cotangents:
    """Cotangents for the backward pass: dO ~ N(0, 1) shaped like o (rounded
    to the io dtype) and dS_T ~ N(0, dS_T_std^2) shaped like S_T, float32, or
    None."""
    dO: np.ndarray
    dS_T: Optional[np.ndarray]


def make_cotangents(w: "PrefillInputs", seed: int, dS_T_std: Optional[float] = 1.0) -> Cotangents:
    """Seeded cotangents for the prefill input set ``w``: drawn in blocks of
    BLOCK tokens from ``PCG64([seed, 2**22, j])`` (dO), then dS_T from
    ``PCG64([seed, 2**22 + 1])``."""
    T, H, dk = w.q.shape
    dv = w.v.shape[-1]
    N = len(w.cu_seqlens) - 1
    rnd = bf16_round if w.io_dtype == "bf16" else (lambda x: x.astype(np.float32))
    dO = np.empty((T, H, dv), np.float32)

    def fill(j: int):
        a, b = j * BLOCK, min(T, (j + 1) * BLOCK)
        rng = np.random.Generator(np.random.PCG64([seed, _COT_STREAM, j]))
        dO[a:b] = rnd(rng.standard_normal((BLOCK, H, dv), dtype=np.float32)[:b - a])

    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range((T + BLOCK - 1) // BLOCK)))
    dST = None
    if dS_T_std is not None:
        rng = np.random.Generator(np.random.PCG64([seed, _COT_STREAM + 1]))
        dST = (rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(dS_T_std)).astype(np.float32)
    return Cotangents(dO, dST)


def _loguniform_lengths(n: int, lo: int, hi: int):
    def draw(rng):
        u = rng.uniform(math.log(lo), math.log(hi), size=n)
        return [int(math.floor(math.exp(x))) for x in u]
    return draw


# Workload descriptors.  seed = 1000 + workload index.
WORKLOADS = {
    "tiny_f32": dict(index=0, kind="prefill", lengths=[256], H=2, dk=64, dv=64, io_dtype="f32"),
    "batch4x4096_bf16": dict(index=1, kind="prefill", lengths=[4096] * 4, H=16, dk=128, dv=128, io_dtype="bf16"),
    "long131072_bf16": dict(index=2, kind="prefill", lengths=[131072], H=32, dk=128, dv=128, io_dtype="bf16",
                            long_memory_frac=0.05),
    "varlen64_bf16": dict(index=3, kind="prefill", lengths=None, H=32, dk=128, dv=128, io_dtype="bf16",
                          S0_std=0.02, varlen=(64, 128, 32768)),
    "decode256x32_bf16": dict(index=4, kind="decode", B=256, H=32, dk=128, dv=128, io_dtype="bf16",
                              steps=1024, S0_std=0.02),
    # the 131072-token shape with the scalar gate (Gated DeltaNet) and without a gate (DeltaNet)
    "long131072_bf16_gdn": dict(index=5, kind="prefill", lengths=[131072], H=32, dk=128, dv=128, io_dtype="bf16",
                                gate="scalar"),
    "long131072_bf16_deltanet": dict(index=6, kind="prefill", lengths=[131072], H=32, dk=128, dv=128,
                                     io_dtype="bf16", gate="none"),
}


def workload_prefill(name: str, lengths_override=None, H_override=None) -> PrefillInputs:
    """Inputs of a standard prefill workload (optionally with fewer heads or
    other lengths, keeping the same distributions and seed)."""
    w = WORKLOADS[name]
    assert w["kind"] == "prefill"
    seed = 1000 + w["index"]
    H = H_override or w["H"]
    draw = None
    lengths = lengths_override if lengths_override is not None else w["lengths"]
    if lengths is None:
        n, lo, hi = w["varlen"]
        draw = _loguniform_lengths(n, lo, hi)
    return make_prefill(lengths, H, w["dk"], w["dv"], w["io_dtype"], seed,
                        S0_std=w.get("S0_std"), long_memory_frac=w.get("long_memory_frac", 0.0),
                        lengths_from_rng=draw, gate=w.get("gate", "channel"))


@dataclasses.dataclass
class DecodeStepInputs:
    q: np.ndarray          # [B, H, dk] float32 (bf16-rounded for bf16 io)
    k: np.ndarray
    v: np.ndarray          # [B, H, dv]
    log_alpha: Optional[np.ndarray]  # [B, H, dk] float32; [B, H] for the scalar gate; None without a gate
    beta: np.ndarray       # [B, H]     float32


def make_decode_state(B: int, H: int, dk: int, dv: int, std: float, seed: int) -> np.ndarray:
    """Initial decode states S ~ N(0, std^2), float32 [B, H, dk, dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_decode_step(B: int, H: int, dk: int, dv: int, io_dtype: str, seed: int, step: int,
                     gate: str = "channel") -> DecodeStepInputs:
    """Fresh per-token decode inputs for step ``step`` (its own PCG64 stream,
    so any step can be regenerated without drawing the earlier ones).
    ``gate``: "channel" (log_alpha [B, H, dk]), "scalar" ([B, H]) or "none"."""
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    q = l2norm_f32(rng.standard_normal((B, H, dk), dtype=np.float32))
    k = l2norm_f32(rng.standard_normal((B, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, dv), dtype=np.float32)
    beta = sigmoid_f32(rng.standard_normal((B, H), dtype=np.float32))
    la = None
    if gate == "channel":
        la = neg_softplus_f32(rng.standard_normal((B, H, dk), dtype=np.float32))
    elif gate == "scalar":
        la = neg_softplus_f32(rng.standard_normal((B, H), dtype=np.float32))
    elif gate != "none":
        raise ValueError(gate)
    if io_dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return DecodeStepInputs(q=q, k=k, v=v, log_alpha=la, beta=beta)
