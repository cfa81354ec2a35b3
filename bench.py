"""Benchmark for libkda on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one kda_prefill call over the whole long-sequence workload: one
sequence of 131072 tokens, 32 heads, dk = dv = 128, bf16 q/k/v/o, fp32
log_alpha/beta/state, chunk 64, 5% long-memory key channels; it returns o and
the final state.  Inputs are resident in HBM before timing starts.  The
decode workload (256 requests x 32 heads, fp32 128x128 states updated in
place for 1024 tokens) is timed in the same run and reported under "decode";
the call rates of the 4 x 4096-token batch and of the 64-sequence varlen
workload follow under "prefill_other" (skip with --no-other), and the
backward pass (kda_prefill_backward) on the 4 x 4096-token batch, checked
against the oracle's backward, and on the long workload under "backward"
(skip with --no-backward).  "prefill_other" also times the long and varlen
workloads under the bounded-workspace schedule inside 1 GiB.

Prints ONE JSON line.  `value` is prefill tokens/s.  Each roofline block
prices the operator's algorithmic bytes per launch against MI355X's 8 TB/s
HBM peak, using HIP-event durations taken on the stream the kernels run on.
The fp64 oracle is timed on the host CPU ("cpu_baseline"): for prefill over
the whole sequence and every head of the last timed call, whose outputs it
also checks element by element ("parity"); for decode over the first steps
of the decode workload ("decode.cpu_baseline").  After the timed loop the
prefill call's recovery flag is read: if the overlapped schedule had to fall
back (its two streams did not run side by side), the timing is not that
schedule's and the script exits with status 3.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# The source files that define each measured kernel sequence (with the
# shared device header): hardware-counter traffic is reported only while
# these are byte-identical to the ones it was measured on.
TRAFFIC_SOURCES = {"prefill": ("kda_prefill.hip", "kda_device.h"), "decode": ("kda_decode.hip", "kda_device.h"),
                   "backward": ("kda_backward.hip", "kda_prefill.hip", "kda_device.h")}


def source_digest(key: str) -> str:
    """sha256 over the HIP sources of the kernels behind ``key``."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_33_amd", "csrc")
    for f in TRAFFIC_SOURCES[key.split("_")[0]]:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except Exception:
        return None
    r = rec.get(key)
    if not r or r.get("source_digest") != source_digest(key):
        return None
    return r.get("bytes_per_launch")


GATE_WIDTH = {"channel": None, "scalar": 1, "none": 0}  # log_alpha floats per (token, head); None = dk


def prefill_algorithmic(T_tok: int, N: int, H: int, dk: int, dv: int, es: int, C: int, with_s0: bool,
                        gate: str = "channel"):
    """Compulsory bytes and algorithmic flops of one prefill call.
    Bytes: read q, k (dk each), v (dv) in the io dtype, log_alpha (dk fp32 per
    token-head; 1 for the scalar gate, none without a gate), beta (fp32);
    write o (dv, io dtype); write S_T (and read S0 when given).
    Flops per token-head: 2 [ (C/2)(3 dk + 2 dv) + 3 dk dv ] -- the two gated
    intra-chunk matrices, the WY factors and the three state contractions,
    triangular products counted at half.  The dense-tile count (as the
    matrix cores execute the triangular products, at full size) is
    2 [ C (3 dk + 2 dv) + 3 dk dv ]."""
    th = T_tok * H
    gw = dk if GATE_WIDTH[gate] is None else GATE_WIDTH[gate]
    per_th = (2 * dk + dv) * es + gw * 4 + 4 + dv * es
    state = N * H * dk * dv * 4 * (2 if with_s0 else 1)
    flops_th = 2 * ((C // 2) * (3 * dk + 2 * dv) + 3 * dk * dv)
    return th * per_th + state, th * flops_th, per_th, flops_th


def prefill_dense_flops_th(dk: int, dv: int, C: int) -> int:
    return 2 * (C * (3 * dk + 2 * dv) + 3 * dk * dv)


def decode_algorithmic(BH: int, dk: int, dv: int, es: int, gate: str = "channel"):
    """Bytes per decode step: state read + write (fp32), q, k, v, o (io dtype),
    log_alpha (fp32: dk per state, 1 for the scalar gate, none without a
    gate), beta."""
    gw = dk if GATE_WIDTH[gate] is None else GATE_WIDTH[gate]
    per = 2 * dk * dv * 4 + (2 * dk + 2 * dv) * es + gw * 4 + 4
    return BH * per, per


def run_prefill(args, torch, kda, synth, oracle):
    wname = args.workload
    t0 = time.time()
    w = synth.workload_prefill(wname)
    log("generated %s in %.1fs: T=%d H=%d" % (wname, time.time() - t0, w.total_tokens, w.num_heads))
    bf = w.io_dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    def up(x, io=False):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.to(tdt) if io else t).cuda()

    q, k, v = up(w.q, True), up(w.k, True), up(w.v, True)
    la, b, cu = up(w.log_alpha), up(w.beta), up(w.cu_seqlens)
    S0 = up(w.S0) if w.S0 is not None else None
    T_tok, H, dk = w.q.shape
    dv = w.v.shape[2]
    N = w.num_seqs
    o = torch.empty((T_tok, H, dv), dtype=tdt, device="cuda")
    ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    host_cu = w.cu_seqlens.tolist()
    stream = torch.cuda.current_stream()

    def step():
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk,
                    one_stream=args.one_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    call_ms = [a.elapsed_time(z) for a, z in ev]
    recovered = kda.prefill_recovered(q, v, cu, chunk=w.chunk, cu_seqlens_host=host_cu, one_stream=args.one_stream)
    avg_call_s = float(np.mean(call_ms)) / 1e3
    es = 2 if bf else 4
    nbytes, nflops, per_th, flops_th = prefill_algorithmic(T_tok, N, H, dk, dv, es, w.chunk, S0 is not None)
    achieved = nbytes / avg_call_s / 1e9
    res = dict(
        wall_s=wall, ms_per_step=wall / args.steps * 1e3, tokens_per_s=T_tok * args.steps / wall,
        call_ms_mean=float(np.mean(call_ms)), call_ms_min=float(np.min(call_ms)),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic("prefill_" + wname),
                      kernel="kda_prefill (chunk_offsets + prep + scan kernels, one launch sequence)",
                      bytes_per_launch=int(nbytes), bytes_per_token_head=per_th,
                      mfma_tflops=round(nflops / avg_call_s / 1e12, 2),
                      mfma_frac=round(nflops / avg_call_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      flops_per_token_head=flops_th,
                      mfma_frac_dense_tiles=round(T_tok * H * prefill_dense_flops_th(dk, dv, w.chunk) / avg_call_s / 1e12
                                                  / MFMA_BF16_PEAK_TFLOPS, 4),
                      dense_flops_per_token_head=prefill_dense_flops_th(dk, dv, w.chunk),
                      # attainable = min(MFMA peak, HBM peak x algorithmic intensity)
                      attainable_tflops=round(min(MFMA_BF16_PEAK_TFLOPS, HBM_PEAK_GBS / 1e3 * flops_th / per_th), 1),
                      attainable_frac=round(nflops / avg_call_s / 1e12
                                            / min(MFMA_BF16_PEAK_TFLOPS, HBM_PEAK_GBS / 1e3 * flops_th / per_th), 4)),
        workload=dict(workload=wname, num_seqs=N, total_tokens=T_tok, heads=H, dk=dk, dv=dv, chunk=w.chunk,
                      io_dtype=w.io_dtype, state_dtype="f32"),
    )
    res["recovered"] = recovered
    if not args.no_cpu_baseline:
        Ts = min(args.cpu_sample_tokens, int(w.cu_seqlens[1]))  # a prefix of the first sequence
        log("cpu baseline: oracle on the first %d tokens x %d heads ..." % (Ts, H))
        t1 = time.perf_counter()
        o_ref, S_ref, used = oracle.prefill(w.q[:Ts], w.k[:Ts], w.v[:Ts], w.log_alpha[:Ts], w.beta[:Ts], [0, Ts],
                                            None if w.S0 is None else w.S0[:1], threads=args.cpu_threads,
                                            return_threads=True)
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = dict(value=round(Ts / dt, 1), unit="tokens/s", cores=int(used), kind="oracle",
                                   sample="first %d of %d tokens, all %d heads, fp64 sequential recurrence, %.1f s"
                                          % (Ts, T_tok, H, dt))
        T1 = min(2048, Ts)
        t1 = time.perf_counter()
        oracle.prefill(w.q[:T1], w.k[:T1], w.v[:T1], w.log_alpha[:T1], w.beta[:T1], [0, T1],
                       None if w.S0 is None else w.S0[:1], threads=1)
        dt1 = time.perf_counter() - t1
        res["cpu_baseline"]["single_thread"] = dict(
            value=round(T1 / dt1, 1), unit="tokens/s",
            sample="first %d tokens, all %d heads, one thread, %.1f s" % (T1, H, dt1))
        # parity of the last timed call over every element the oracle covered
        og = o[:Ts].float().cpu().numpy().astype(np.float64)
        par = dict(o_rel_err=float(np.max(np.abs(og - o_ref)) / np.max(np.abs(o_ref))), tokens=Ts, heads=H,
                   tol=1e-2 if bf else 1e-4)
        del og
        if Ts == T_tok and N == 1:
            sg = ST.cpu().numpy().astype(np.float64)
            par["S_T_rel_err"] = float(np.max(np.abs(sg - S_ref)) / np.max(np.abs(S_ref)))
        par["pass"] = par["o_rel_err"] <= par["tol"] and par.get("S_T_rel_err", 0.0) <= par["tol"]
        res["parity"] = par
        del o_ref, S_ref
    del q, k, v, la, b, o, ST
    torch.cuda.empty_cache()
    return res


def run_prefill_rate(wname, args, torch, kda, synth, stages=False, bounded=None):
    """Call time and rate of another prefill workload (no CPU baseline):
    context for the main line, which times the 131072-token workload.  With
    ``stages`` every input and output stage runs (raw q and k, the gate
    projection's output, RMSNorm and the sigmoid output gate).  ``bounded``
    (bytes) runs the bounded-workspace schedule inside that much workspace."""
    w = synth.workload_prefill(wname)
    stage_kw = {}
    if stages:
        si = synth.make_stage_inputs(w, 4242)
        w.q, w.k = si.q_raw, si.k_raw
        w.log_alpha = si.z_gate
    bf = w.io_dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    def up(x, io=False):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.to(tdt) if io else t).cuda()

    q, k, v = up(w.q, True), up(w.k, True), up(w.v, True)
    la = up(w.log_alpha) if w.log_alpha is not None else None
    b, cu = up(w.beta), up(w.cu_seqlens)
    S0 = up(w.S0) if w.S0 is not None else None
    if stages:
        stage_kw = dict(l2norm_qk=True, gate_softplus=True, norm_weight=up(si.norm_weight),
                        out_gate=up(si.z_out, True))
        del si
    T_tok, H, dk = w.q.shape
    dv = w.v.shape[2]
    N = w.num_seqs
    o = torch.empty((T_tok, H, dv), dtype=tdt, device="cuda")
    ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    host_cu = w.cu_seqlens.tolist()
    stream = torch.cuda.current_stream()
    if bounded:
        kda.clear_workspace_cache()  # the bounded call gets a workspace of its own size
        torch.cuda.empty_cache()
    for _ in range(5):  # the two-stream schedules settle over their first calls
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk,
                    one_stream=args.one_stream, max_workspace_bytes=bounded, **stage_kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record(stream)
    for _ in range(n):
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk,
                    one_stream=args.one_stream, max_workspace_bytes=bounded, **stage_kw)
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) / n / 1e3
    recovered = kda.prefill_recovered(q, v, cu, chunk=w.chunk, cu_seqlens_host=host_cu, one_stream=args.one_stream,
                                      max_workspace_bytes=bounded)
    if bounded:
        kda.clear_workspace_cache()
    nbytes, _, per_th, _ = prefill_algorithmic(T_tok, N, H, dk, dv, 2 if bf else 4, w.chunk, S0 is not None, w.gate)
    if stages:  # the output gate's pre-activation is read once more per token-head
        nbytes += T_tok * H * dv * (2 if bf else 4)
        per_th += dv * (2 if bf else 4)
    del q, k, v, la, b, o, ST, S0, stage_kw
    torch.cuda.empty_cache()
    achieved = nbytes / call_s / 1e9
    label = wname + ("+stages" if stages else "") + ("+bounded%dMiB" % (bounded >> 20) if bounded else "")
    return dict(workload=label, gate=w.gate, num_seqs=N, total_tokens=T_tok, heads=H,
                workspace_limit_bytes=bounded, call_ms=round(call_s * 1e3, 4), tokens_per_s=round(T_tok / call_s, 1),
                hbm_frac=round(achieved / HBM_PEAK_GBS, 4), recovered=recovered,
                roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(achieved / HBM_PEAK_GBS, 4), bytes_per_launch=int(nbytes),
                              bytes_per_token_head=per_th))


FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 MFMA


def backward_algorithmic(T_tok: int, N: int, H: int, dk: int, dv: int, es: int, C: int, with_s0: bool,
                         gate: str = "channel"):
    """Compulsory bytes and method flops of one kda_prefill_backward call.
    Bytes: read q, k, v, dO (io dtype), log_alpha (gate width x 4), beta;
    write dq, dk, dv (io dtype), dlog_alpha, dbeta; states: read S0 and dS_T,
    write dS0 (fp32).  Flops per token-head of the chunked backward (64-token
    chunks, triangular C x C products at half): 20 dk dv (forward recompute
    4 + 2, state cotangents 6, value-side cotangents 8) + 6 C dk (the gated
    pair matrices A and P, 2; the gated pair sums, 4) + 8 C dv (the
    triangular products with T, P and their transposes in the two state
    passes and the value-side kernel, 6; the cotangent pair matrices dP and
    dM, 2)."""
    th = T_tok * H
    gw = dk if GATE_WIDTH[gate] is None else GATE_WIDTH[gate]
    per_th = 2 * ((2 * dk + dv) * es + gw * 4 + 4) + dv * es
    state = N * H * dk * dv * 4 * (3 if with_s0 else 2)
    flops_th = 20 * dk * dv + 6 * C * dk + 8 * C * dv
    return th * per_th + state, th * flops_th, per_th, flops_th


def run_backward(wname, args, torch, kda, synth, oracle, check: bool):
    """kda_prefill_backward on a workload: call time, roofline against the
    fp32 MFMA peak (the backward's products run in fp32), and, when
    ``check``, the fp64 oracle's backward timed on the host over the whole
    workload and compared element by element."""
    w = synth.workload_prefill(wname)
    cot = synth.make_cotangents(w, 7000 + synth.WORKLOADS[wname]["index"], dS_T_std=0.1)
    bf = w.io_dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    def up(x, io=False):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.to(tdt) if io else t).cuda()

    T_tok, H, dk = w.q.shape
    dv = w.v.shape[2]
    N = w.num_seqs
    args_d = [up(w.q, True), up(w.k, True), up(w.v, True), up(w.log_alpha) if w.log_alpha is not None else None,
              up(w.beta), up(w.cu_seqlens), up(w.S0) if w.S0 is not None else None, up(cot.dO, True), up(cot.dS_T)]
    host_cu = w.cu_seqlens.tolist()
    for _ in range(2):
        g = kda.prefill_backward(*args_d, cu_seqlens_host=host_cu)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    e0.record(stream)
    for _ in range(n):
        g = kda.prefill_backward(*args_d, cu_seqlens_host=host_cu)
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) / n / 1e3
    nbytes, nflops, per_th, flops_th = backward_algorithmic(T_tok, N, H, dk, dv, 2 if bf else 4, 64,
                                                            w.S0 is not None, w.gate)
    tfl = nflops / call_s / 1e12
    traffic = measured_traffic("backward_" + wname)
    # The backward's products run as split-bf16 (three bf16 MFMAs per fp32-
    # accurate product), so the peak is the bf16 MFMA one; the fp32 MFMA
    # figure and the counted HBM rate are given beside it.
    res = dict(workload=wname, num_seqs=N, total_tokens=T_tok, heads=H, call_ms=round(call_s * 1e3, 4),
               tokens_per_s=round(T_tok / call_s, 1),
               roofline=dict(bound="mfma", achieved=round(tfl, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                             frac=round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), traffic=traffic,
                             kernel="kda_prefill_backward (prep, states, grad_v, grad_k)",
                             products="split-bf16 (3 bf16 MFMAs per product; the chain passes with bf16 io: 2, single-bf16 block factors)",
                             fp32_mfma_frac=round(tfl / FP32_MFMA_PEAK_TFLOPS, 4),
                             flops_per_launch=int(nflops), flops_per_token_head=flops_th,
                             hbm_achieved=round(nbytes / call_s / 1e9, 1), hbm_frac=round(nbytes / call_s / 1e9 / HBM_PEAK_GBS, 4),
                             counted_hbm_frac=(round(traffic / call_s / 1e9 / HBM_PEAK_GBS, 4) if traffic else None),
                             bytes_per_launch=int(nbytes), bytes_per_token_head=per_th))
    if check:
        log("backward cpu baseline: oracle backward on %d tokens x %d heads ..." % (T_tok, H))
        t1 = time.perf_counter()
        ref = oracle.backward(w.q, w.k, w.v, w.log_alpha_channels(), w.beta, w.cu_seqlens, w.S0, cot.dO, cot.dS_T,
                              threads=args.cpu_threads)
        dt = time.perf_counter() - t1
        cores = os.cpu_count() if args.cpu_threads <= 0 else args.cpu_threads
        res["cpu_baseline"] = dict(value=round(T_tok / dt, 1), unit="tokens/s", cores=int(min(cores, N * H)),
                                   kind="oracle", sample="whole workload (%d x %d tokens, %d heads), fp64 reverse-mode "
                                                         "recurrence, %.1f s" % (N, T_tok // max(N, 1), H, dt))
        if w.gate == "scalar":
            ref["dlog_alpha"] = ref["dlog_alpha"].sum(axis=-1)
        par = dict(tol=1e-2 if bf else 1e-4)
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"):
            if g[name] is None or ref[name] is None:
                continue
            x = g[name].float().cpu().numpy().astype(np.float64)
            par[name + "_rel_err"] = float(np.max(np.abs(x - ref[name])) / np.max(np.abs(ref[name])))
        par["pass"] = all(v_ <= par["tol"] for k_, v_ in par.items() if k_.endswith("_rel_err"))
        res["parity"] = par
    del args_d, g
    kda.clear_workspace_cache()
    torch.cuda.empty_cache()
    return res


def decode_cpu_baseline(args, synth, oracle, B, H, dk, dv, std, seed):
    """fp64 oracle decode rate: the first steps of the decode workload on all
    host cores (every state), and on one thread (a slice of the states)."""
    S = synth.make_decode_state(B, H, dk, dv, std, seed).astype(np.float64)
    n = max(1, args.cpu_decode_steps)
    xs = [synth.make_decode_step(B, H, dk, dv, "bf16", seed, t) for t in range(n)]
    t0 = time.perf_counter()
    for x in xs:
        _, S = oracle.decode_step(x.q, x.k, x.v, x.log_alpha, x.beta, S, threads=args.cpu_threads, inplace=True)
    dt = time.perf_counter() - t0
    cores = os.cpu_count() if args.cpu_threads <= 0 else args.cpu_threads
    res = dict(value=round(B * H * n / dt, 1), unit="state-updates/s", cores=int(cores), kind="oracle",
               sample="first %d of the workload's steps, all %d states, fp64, %.1f s" % (n, B * H, dt))
    Bs = max(1, B // 16)
    S1 = S[:Bs].copy()
    t0 = time.perf_counter()
    for x in xs[:2]:
        _, S1 = oracle.decode_step(x.q[:Bs], x.k[:Bs], x.v[:Bs], x.log_alpha[:Bs], x.beta[:Bs], S1, threads=1,
                                   inplace=True)
    dt1 = time.perf_counter() - t0
    res["single_thread"] = dict(value=round(Bs * H * 2 / dt1, 1), unit="state-updates/s",
                                sample="2 steps of %d states, one thread, %.1f s" % (Bs * H, dt1))
    return res


def run_decode(args, torch, kda, synth, oracle=None, gate="channel", steps=None, stages=False):
    wd = synth.WORKLOADS["decode256x32_bf16"]
    B, H, dk, dv = wd["B"], wd["H"], wd["dk"], wd["dv"]
    steps = steps or args.decode_steps
    seed = 1000 + wd["index"]
    t0 = time.time()
    S_host = synth.make_decode_state(B, H, dk, dv, wd["S0_std"], seed)
    S0 = torch.from_numpy(S_host).cuda()
    del S_host
    import concurrent.futures
    qs, ks, vs, las, bs = [], [], [], [], []
    blk = 64
    with concurrent.futures.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        for s0 in range(0, steps, blk):
            xs = list(ex.map(lambda t: synth.make_decode_step(B, H, dk, dv, "bf16", seed, t, gate=gate),
                             range(s0, min(steps, s0 + blk))))
            for x in xs:
                qs.append(torch.from_numpy(x.q).to(torch.bfloat16).cuda())
                ks.append(torch.from_numpy(x.k).to(torch.bfloat16).cuda())
                vs.append(torch.from_numpy(x.v).to(torch.bfloat16).cuda())
                las.append(torch.from_numpy(x.log_alpha).cuda() if x.log_alpha is not None else None)
                bs.append(torch.from_numpy(x.beta).cuda())
    log("generated decode inputs (%d steps) in %.1fs" % (steps, time.time() - t0))
    S = S0.clone()
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    stage_kw = {}
    if stages:  # every input and output stage (values drawn once, reused per step)
        g = torch.Generator(device="cpu").manual_seed(4243)
        stage_kw = dict(l2norm_qk=True, gate_softplus=True,
                        norm_weight=(0.5 + torch.rand(dv, generator=g)).cuda(),
                        out_gate=torch.randn((B, H, dv), generator=g).to(torch.bfloat16).cuda())
    for t in range(min(16, steps)):  # warm-up on a scratch copy of the state
        kda.decode_step(qs[t], ks[t], vs[t], las[t], bs[t], S, o=o, **stage_kw)
    S.copy_(S0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for t in range(steps):
        kda.decode_step(qs[t], ks[t], vs[t], las[t], bs[t], S, o=o, **stage_kw)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_s = e0.elapsed_time(e1) / 1e3 / steps
    nbytes, per = decode_algorithmic(B * H, dk, dv, 2, gate)
    if stages:  # the output gate's pre-activation
        nbytes += B * H * dv * 2
        per += dv * 2
    achieved = nbytes / step_s / 1e9
    res = dict(
        metric="decode state-updates/s", gate=gate, stages=stages, value=round(B * H * steps / wall, 1), unit="state-updates/s",
        us_per_step=round(step_s * 1e6, 2),
        event_updates_per_s=round(B * H / step_s, 1),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic("decode"),
                      kernel="decode_kernel", bytes_per_launch=int(nbytes), bytes_per_update=per),
        workload=dict(workload="decode256x32_bf16", B=B, heads=H, dk=dk, dv=dv, steps=steps,
                      state_bytes=B * H * dk * dv * 4),
    )
    del qs, ks, vs, las, bs, S, S0
    torch.cuda.empty_cache()
    if oracle is not None and not args.no_cpu_baseline and gate == "channel":
        log("cpu baseline: decode oracle ...")
        res["cpu_baseline"] = decode_cpu_baseline(args, synth, oracle, B, H, dk, dv, wd["S0_std"], seed)
    return res


def copy_probe(nbytes: int, torch):
    """A plain device copy of known size, for scaling hardware byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    bb = torch.empty_like(a)
    for _ in range(3):
        bb.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long131072_bf16")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the 4x4096 and varlen prefill rates")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1 << 30, help="oracle tokens (default: all)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--cpu-decode-steps", type=int, default=16)
    ap.add_argument("--one-stream", action="store_true",
                    help="prefill on the caller's stream only (for hardware-counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, help="run only a device copy of this many bytes")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass lines")
    ap.add_argument("--backward-workloads", default="batch4x4096_bf16,long131072_bf16",
                    help="comma list of workloads for the backward lines (the first is checked against the oracle)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (each GPU would run "
              "its own heads or sequences independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, torch)
        return
    import gated_delta_rule_33_amd as kda
    import oracle
    import synth
    kda.load_library()

    pre = run_prefill(args, torch, kda, synth, oracle)
    dec = None if args.no_decode else run_decode(args, torch, kda, synth, oracle)
    other = [] if args.no_other else [run_prefill_rate(n, args, torch, kda, synth)
                                      for n in ("batch4x4096_bf16", "varlen64_bf16", "long131072_bf16_gdn",
                                                "long131072_bf16_deltanet")]
    if not args.no_other:
        other.append(run_prefill_rate("long131072_bf16", args, torch, kda, synth, stages=True))
        # the bounded-workspace schedule inside 1 GiB (the one-stream workspace is 4.1 GB and 13.2 GB)
        other += [run_prefill_rate(n, args, torch, kda, synth, bounded=1 << 30)
                  for n in ("long131072_bf16", "varlen64_bf16")]
    dec_gates = [] if (args.no_decode or args.no_other) else [
        run_decode(args, torch, kda, synth, None, gate=g, steps=min(256, args.decode_steps)) for g in ("scalar", "none")]
    if dec_gates:
        dec_gates.append(run_decode(args, torch, kda, synth, None, steps=min(256, args.decode_steps), stages=True))
    bwd = [] if args.no_backward else [
        run_backward(name, args, torch, kda, synth, oracle, check=(i == 0 and not args.no_cpu_baseline))
        for i, name in enumerate(x for x in args.backward_workloads.split(",") if x)]
    wl = pre["workload"]
    line = {
        "metric": "KDA prefill tokens/s (MFMA % peak) at T=128k; decode state-updates/s (HBM %)",
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64, distributions of the 131072-token workload)",
        "config": {"workload": wl["workload"], "global_batch": wl["num_seqs"], "seq_len": wl["total_tokens"],
                   "heads": wl["heads"], "dk": wl["dk"], "dv": wl["dv"], "chunk": wl["chunk"],
                   "io_dtype": wl["io_dtype"], "state_dtype": "f32", "parallelism": "single-gpu"},
        "roofline": pre["roofline"],
        "prefill_call_ms": {"mean": round(pre["call_ms_mean"], 4), "min": round(pre["call_ms_min"], 4)},
    }
    line["prefill_recovered"] = pre["recovered"]
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
        line["parity"] = pre["parity"]
    if dec is not None:
        line["decode"] = dec
    if other:
        line["prefill_other"] = other
    if dec_gates:
        line["decode_gate_forms"] = dec_gates
    if bwd:
        line["backward"] = bwd
    print(json.dumps(line), flush=True)
    if pre["recovered"] or any(x.get("recovered") for x in other):
        log("the overlapped prefill schedule fell back to its recovery launches: timing invalid")
        sys.exit(3)
    if "parity" in pre and not pre["parity"]["pass"]:
        log("parity of the last timed call failed")
        sys.exit(4)
    if any("parity" in x and not x["parity"]["pass"] for x in bwd):
        log("backward parity failed")
        sys.exit(4)


if __name__ == "__main__":
    main()
