"""Benchmark for libkda on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one kda_prefill call over the whole long-sequence workload: one
sequence of 131072 tokens, 32 heads, dk = dv = 128, bf16 q/k/v/o, fp32
log_alpha/beta/state, chunk 64, 5% long-memory key channels; it returns o and
the final state.  Inputs are resident in HBM before timing starts.  The
decode workload (256 requests x 32 heads, fp32 128x128 states updated in
place for 1024 tokens) is timed in the same run and reported under "decode";
the call rates of the 4 x 4096-token batch and of the 64-sequence varlen
workload follow under "prefill_other" (skip with --no-other).

Prints ONE JSON line.  `value` is prefill tokens/s.  Each roofline block
prices the operator's algorithmic bytes per launch against MI355X's 8 TB/s
HBM peak, using HIP-event durations taken on the stream the kernels run on.
The fp64 oracle is timed on a bounded sample on the host CPU ("cpu_baseline")
and its outputs double as a sampled parity check.
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


def source_digest() -> str:
    """sha256 over the HIP sources; hardware-counter traffic is only reported
    while it was measured on the same kernels."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_33_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except Exception:
        return None
    r = rec.get(key)
    if not r or r.get("source_digest") != source_digest():
        return None
    return r.get("bytes_per_launch")


def prefill_algorithmic(T_tok: int, N: int, H: int, dk: int, dv: int, es: int, C: int, with_s0: bool):
    """Compulsory bytes and algorithmic flops of one prefill call.
    Bytes: read q, k (dk each), v (dv) in the io dtype, log_alpha (dk fp32),
    beta (fp32); write o (dv, io dtype); write S_T (and read S0 when given).
    Flops per token-head: 2 [ (C/2)(3 dk + 2 dv) + 3 dk dv ] -- the two gated
    intra-chunk matrices, the WY factors and the three state contractions,
    triangular products counted at half.  The dense-tile count (as the
    matrix cores execute the triangular products, at full size) is
    2 [ C (3 dk + 2 dv) + 3 dk dv ]."""
    th = T_tok * H
    per_th = (2 * dk + dv) * es + dk * 4 + 4 + dv * es
    state = N * H * dk * dv * 4 * (2 if with_s0 else 1)
    flops_th = 2 * ((C // 2) * (3 * dk + 2 * dv) + 3 * dk * dv)
    return th * per_th + state, th * flops_th, per_th, flops_th


def prefill_dense_flops_th(dk: int, dv: int, C: int) -> int:
    return 2 * (C * (3 * dk + 2 * dv) + 3 * dk * dv)


def decode_algorithmic(BH: int, dk: int, dv: int, es: int):
    """Bytes per decode step: state read + write (fp32), q, k, v, o (io dtype),
    log_alpha (fp32), beta."""
    per = 2 * dk * dv * 4 + (2 * dk + 2 * dv) * es + dk * 4 + 4
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
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk)

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
    if not args.no_cpu_baseline:
        Ts = min(args.cpu_sample_tokens, int(w.cu_seqlens[1]))  # a prefix of the first sequence
        log("cpu baseline: oracle on the first %d tokens x %d heads ..." % (Ts, H))
        t1 = time.perf_counter()
        o_ref, _, used = oracle.prefill(w.q[:Ts], w.k[:Ts], w.v[:Ts], w.log_alpha[:Ts], w.beta[:Ts], [0, Ts],
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
        og = o[:Ts].float().cpu().numpy().astype(np.float64)
        res["parity_sample"] = dict(o_rel_err=float(np.max(np.abs(og - o_ref)) / np.max(np.abs(o_ref))),
                                    tokens=Ts, tol=1e-2 if bf else 1e-4)
    del q, k, v, la, b, o, ST
    torch.cuda.empty_cache()
    return res


def run_prefill_rate(wname, args, torch, kda, synth):
    """Call time and rate of another prefill workload (no CPU baseline):
    context for the main line, which times the 131072-token workload."""
    w = synth.workload_prefill(wname)
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
    for _ in range(2):
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    e0.record(stream)
    for _ in range(n):
        kda.prefill(q, k, v, la, b, cu, S0, o=o, S_T=ST, cu_seqlens_host=host_cu, chunk=w.chunk)
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) / n / 1e3
    nbytes, _, _, _ = prefill_algorithmic(T_tok, N, H, dk, dv, 2 if bf else 4, w.chunk, S0 is not None)
    del q, k, v, la, b, o, ST, S0
    torch.cuda.empty_cache()
    return dict(workload=wname, num_seqs=N, total_tokens=T_tok, heads=H, call_ms=round(call_s * 1e3, 4),
                tokens_per_s=round(T_tok / call_s, 1),
                hbm_frac=round(nbytes / call_s / 1e9 / HBM_PEAK_GBS, 4))


def run_decode(args, torch, kda, synth):
    wd = synth.WORKLOADS["decode256x32_bf16"]
    B, H, dk, dv, steps = wd["B"], wd["H"], wd["dk"], wd["dv"], args.decode_steps
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
            xs = list(ex.map(lambda t: synth.make_decode_step(B, H, dk, dv, "bf16", seed, t),
                             range(s0, min(steps, s0 + blk))))
            for x in xs:
                qs.append(torch.from_numpy(x.q).to(torch.bfloat16).cuda())
                ks.append(torch.from_numpy(x.k).to(torch.bfloat16).cuda())
                vs.append(torch.from_numpy(x.v).to(torch.bfloat16).cuda())
                las.append(torch.from_numpy(x.log_alpha).cuda())
                bs.append(torch.from_numpy(x.beta).cuda())
    log("generated decode inputs (%d steps) in %.1fs" % (steps, time.time() - t0))
    S = S0.clone()
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for t in range(min(16, steps)):  # warm-up on a scratch copy of the state
        kda.decode_step(qs[t], ks[t], vs[t], las[t], bs[t], S, o=o)
    S.copy_(S0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for t in range(steps):
        kda.decode_step(qs[t], ks[t], vs[t], las[t], bs[t], S, o=o)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_s = e0.elapsed_time(e1) / 1e3 / steps
    nbytes, per = decode_algorithmic(B * H, dk, dv, 2)
    achieved = nbytes / step_s / 1e9
    res = dict(
        metric="decode state-updates/s", value=round(B * H * steps / wall, 1), unit="state-updates/s",
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
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long131072_bf16")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the 4x4096 and varlen prefill rates")
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536)
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, default=0, help="run only a device copy of this many bytes")
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
    dec = None if args.no_decode else run_decode(args, torch, kda, synth)
    other = [] if args.no_other else [run_prefill_rate(n, args, torch, kda, synth)
                                      for n in ("batch4x4096_bf16", "varlen64_bf16")]
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
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
        line["parity_sample"] = pre["parity_sample"]
    if dec is not None:
        line["decode"] = dec
    if other:
        line["prefill_other"] = other
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
