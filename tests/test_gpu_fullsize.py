"""Parity at the full sizes of the standard workloads, in the launch
configuration the benchmark times, over every output element: the GPU
computes the whole workload, the fp64 oracle recomputes every head of every
sequence (in groups of heads, to bound host memory), and the metric is the
global max|x - x_ref| / max|x_ref| over all elements, separately for o and
S_T.  The decode workload compares o at every one of its 1024 steps for all
8192 states, and the whole state after the last step."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, assert_not_recovered, dev, have_gpu, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


class GlobalErr:
    """Running max|x - ref| and max|ref| over several pieces of one output."""

    def __init__(self, name):
        self.name, self.num, self.den = name, 0.0, 0.0

    def add(self, got, ref):
        assert np.all(np.isfinite(got)), self.name + ": non-finite output"
        if ref.size:
            self.num = max(self.num, float(np.max(np.abs(got - ref))))
            self.den = max(self.den, float(np.max(np.abs(ref))))

    def check(self, tol):
        e = self.num / self.den if self.den > 0 else self.num
        log("  %-34s rel_err %.3e (tol %.0e) max|ref| %.3e" % (self.name, e, tol, self.den))
        assert e <= tol, "%s: rel err %.3e > %.0e" % (self.name, e, tol)
        return e


def _run(name, group=8, overlapped=False):
    import torch
    import gated_delta_rule_33_amd as kda
    w = synth.workload_prefill(name)
    T, H = w.total_tokens, w.num_heads
    log("full-size %s: T=%d H=%d N=%d, every head checked" % (name, T, H, w.num_seqs))
    dt = w.io_dtype
    q, k, v = dev(w.q, dt), dev(w.k, dt), dev(w.v, dt)
    la = dev(w.log_alpha) if w.log_alpha is not None else None
    b, cu = dev(w.beta), dev(w.cu_seqlens)
    S0 = dev(w.S0) if w.S0 is not None else None
    host_cu = w.cu_seqlens.tolist()
    o, S = kda.prefill(q, k, v, la, b, cu, S0, cu_seqlens_host=host_cu, chunk=w.chunk)
    torch.cuda.synchronize()
    if overlapped:
        assert_not_recovered({"recovered": kda.prefill_recovered(q, v, cu, chunk=w.chunk, cu_seqlens_host=host_cu)})
    del q, k, v, la, b
    eo, es = GlobalErr("o (all %d heads)" % H), GlobalErr("S_T (all %d heads)" % H)
    for h0 in range(0, H, group):
        hs = list(range(h0, min(H, h0 + group)))
        if w.gate == "channel":
            la_h = w.log_alpha[:, hs]
        elif w.gate == "scalar":
            la_h = np.ascontiguousarray(np.broadcast_to(w.log_alpha[:, hs, None], (T, len(hs), w.q.shape[2])))
        else:
            la_h = np.zeros((T, len(hs), w.q.shape[2]), np.float32)
        o_ref, S_ref = oracle.prefill(w.q[:, hs], w.k[:, hs], w.v[:, hs], la_h, w.beta[:, hs],
                                      w.cu_seqlens, None if w.S0 is None else w.S0[:, hs])
        eo.add(host(o[:, h0:h0 + len(hs)]), o_ref)
        es.add(host(S[:, h0:h0 + len(hs)]), S_ref)
        del o_ref, S_ref
        log("  heads %d..%d done" % (hs[0], hs[-1]))
    return eo.check(TOL[dt]), es.check(TOL[dt])


def test_batch4x4096_all_heads():
    _run("batch4x4096_bf16")


def test_long131072_all_heads():
    _run("long131072_bf16", overlapped=True)


def test_varlen64_all_heads():
    _run("varlen64_bf16", group=4)


@pytest.mark.parametrize("name", ["long131072_bf16_gdn", "long131072_bf16_deltanet"])
def test_long131072_gate_forms_all_heads(name):
    """The 131072-token shape with one forget rate per head (Gated DeltaNet)
    and without a gate (DeltaNet)."""
    _run(name, overlapped=True)


def test_decode_full_size_every_state():
    """The benchmark's decode workload (B=256, H=32, d=128, bf16 q/k/v, fp32
    state, 1024 steps): o of all 8192 states at every step, and all states
    after the last step, against the fp64 oracle stepped alongside."""
    import concurrent.futures
    import torch
    import gated_delta_rule_33_amd as kda
    wd = synth.WORKLOADS["decode256x32_bf16"]
    B, H, dk, dv, steps = wd["B"], wd["H"], wd["dk"], wd["dv"], wd["steps"]
    seed = 1000 + wd["index"]
    log("decode full size B=%d H=%d steps=%d, every state" % (B, H, steps))
    S = synth.make_decode_state(B, H, dk, dv, wd["S0_std"], seed)
    Sd = dev(S)
    Sref = S.astype(np.float64)
    del S
    eo = GlobalErr("o (all states, all %d steps)" % steps)
    ex = concurrent.futures.ThreadPoolExecutor(8)
    blk = 32
    for t0 in range(0, steps, blk):
        xs = list(ex.map(lambda t: synth.make_decode_step(B, H, dk, dv, "bf16", seed, t), range(t0, t0 + blk)))
        for x in xs:
            o = kda.decode_step(dev(x.q, "bf16"), dev(x.k, "bf16"), dev(x.v, "bf16"), dev(x.log_alpha),
                                dev(x.beta), Sd)
            o_ref, Sref = oracle.decode_step(x.q, x.k, x.v, x.log_alpha, x.beta, Sref, inplace=True)
            eo.add(host(o), o_ref)
        if (t0 // blk) % 8 == 7:
            log("  step %d" % (t0 + blk))
    ex.shutdown()
    torch.cuda.synchronize()
    eo.check(TOL["bf16"])
    es = GlobalErr("S after %d steps (all states)" % steps)
    es.add(host(Sd), Sref)
    es.check(TOL["bf16"])


def _run_backward(name, group=8):
    """kda_prefill_backward over the whole workload against the oracle's
    backward, every element of every gradient (heads in groups)."""
    import torch
    import gated_delta_rule_33_amd as kda
    w = synth.workload_prefill(name)
    cot = synth.make_cotangents(w, 7000 + synth.WORKLOADS[name]["index"], dS_T_std=0.1)
    T, H = w.total_tokens, w.num_heads
    log("full-size backward %s: T=%d H=%d N=%d, every head checked" % (name, T, H, w.num_seqs))
    dt = w.io_dtype
    g = kda.prefill_backward(dev(w.q, dt), dev(w.k, dt), dev(w.v, dt), dev(w.log_alpha), dev(w.beta),
                             dev(w.cu_seqlens), dev(w.S0) if w.S0 is not None else None, dev(cot.dO, dt),
                             dev(cot.dS_T), cu_seqlens_host=w.cu_seqlens.tolist())
    torch.cuda.synchronize()
    kda.clear_workspace_cache()
    names = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")
    errs = {n: GlobalErr("%s (all %d heads)" % (n, H)) for n in names}
    la = w.log_alpha_channels()
    for h0 in range(0, H, group):
        hs = list(range(h0, min(H, h0 + group)))
        ref = oracle.backward(w.q[:, hs], w.k[:, hs], w.v[:, hs], la[:, hs], w.beta[:, hs], w.cu_seqlens,
                              None if w.S0 is None else w.S0[:, hs], cot.dO[:, hs], cot.dS_T[:, hs])
        for n in names:
            sl = g[n][:, h0:h0 + len(hs)]
            errs[n].add(host(sl), ref[n])
        del ref
        log("  heads %d..%d done" % (hs[0], hs[-1]))
    return {n: errs[n].check(TOL[dt]) for n in names}


def test_backward_long131072_all_heads():
    _run_backward("long131072_bf16", group=16)


def test_backward_varlen64_all_heads():
    """64 sequences of ragged lengths (422,049 tokens), 32 heads, S0 given:
    the backward over many sequences at once (partial last chunks, chunk
    offsets, the longest-first order), every element of every gradient."""
    _run_backward("varlen64_bf16", group=4)
