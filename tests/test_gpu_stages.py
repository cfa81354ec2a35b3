"""GPU parity of the input and output stages (kda_stages) against the fp64
oracle's stage definitions (oracle/stages.py): q and k L2-normalised in the
prep and decode kernels, the gate activation log alpha = -softplus(z), and
the head-wise RMSNorm with the sigmoid output gate (an extra pass over o in
prefill, fused into the decode kernel).

The RMSNorm divides each (token, head) row by its own RMS, so an error that
is small against max|o| (the bound the chunked bf16 prefill meets) grows by
max|o| / rms(row) on rows with small outputs.  For bf16 prefill with an
output stage the two parts are therefore checked separately, each to the
bf16 bound: o (with the input stages) against the oracle, and the output
stage against the oracle's definition applied to that same o.  The fp32
path and decode are checked end to end."""
import numpy as np
import pytest

import synth
from oracle import stages as ostages
from tests.gpu_helpers import TOL, assert_not_recovered, check, dev, gpu_prefill, have_gpu, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

COMBOS = {
    "input": dict(l2norm_qk=True, gate_softplus=True),
    "output": dict(norm=True, gate_out=True),
    "norm": dict(norm=True),
    "gate_out": dict(gate_out=True),
    "all": dict(l2norm_qk=True, gate_softplus=True, norm=True, gate_out=True),
}


def _staged(w, si, combo, **run_kw):
    """Run the GPU prefill with the stages of ``combo`` on the stage inputs
    ``si`` and the fp64 oracle on the same values."""
    c = COMBOS[combo]
    dt = w.io_dtype
    l2 = c.get("l2norm_qk", False)
    sp = c.get("gate_softplus", False) and w.log_alpha is not None
    wq = synth.PrefillInputs(si.q_raw if l2 else w.q, si.k_raw if l2 else w.k, w.v,
                             si.z_gate if sp else w.log_alpha, w.beta, w.cu_seqlens, w.S0, dt, w.chunk, w.gate)
    kw = dict(l2norm_qk=l2, gate_softplus=sp, l2norm_eps=1e-6, norm_eps=1e-6)
    if c.get("norm"):
        kw["norm_weight"] = dev(si.norm_weight)
    if c.get("gate_out"):
        kw["out_gate"] = dev(si.z_out, dt)
    o, S = gpu_prefill(wq, **kw, **run_kw)
    y_ref, S_ref = ostages.prefill_staged(wq.q, wq.k, wq.v, wq.log_alpha, wq.beta, wq.cu_seqlens, wq.S0,
                                          l2norm_qk=l2, l2norm_eps=1e-6, gate_softplus=sp,
                                          out_gate=si.z_out if c.get("gate_out") else None,
                                          norm_weight=si.norm_weight if c.get("norm") else None, norm_eps=1e-6)
    return o, S, y_ref, S_ref


def _check_staged(w, si, combo, **run_kw):
    """End to end for fp32; for bf16 with an output stage, o (input stages
    only) against the oracle and the output stage against its definition
    applied to the kernel's own o."""
    c = COMBOS[combo]
    y, S, y_ref, S_ref = _staged(w, si, combo, **run_kw)
    check("S_T", S, S_ref, TOL[w.io_dtype])
    if w.io_dtype == "f32" or not (c.get("norm") or c.get("gate_out")):
        check("y", y, y_ref, TOL[w.io_dtype])
        return y, S
    inner = {k: v for k, v in c.items() if k in ("l2norm_qk", "gate_softplus")}
    COMBOS["_inner"] = inner
    try:
        o, _, o_ref, _ = _staged(w, si, "_inner", **run_kw)
    finally:
        del COMBOS["_inner"]
    check("o (input stages)", o, o_ref, TOL[w.io_dtype])
    y_of_o = ostages.output_stage(o, si.z_out if c.get("gate_out") else None,
                                  si.norm_weight if c.get("norm") else None, 1e-6)
    check("y = stage(o)", y, y_of_o, TOL[w.io_dtype])
    log("  end to end y vs oracle (informative): %.3e" % (np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref))))
    return y, S


@pytest.mark.parametrize("combo", list(COMBOS))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["channel", "scalar", "none"])
def test_prefill_stages(combo, dt, gate):
    log("prefill stages=%s dt=%s gate=%s" % (combo, dt, gate))
    w = synth.make_prefill([1, 63, 64, 65, 200, 0, 129], H=3, dk=128, dv=128, io_dtype=dt, seed=61, S0_std=0.05,
                           gate=gate)
    si = synth.make_stage_inputs(w, 62)
    _check_staged(w, si, combo)


@pytest.mark.parametrize("dk,dv,chunk", [(64, 64, 32), (128, 64, 16), (64, 128, 64)])
def test_prefill_stages_shapes(dk, dv, chunk):
    log("prefill stages all dk=%d dv=%d chunk=%d" % (dk, dv, chunk))
    w = synth.make_prefill([300, 5, 77], H=2, dk=dk, dv=dv, io_dtype="bf16", seed=63, S0_std=0.05, chunk=chunk)
    si = synth.make_stage_inputs(w, 64)
    _check_staged(w, si, "all")


def test_prefill_stages_overlapped_and_one_stream():
    """All stages through the overlapped two-stream schedule and the
    one-stream schedule: both match the oracle, bitwise equal to each other."""
    w = synth.make_prefill([6000, 3000], H=2, dk=128, dv=128, io_dtype="bf16", seed=65, S0_std=0.05)
    si = synth.make_stage_inputs(w, 66)
    log("prefill stages overlapped")
    rep = {}
    o, S = _check_staged(w, si, "all", report=rep)
    assert_not_recovered(rep)
    o1, S1, _, _ = _staged(w, si, "all", one_stream=True)
    assert np.array_equal(o1, o) and np.array_equal(S1, S)


def test_gate_softplus_extreme_projection_outputs():
    """Gate projection outputs of +-60 (log alpha from ~-60 to ~-1e-26):
    the activation and the exact diagonal path together stay within bounds."""
    w = synth.make_prefill([200, 64], H=2, dk=128, dv=128, io_dtype="f32", seed=67, S0_std=0.05)
    si = synth.make_stage_inputs(w, 68)
    si.z_gate[:] = np.where(np.random.default_rng(680).random(si.z_gate.shape) < 0.5, 60.0, -60.0)
    log("prefill softplus extremes")
    o, S, y_ref, S_ref = _staged(w, si, "input")
    check("o", o, y_ref, TOL["f32"])
    check("S_T", S, S_ref, TOL["f32"])


@pytest.mark.parametrize("combo", list(COMBOS))
@pytest.mark.parametrize("gate", ["channel", "scalar", "none"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_stages(combo, gate, dt):
    import gated_delta_rule_33_amd as kda
    c = COMBOS[combo]
    log("decode stages=%s gate=%s dt=%s" % (combo, gate, dt))
    for dk, dv in ((128, 128), (64, 128), (128, 64)):
        B, H, steps = 3, 2, 4
        S = synth.make_decode_state(B, H, dk, dv, 0.02, seed=69)
        Sd = dev(S)
        Sref = S.astype(np.float64)
        for t in range(steps):
            x = synth.make_decode_step(B, H, dk, dv, dt, seed=70, step=t, gate=gate)
            # a one-token "prefill" view of the step, for the stage inputs
            wx = synth.PrefillInputs(x.q, x.k, x.v, x.log_alpha, x.beta, np.array([0, B], np.int32), None, dt,
                                     64, gate)
            si = synth.make_stage_inputs(wx, 71 + t)
            l2 = c.get("l2norm_qk", False)
            sp = c.get("gate_softplus", False) and x.log_alpha is not None
            qv, kv = (si.q_raw, si.k_raw) if l2 else (x.q, x.k)
            gz = si.z_gate if sp else x.log_alpha
            kw = dict(l2norm_qk=l2, gate_softplus=sp)
            if c.get("norm"):
                kw["norm_weight"] = dev(si.norm_weight)
            if c.get("gate_out"):
                kw["out_gate"] = dev(si.z_out, dt)
            y = kda.decode_step(dev(qv, dt), dev(kv, dt), dev(x.v, dt), dev(gz) if gz is not None else None,
                                dev(x.beta), Sd, **kw)
            y_ref, Sref = ostages.decode_staged(qv, kv, x.v, gz, x.beta, Sref, l2norm_qk=l2, gate_softplus=sp,
                                                out_gate=si.z_out if c.get("gate_out") else None,
                                                norm_weight=si.norm_weight if c.get("norm") else None)
            check("y %dx%d step %d" % (dk, dv, t), host(y), y_ref, TOL[dt])
        check("S %dx%d" % (dk, dv), host(Sd), Sref, TOL[dt])
