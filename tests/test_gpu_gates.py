"""GPU parity of the scalar-gate (Gated DeltaNet: one forget rate per head and
token) and no-gate (DeltaNet: alpha = 1) specialisations of the prefill and
decode kernels against the fp64 oracle, which takes the same gate repeated
over the key channels (or zeros).  The oracle's own pins tie exactly these
inputs to independent GDN and DeltaNet recurrences."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, assert_not_recovered, check, dev, gpu_prefill, have_gpu, host, log, oracle_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

RAGGED = [1, 63, 64, 65, 200, 0, 31, 129]


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (64, 128, 32), (128, 64, 64), (64, 64, 32), (128, 128, 16)])
def test_prefill_gate_forms(gate, dt, dk, dv, chunk):
    log("prefill gate=%s dt=%s dk=%d dv=%d chunk=%d" % (gate, dt, dk, dv, chunk))
    w = synth.make_prefill(RAGGED, H=3, dk=dk, dv=dv, io_dtype=dt, seed=51, S0_std=0.05, chunk=chunk, gate=gate)
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL[dt])
    check("S_T", S, S_ref, TOL[dt])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", [("all-60", -60.0), ("spikes-1e4", -1e4), ("all-0", 0.0)], ids=lambda c: c[0])
def test_prefill_scalar_gate_extremes(dt, case):
    """Scalar gates at -60 on every token, isolated -1e4 decays, or exactly
    0 (the scalar path with alpha = 1, which must equal DeltaNet)."""
    name, la = case
    w = synth.make_prefill([200, 64, 17], H=2, dk=128, dv=128, io_dtype=dt, seed=52, S0_std=0.05, gate="scalar")
    if name.startswith("all"):
        w.log_alpha[:] = la
    else:
        w.log_alpha[np.random.default_rng(520).random(w.log_alpha.shape) < 0.05] = la
    w.beta[:] = 1.0
    log("prefill scalar gate extremes dt=%s %s" % (dt, name))
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL[dt])
    check("S_T", S, S_ref, TOL[dt])
    if name == "all-0":
        wn = synth.PrefillInputs(w.q, w.k, w.v, None, w.beta, w.cu_seqlens, w.S0, dt, gate="none")
        on, Sn = gpu_prefill(wn)
        assert np.max(np.abs(on - o)) <= 1e-5 * np.max(np.abs(o))
        assert np.max(np.abs(Sn - S)) <= 1e-5 * np.max(np.abs(S))


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_prefill_gate_forms_overlapped(gate):
    """The overlapped two-stream schedule (few pairs, 200+ chunk indices)."""
    w = synth.make_prefill([5000, 3000, 4096], H=2, dk=128, dv=128, io_dtype="bf16", seed=53, S0_std=0.05,
                           gate=gate)
    log("prefill gate=%s overlapped" % gate)
    rep = {}
    o, S = gpu_prefill(w, report=rep)
    assert_not_recovered(rep)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL["bf16"])
    check("S_T", S, S_ref, TOL["bf16"])


def test_scalar_gate_equals_channel_gate_repeated():
    """A scalar gate through the scalar path and the same rate repeated over
    the channels through the per-channel path agree (fp32, to rounding)."""
    w = synth.make_prefill([333, 70], H=2, dk=128, dv=128, io_dtype="f32", seed=54, S0_std=0.05, gate="scalar")
    wc = synth.PrefillInputs(w.q, w.k, w.v, w.log_alpha_channels(), w.beta, w.cu_seqlens, w.S0, "f32")
    o, S = gpu_prefill(w)
    oc, Sc = gpu_prefill(wc)
    assert np.max(np.abs(o - oc)) <= 1e-5 * np.max(np.abs(oc))
    assert np.max(np.abs(S - Sc)) <= 1e-5 * np.max(np.abs(Sc))


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_decode_gate_forms(gate, dt, dk, dv):
    import gated_delta_rule_33_amd as kda
    B, H, steps = 5, 3, 6
    log("decode gate=%s dt=%s dk=%d dv=%d" % (gate, dt, dk, dv))
    S = synth.make_decode_state(B, H, dk, dv, 0.02, seed=55)
    Sd = dev(S)
    Sref = S.astype(np.float64)
    for t in range(steps):
        x = synth.make_decode_step(B, H, dk, dv, dt, seed=56, step=t, gate=gate)
        la_dev = dev(x.log_alpha) if x.log_alpha is not None else None
        o = kda.decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), la_dev, dev(x.beta), Sd)
        la = np.zeros((B, H, dk), np.float32) if x.log_alpha is None else np.broadcast_to(
            x.log_alpha[:, :, None], (B, H, dk))
        o_ref, Sref = oracle.decode_step(x.q, x.k, x.v, la, x.beta, Sref)
        check("o step %d" % t, host(o), o_ref, TOL[dt])
    check("S after %d steps" % steps, host(Sd), Sref, TOL[dt])
