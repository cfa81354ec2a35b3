"""GPU parity of kda_decode_step against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, check, dev, have_gpu, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_decode_steps_match_oracle(dt, dk, dv):
    import gated_delta_rule_33_amd as kda
    B, H, steps = 5, 3, 6
    log("decode parity dt=%s dk=%d dv=%d B=%d H=%d steps=%d" % (dt, dk, dv, B, H, steps))
    S = synth.make_decode_state(B, H, dk, dv, 0.02, seed=77)
    Sd = dev(S)
    Sref = S.astype(np.float64)
    for t in range(steps):
        x = synth.make_decode_step(B, H, dk, dv, dt, seed=78, step=t)
        o = kda.decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.log_alpha), dev(x.beta), Sd)
        o_ref, Sref = oracle.decode_step(x.q, x.k, x.v, x.log_alpha, x.beta, Sref)
        check("o step %d" % t, host(o), o_ref, TOL[dt])
    check("S after %d steps" % steps, host(Sd), Sref, TOL[dt])


@pytest.mark.parametrize("B,H", [(1, 1), (3, 1), (1, 17), (43, 3)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_decode_odd_batch_counts(B, H, dk, dv):
    """Batch x head counts that fill no power-of-two grid (1, 3, 17 and 129
    states), bf16 io, three steps."""
    import gated_delta_rule_33_amd as kda
    log("decode odd counts B=%d H=%d dk=%d dv=%d" % (B, H, dk, dv))
    S = synth.make_decode_state(B, H, dk, dv, 0.02, seed=91)
    Sd = dev(S)
    Sref = S.astype(np.float64)
    for t in range(3):
        x = synth.make_decode_step(B, H, dk, dv, "bf16", seed=92, step=t)
        o = kda.decode_step(dev(x.q, "bf16"), dev(x.k, "bf16"), dev(x.v, "bf16"), dev(x.log_alpha), dev(x.beta), Sd)
        o_ref, Sref = oracle.decode_step(x.q, x.k, x.v, x.log_alpha, x.beta, Sref)
        check("o step %d" % t, host(o), o_ref, TOL["bf16"])
    check("S after 3 steps", host(Sd), Sref, TOL["bf16"])


def test_decode_zero_batch_is_noop():
    import gated_delta_rule_33_amd as kda
    import torch
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    S = torch.zeros((0, 2, 64, 64), dtype=torch.float32, device="cuda")
    o = kda.decode_step(q, q, q, q.float(), torch.zeros((0, 2), device="cuda"), S)
    assert o.shape == (0, 2, 64)
