"""Pins for the oracle's input and output stages (oracle/stages.py): each
checked against a fact of the mathematics, not against its own formula."""
import numpy as np

import oracle
from oracle import stages


def test_l2norm_unit_norm_scale_invariance_and_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.1, 50, size=(7, 3, 1))
    y = stages.l2norm(x, 1e-6)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(stages.l2norm(3.7 * x, 1e-6), y, atol=1e-14)          # scale invariance
    assert np.allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x)   # direction kept
    z = np.zeros((2, 4))
    assert np.array_equal(stages.l2norm(z, 1e-6), z)                       # eps guards 0/0
    tiny = np.full((1, 4), 1e-9)
    assert np.allclose(stages.l2norm(tiny, 1e-6), tiny / 1e-6)             # below eps: divided by eps


def test_gate_activation_closed_forms():
    assert abs(stages.gate_log_alpha(0.0) + np.log(2.0)) < 1e-15            # softplus(0) = ln 2
    z = np.linspace(-30, 30, 121)
    # -softplus(z) = log(sigmoid(-z)) = -logaddexp(0, z)
    assert np.allclose(stages.gate_log_alpha(z), -np.logaddexp(0.0, z), rtol=1e-14, atol=1e-300)
    assert np.allclose(np.exp(stages.gate_log_alpha(z)), 1.0 / (1.0 + np.exp(z)), rtol=1e-12)
    assert abs(stages.gate_log_alpha(800.0) + 800.0) < 1e-12               # no overflow, -> -z
    assert abs(stages.gate_log_alpha(-800.0)) < 1e-300 + 1e-320             # -> -e^{z}
    assert np.all(stages.gate_log_alpha(z) < 0)


def test_output_stage_norm_and_gate():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((5, 2, 32)) * 3.0
    w = np.ones(32)
    y = stages.output_stage(o, None, w, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)    # unit RMS
    assert np.allclose(stages.output_stage(2.5 * o, None, w, eps=0.0), y)    # scale invariance
    w2 = rng.uniform(0.5, 2.0, 32)
    assert np.allclose(stages.output_stage(o, None, w2, eps=0.0), y * w2)    # weight per value channel
    g0 = np.zeros_like(o)
    assert np.allclose(stages.output_stage(o, g0, w, eps=0.0), 0.5 * y)      # sigmoid(0) = 1/2
    assert np.allclose(stages.output_stage(o, g0), 0.5 * o)                  # gate alone
    big = np.full_like(o, 60.0)
    assert np.allclose(stages.output_stage(o, big), o)                       # sigmoid(+inf) -> 1
    assert np.allclose(stages.sigmoid(-np.linspace(0, 40, 9)) + stages.sigmoid(np.linspace(0, 40, 9)), 1.0)
    # eps: a zero output row stays zero and finite
    assert np.array_equal(stages.output_stage(np.zeros((1, 8)), None, np.ones(8), 1e-6), np.zeros((1, 8)))


def test_staged_prefill_reduces_to_plain_and_decode():
    """With no stage selected the staged prefill is the plain oracle; the
    staged decode step equals one staged prefill token."""
    rng = np.random.default_rng(3)
    T, H, dk, dv = 9, 2, 6, 5
    q, k, v = (rng.standard_normal((T, H, d)) for d in (dk, dk, dv))
    z = rng.standard_normal((T, H, dk))
    b = rng.uniform(0, 1, (T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o1, S1 = stages.prefill_staged(q, k, v, z, b, [0, T], S0)
    o2, S2 = oracle.prefill(q, k, v, z, b, [0, T], S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    zo = rng.standard_normal((T, H, dv))
    w = rng.uniform(0.5, 1.5, dv)
    kw = dict(l2norm_qk=True, gate_softplus=True, norm_weight=w)
    y, ST = stages.prefill_staged(q, k, v, z, b, [0, T], S0, out_gate=zo, **kw)
    S = S0[0:1].copy()
    for t in range(T):
        yt, S = stages.decode_staged(q[t:t + 1], k[t:t + 1], v[t:t + 1], z[t:t + 1], b[t:t + 1], S,
                                     out_gate=zo[t:t + 1], **kw)
        assert np.allclose(yt[0], y[t], rtol=1e-12, atol=1e-12)
    assert np.allclose(S, ST, rtol=1e-12, atol=1e-12)
