"""Seeded synthetic inputs: reproducibility, shapes and distributions."""
import numpy as np

import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, 1e-40], np.float32)
    r = synth.bf16_round(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even (mantissa 0)
    assert r[2] == np.float32(1.0 + 2 ** -7)  # tie -> even (rounds up)
    assert r[3] == -2.5
    bits = synth.bf16_bits(r)
    assert np.array_equal(synth.bf16_bits(synth.bf16_to_f32(bits)), bits)


def test_seeded_reproducible():
    a = synth.workload_prefill("tiny_f32")
    b = synth.workload_prefill("tiny_f32")
    for f in ("q", "k", "v", "log_alpha", "beta", "cu_seqlens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_tiny_workload_distributions():
    w = synth.workload_prefill("tiny_f32")
    assert w.q.shape == (256, 2, 64) and w.v.shape == (256, 2, 64)
    assert np.allclose(np.linalg.norm(w.q, axis=-1), 1.0, atol=1e-5)
    assert np.allclose(np.linalg.norm(w.k, axis=-1), 1.0, atol=1e-5)
    assert np.all(w.log_alpha < 0) and np.all((w.beta > 0) & (w.beta < 1))
    # -softplus(N(0,1)) has mean about -0.806
    assert abs(float(w.log_alpha.mean()) + 0.806) < 0.02
    assert w.S0 is None and w.io_dtype == "f32"


def test_varlen_offsets_and_state():
    w = synth.workload_prefill("varlen64_bf16", H_override=1)
    cu = w.cu_seqlens
    L = np.diff(cu)
    assert cu[0] == 0 and np.all(L >= 128) and np.all(L < 32768) and len(L) == 64
    assert w.S0.shape == (64, 1, 128, 128) and abs(float(w.S0.std()) - 0.02) < 1e-3
    assert np.array_equal(synth.bf16_round(w.q), w.q)


def test_long_memory_mask():
    w = synth.make_prefill([300], H=3, dk=128, dv=16, io_dtype="bf16", seed=7, long_memory_frac=0.05)
    for h in range(3):
        near_one = np.all(w.log_alpha[:, h, :] > -1e-3, axis=0)
        assert int(near_one.sum()) == 6


def test_decode_steps_regenerate_independently():
    a = synth.make_decode_step(2, 3, 8, 4, "bf16", 99, 5)
    b = synth.make_decode_step(2, 3, 8, 4, "bf16", 99, 5)
    c = synth.make_decode_step(2, 3, 8, 4, "bf16", 99, 6)
    assert np.array_equal(a.q, b.q) and not np.array_equal(a.q, c.q)


def test_gate_forms():
    """The scalar gate draws one rate per (token, head) as the last draw of a
    block (so q, k, v and beta equal the per-channel workload's), and no gate
    draws none."""
    ch = synth.make_prefill([100, 5000], H=3, dk=64, dv=64, io_dtype="bf16", seed=7)
    sc = synth.make_prefill([100, 5000], H=3, dk=64, dv=64, io_dtype="bf16", seed=7, gate="scalar")
    no = synth.make_prefill([100, 5000], H=3, dk=64, dv=64, io_dtype="bf16", seed=7, gate="none")
    for w in (sc, no):
        assert np.array_equal(w.q, ch.q) and np.array_equal(w.k, ch.k)
        assert np.array_equal(w.v, ch.v) and np.array_equal(w.beta, ch.beta)
    assert sc.log_alpha.shape == (5100, 3) and no.log_alpha is None
    assert np.all(sc.log_alpha < 0)
    full = sc.log_alpha_channels()
    assert full.shape == (5100, 3, 64) and np.all(full == sc.log_alpha[:, :, None])
    assert np.all(no.log_alpha_channels() == 0)
    x = synth.make_decode_step(4, 2, 64, 64, "bf16", 9, 3, gate="scalar")
    y = synth.make_decode_step(4, 2, 64, 64, "bf16", 9, 3)
    assert x.log_alpha.shape == (4, 2) and np.array_equal(x.q, y.q) and np.array_equal(x.beta, y.beta)
    assert synth.make_decode_step(4, 2, 64, 64, "bf16", 9, 3, gate="none").log_alpha is None
