"""The fp64 oracle against its pins (closed forms, the explicit product form,
exact special cases) and its composition identities.  CPU only."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.prefill)


def test_bruteforce_several_shapes():
    for dk, dv, T, seed in [(3, 3, 1, 10), (4, 7, 9, 11), (8, 2, 16, 12)]:
        P.pin_bruteforce(oracle.prefill, dk=dk, dv=dv, T=T, seed=seed)


def _inputs(seed, lengths, H=3, dk=6, dv=5, s0=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, k, v, la, b = P._rand_inputs(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) if s0 else None
    return q, k, v, la, b, cu, S0


def test_split_resume_is_bitwise():
    """prefill(x[:t]) -> S_t, then prefill(x[t:], S0=S_t) equals prefill(x)."""
    q, k, v, la, b, cu, S0 = _inputs(20, [41])
    o, ST = oracle.prefill(q, k, v, la, b, cu, S0)
    for t in (1, 17, 40):
        oa, Sa = oracle.prefill(q[:t], k[:t], v[:t], la[:t], b[:t], [0, t], S0)
        ob, Sb = oracle.prefill(q[t:], k[t:], v[t:], la[t:], b[t:], [0, 41 - t], Sa)
        assert np.array_equal(np.concatenate([oa, ob]), o)
        assert np.array_equal(Sb, ST)


def test_packed_equals_separate_and_empty_sequences():
    lengths = [5, 0, 13, 1, 0, 7]
    q, k, v, la, b, cu, S0 = _inputs(21, lengths)
    o, ST = oracle.prefill(q, k, v, la, b, cu, S0, threads=3)
    for n, L in enumerate(lengths):
        s, e = int(cu[n]), int(cu[n + 1])
        on, Sn = oracle.prefill(q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], [0, L], S0[n:n + 1], threads=1)
        assert np.array_equal(o[s:e], on)
        assert np.array_equal(ST[n], Sn[0])
        if L == 0:
            assert np.array_equal(ST[n], S0[n])


def test_decode_steps_equal_prefill():
    """T decode steps from S0 reproduce the prefill outputs and final state."""
    q, k, v, la, b, cu, S0 = _inputs(22, [9], H=2)
    o, ST = oracle.prefill(q, k, v, la, b, cu, S0)
    S = S0.copy()
    for t in range(9):
        ot, S = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], b[t:t + 1], S)
        assert np.array_equal(ot[0], o[t])
    assert np.array_equal(S, ST)


def test_decode_batch_is_independent_per_row():
    rng = np.random.default_rng(23)
    B, H, dk, dv = 4, 2, 5, 3
    q, k, v, la, b = P._rand_inputs(rng, B, H, dk, dv)
    S = rng.standard_normal((B, H, dk, dv))
    o, Sn = oracle.decode_step(q, k, v, la, b, S, threads=2)
    for i in range(B):
        oi, Si = oracle.decode_step(q[i:i + 1], k[i:i + 1], v[i:i + 1], la[i:i + 1], b[i:i + 1], S[i:i + 1])
        assert np.array_equal(oi[0], o[i]) and np.array_equal(Si[0], Sn[i])


def test_zero_state_default():
    q, k, v, la, b, cu, _ = _inputs(24, [6, 4], s0=False)
    o1, S1 = oracle.prefill(q, k, v, la, b, cu, None)
    o2, S2 = oracle.prefill(q, k, v, la, b, cu, np.zeros((2, 3, 6, 5)))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_rejects_bad_offsets():
    q, k, v, la, b, cu, S0 = _inputs(25, [3, 3])
    with pytest.raises(Exception):
        oracle.prefill(q, k, v, la, b, np.array([0, 4, 3], np.int32), S0)
