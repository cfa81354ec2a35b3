"""Pins for the fp64 oracle: checks fixed by the pages and by mathematics,
not by re-running the oracle's own formula.

Each ``pin_*`` takes a ``prefill`` callable with the oracle's signature and
raises AssertionError when the callable disagrees with the fact it pins.
They are used twice: against the real oracle (``test_oracle_pins.py``) and
against deliberately broken copies of it (``test_oracle_mutants.py``), where
every broken copy must fail at least one pin.
"""
from __future__ import annotations

import numpy as np

from oracle.brute import unified_form


def _rand_inputs(rng, T, H, dk, dv, la_scale=1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -la_scale * np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, la, b


def pin_bruteforce(prefill, dk=5, dv=4, T=12, seed=0, tol=1e-12):
    """Whole map against the explicit transition-product form (unified
    recurrent form of the deep-read report, sections 2.4 and 6.1)."""
    rng = np.random.default_rng(seed)
    H = 2
    q, k, v, la, b = _rand_inputs(rng, T, H, dk, dv, la_scale=0.7)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, ST = prefill(q, k, v, la, b, [0, T], S0)
    for h in range(H):
        o_ref, S_ref = unified_form(q[:, h], k[:, h], v[:, h], la[:, h], b[:, h], S0[0, h])
        assert np.max(np.abs(o[:, h] - o_ref)) <= tol * max(1.0, np.max(np.abs(o_ref)))
        assert np.max(np.abs(ST[0, h] - S_ref)) <= tol * max(1.0, np.max(np.abs(S_ref)))


def pin_pure_decay(prefill, dk=6, dv=4, T=20, seed=1, tol=1e-12):
    """beta = 0 switches the delta rule off, leaving per-key-channel decay:
    o_t = S0^T (exp(g_t) * q_t), S_T = Diag(exp(g_T)) S0 with g_t the running
    sum of log_alpha.  dk != dv also pins the gate to the key axis."""
    rng = np.random.default_rng(seed)
    H = 1
    q, k, v, la, _ = _rand_inputs(rng, T, H, dk, dv, la_scale=0.3)
    b = np.zeros((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, ST = prefill(q, k, v, la, b, [0, T], S0)
    g = np.cumsum(la[:, 0], axis=0)
    o_ref = (np.exp(g) * q[:, 0]) @ S0[0, 0]
    assert np.max(np.abs(o[:, 0] - o_ref)) <= tol
    assert np.max(np.abs(ST[0, 0] - np.exp(g[-1])[:, None] * S0[0, 0])) <= tol


def pin_exact_readback(prefill, dk=7, dv=5, T=25, seed=2, tol=1e-12):
    """With unit-norm k and beta = 1 the update makes S_t^T k_t = v_t exactly,
    whatever alpha and S0 are (the erase removes the decayed content along k,
    the write puts v there).  Reading with q_t = k_t therefore returns v_t."""
    rng = np.random.default_rng(seed)
    H = 2
    _, k, v, la, _ = _rand_inputs(rng, T, H, dk, dv)
    b = np.ones((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _ = prefill(k.copy(), k, v, la, b, [0, T], S0)
    assert np.max(np.abs(o - v)) <= tol


def pin_orthonormal_memory(prefill, d=6, dv=4, seed=3, tol=1e-12):
    """alpha = 1 reduces KDA to the delta rule (DeltaNet).  With orthonormal
    keys and beta = 1 the delta rule is an exact key-value memory: writing v
    under key u_j replaces whatever u_j held, and reading u_m for a key never
    written returns S0^T u_m (the report's section 2.2: erase along the key,
    then write)."""
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    order = [0, 2, 0, 3, 2, 2, 4]  # keys 1 and 5 are never written
    T = len(order) + 2
    k = np.zeros((T, 1, d))
    q = np.zeros((T, 1, d))
    v = rng.standard_normal((T, 1, dv))
    for t, j in enumerate(order):
        k[t, 0] = U[:, j]
        q[t, 0] = U[:, j]
    # two read-only probe steps: beta = 0, query an unwritten key
    k[len(order), 0] = U[:, 1]
    q[len(order), 0] = U[:, 1]
    k[len(order) + 1, 0] = U[:, 5]
    q[len(order) + 1, 0] = U[:, 5]
    b = np.ones((T, 1))
    b[len(order):] = 0.0
    la = np.zeros((T, 1, d))
    S0 = rng.standard_normal((1, 1, d, dv))
    o, ST = prefill(q, k, v, la, b, [0, T], S0)
    last = {}
    for t, j in enumerate(order):
        last[j] = v[t, 0]
        assert np.max(np.abs(o[t, 0] - v[t, 0])) <= tol
    assert np.max(np.abs(o[len(order), 0] - S0[0, 0].T @ U[:, 1])) <= tol
    assert np.max(np.abs(o[len(order) + 1, 0] - S0[0, 0].T @ U[:, 5])) <= tol
    # full final memory: written keys hold their last value, the rest keep S0
    expect = np.zeros((d, dv))
    for j in range(d):
        expect += np.outer(U[:, j], last[j] if j in last else S0[0, 0].T @ U[:, j])
    assert np.max(np.abs(ST[0, 0] - expect)) <= tol


def pin_scalar_gate_rescaling(prefill, d=5, dv=3, T=18, seed=4, tol=1e-10):
    """alpha equal across channels gives Gated DeltaNet (scalar gate, the
    zhaixingw.cn explainer's GDN update).  A scalar gate commutes with the
    erase, so with c_t = prod_{u<=t} alpha_u the GDN run equals c_t times a
    DeltaNet (alpha = 1) run on v_t / c_t: o_t(GDN) = c_t o_t(DN)."""
    rng = np.random.default_rng(seed)
    q, k, v, _, b = _rand_inputs(rng, T, 1, d, dv)
    a = -0.2 * np.log1p(np.exp(rng.standard_normal(T)))
    la = np.repeat(a[:, None, None], d, axis=2)
    c = np.exp(np.cumsum(a))
    S0 = rng.standard_normal((1, 1, d, dv))
    o_gdn, S_gdn = prefill(q, k, v, la, b, [0, T], S0)
    o_dn, S_dn = prefill(q, k, v / c[:, None, None], np.zeros_like(la), b, [0, T], S0)
    assert np.max(np.abs(o_gdn - c[:, None, None] * o_dn)) <= tol
    assert np.max(np.abs(S_gdn - c[-1] * S_dn)) <= tol


def pin_single_token(prefill, dk=4, dv=6, seed=5, tol=1e-13):
    """T = 1 closed form: with D = Diag(alpha) and S~ = D S0,
    o = S~^T q + beta (v - S~^T k) (k^T q)  and  S_1 = S~ + beta k (v - S~^T k)^T."""
    rng = np.random.default_rng(seed)
    q, k, v, la, b = _rand_inputs(rng, 1, 1, dk, dv)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = prefill(q, k, v, la, b, [0, 1], S0)
    St = np.exp(la[0, 0])[:, None] * S0[0, 0]
    delta = b[0, 0] * (v[0, 0] - St.T @ k[0, 0])
    assert np.max(np.abs(o[0, 0] - (St.T @ q[0, 0] + delta * (k[0, 0] @ q[0, 0])))) <= tol
    assert np.max(np.abs(ST[0, 0] - (St + np.outer(k[0, 0], delta)))) <= tol


def pin_linearity(prefill, dk=5, dv=4, T=15, seed=6, tol=1e-12):
    """For fixed q, k, alpha, beta the map (S0, V) -> (o, S_T) is linear."""
    rng = np.random.default_rng(seed)
    q, k, v, la, b = _rand_inputs(rng, T, 2, dk, dv)
    S0 = rng.standard_normal((1, 2, dk, dv))
    o, ST = prefill(q, k, v, la, b, [0, T], S0)
    o1, S1 = prefill(q, k, v, la, b, [0, T], np.zeros_like(S0))
    o2, S2 = prefill(q, k, np.zeros_like(v), la, b, [0, T], S0)
    assert np.max(np.abs(o - o1 - o2)) <= tol
    assert np.max(np.abs(ST - S1 - S2)) <= tol


ALL_PINS = [pin_bruteforce, pin_pure_decay, pin_exact_readback, pin_orthonormal_memory,
            pin_scalar_gate_rescaling, pin_single_token, pin_linearity]
