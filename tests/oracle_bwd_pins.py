"""Pins for the oracle's backward pass: facts fixed by calculus and by the
forward recurrence, not by re-running the backward formula.

Each ``pin_*`` takes ``backward`` and ``prefill`` callables with the
oracle's signatures and raises AssertionError when the backward disagrees
with the fact it pins.  The forward (``prefill``) is pinned on its own
(``oracle_pins.py``); here it only serves as the function being
differentiated.  Used against the real oracle (``test_oracle_backward.py``)
and against broken copies of its backward, each of which must fail a pin.

The loss throughout is L = sum_t <dO_t, o_t> + <dS_T, S_T>.
"""
from __future__ import annotations

import numpy as np

from tests.oracle_pins import _rand_inputs


def _case(seed, lengths, H=2, dk=5, dv=4, la_scale=1.0, s0=True, dst=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, k, v, la, b = _rand_inputs(rng, T, H, dk, dv, la_scale=la_scale)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(lengths)
    S0 = rng.standard_normal((N, H, dk, dv)) if s0 else None
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv)) if dst else None
    return dict(q=q, k=k, v=v, la=la, b=b, cu=cu, S0=S0, dO=dO, dST=dST, rng=rng)


def _loss(prefill, c, **over):
    a = dict(c)
    a.update(over)
    o, ST = prefill(a["q"], a["k"], a["v"], a["la"], a["b"], a["cu"], a["S0"])
    L = float(np.sum(o * a["dO"]))
    if a["dST"] is not None:
        L += float(np.sum(ST * a["dST"]))
    return L


def _grads(backward, c):
    return backward(c["q"], c["k"], c["v"], c["la"], c["b"], c["cu"], c["S0"], c["dO"], c["dST"])


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "la": "dlog_alpha", "b": "dbeta", "S0": "dS0"}


def pin_bwd_finite_differences(backward, prefill, seed=30, tol=1e-7):
    """Directional derivatives by central differences of the forward map, one
    random direction per input, against <gradient, direction>.  Three
    sequences (one empty, one longer than the backward's 64-token
    checkpoint span), nonzero S0 and dS_T.  Truncation error of the central
    difference is O(h^2) ~ 1e-10 relative here."""
    c = _case(seed, [70, 0, 9])
    g = _grads(backward, c)
    h = 1e-5
    for name, gname in GRAD_OF.items():
        x = c[name]
        d = c["rng"].standard_normal(x.shape)
        fd = (_loss(prefill, c, **{name: x + h * d}) - _loss(prefill, c, **{name: x - h * d})) / (2 * h)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= tol * max(1.0, abs(an)), (name, fd, an)


def pin_bwd_homogeneity(backward, prefill, seed=31, tol=1e-11):
    """Euler's identity for maps homogeneous of degree one.  For fixed q, k,
    alpha, beta the recurrence is linear in (v, S0) jointly, so
    <v, dv> + <S0, dS0> = L.  The outputs are linear in q and S_T does not
    depend on q, so <q, dq> = sum <dO, o>."""
    c = _case(seed, [23, 11])
    g = _grads(backward, c)
    L = _loss(prefill, c)
    lhs = float(np.sum(c["v"] * g["dv"]) + np.sum(c["S0"] * g["dS0"]))
    assert abs(lhs - L) <= tol * max(1.0, abs(L)), (lhs, L)
    Lo = _loss(prefill, c, dST=None)
    lq = float(np.sum(c["q"] * g["dq"]))
    assert abs(lq - Lo) <= tol * max(1.0, abs(Lo)), (lq, Lo)


def pin_bwd_pure_decay(backward, prefill, seed=32, tol=1e-11):
    """beta = 0 leaves S_t = Diag(e^{g_t}) S0 and o_t = S0^T (e^{g_t} q_t) with
    g_t the running sum of log alpha.  Closed forms: dq_t = e^{g_t} (S0 dO_t);
    dv = dk = 0; dS0 = sum_t (e^{g_t} q_t) dO_t^T + Diag(e^{g_T}) dS_T;
    dlog_alpha_u = sum_{t >= u} e^{g_t} q_t (S0 dO_t) + e^{g_T} rowsum(S0 dS_T);
    dbeta_t = k_t^T G_t (v_t - S0^T (e^{g_t} k_t)) with G_t = dL/dS_t =
    sum_{u >= t} Diag(e^{g_u - g_t}) q_u dO_u^T + Diag(e^{g_T - g_t}) dS_T."""
    c = _case(seed, [15], H=1, dk=6, dv=3, la_scale=0.4)
    c["b"] = np.zeros_like(c["b"])
    g = _grads(backward, c)
    q, k, v, la, S0, dO, dST = (c["q"][:, 0], c["k"][:, 0], c["v"][:, 0], c["la"][:, 0], c["S0"][0, 0],
                                c["dO"][:, 0], c["dST"][0, 0])
    T = q.shape[0]
    gs = np.cumsum(la, axis=0)
    eg = np.exp(gs)
    SdO = dO @ S0.T  # rows: S0 dO_t
    assert np.max(np.abs(g["dq"][:, 0] - eg * SdO)) <= tol
    assert np.max(np.abs(g["dv"])) == 0.0 and np.max(np.abs(g["dk"])) == 0.0
    dS0 = (eg * q).T @ dO + eg[-1][:, None] * dST
    assert np.max(np.abs(g["dS0"][0, 0] - dS0)) <= tol * max(1.0, np.max(np.abs(dS0)))
    per_t = eg * q * SdO
    dla = np.cumsum(per_t[::-1], axis=0)[::-1] + (eg[-1] * np.sum(S0 * dST, axis=1))[None, :]
    assert np.max(np.abs(g["dlog_alpha"][:, 0] - dla)) <= tol * max(1.0, np.max(np.abs(dla)))
    for t in range(T):
        G = sum(np.exp(gs[u] - gs[t])[:, None] * np.outer(q[u], dO[u]) for u in range(t, T))
        G = G + np.exp(gs[-1] - gs[t])[:, None] * dST
        db = k[t] @ G @ (v[t] - S0.T @ (eg[t] * k[t]))
        assert abs(g["dbeta"][t, 0] - db) <= tol * max(1.0, abs(db)), (t, g["dbeta"][t, 0], db)


def pin_bwd_split_resume(backward, prefill, seed=33, tol=1e-12):
    """Cutting a sequence at t: the backward of the tail from S_t with dS_T
    gives dS_t, and the backward of the head with dS_t as its final-state
    cotangent gives the head's gradients; together they equal the whole
    sequence's backward (the state is the only link between the parts)."""
    c = _case(seed, [30])
    g = _grads(backward, c)
    for t in (1, 13, 29):
        _, St = prefill(c["q"][:t], c["k"][:t], c["v"][:t], c["la"][:t], c["b"][:t], [0, t], c["S0"])
        tail = backward(c["q"][t:], c["k"][t:], c["v"][t:], c["la"][t:], c["b"][t:], [0, 30 - t], St,
                        c["dO"][t:], c["dST"])
        head = backward(c["q"][:t], c["k"][:t], c["v"][:t], c["la"][:t], c["b"][:t], [0, t], c["S0"],
                        c["dO"][:t], tail["dS0"])
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            whole = g[name]
            joined = np.concatenate([head[name], tail[name]])
            assert np.max(np.abs(joined - whole)) <= tol * max(1.0, np.max(np.abs(whole))), (t, name)
        assert np.max(np.abs(head["dS0"] - g["dS0"])) <= tol * max(1.0, np.max(np.abs(g["dS0"])))


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_homogeneity, pin_bwd_pure_decay, pin_bwd_split_resume]
