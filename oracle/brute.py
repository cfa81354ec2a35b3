"""Brute-force explicit-product form of KDA, for tiny sizes only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The "Kimi Linear" deep-read report (zako-mio knowledge base), sections 2.4
and 6.1, writes every attention variant in one recurrent form: the output at
step t is a sum over earlier steps j of q_t^T times the ordered product of
data-dependent transition matrices A_{j+1} ... A_t times k_j v_j^T.  For KDA
the transition is A_i = (I - beta_i k_i k_i^T) Diag(alpha_i) (section 2.3)
and each write carries its strength beta_j.  With an initial state S0 the
product over all steps also carries S0 forward.

This module evaluates exactly that sum with explicit dense dk x dk matrices
and no recurrence, so it shares no arithmetic structure with the sequential
C oracle: a dropped term, a transposed operand or a wrong gate axis in either
one shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np


def transition(k_t: np.ndarray, log_alpha_t: np.ndarray, beta_t: float) -> np.ndarray:
    """A_t = (I - beta_t k_t k_t^T) Diag(exp(log_alpha_t)), a dk x dk matrix."""
    dk = k_t.shape[0]
    erase = np.eye(dk) - beta_t * np.outer(k_t, k_t)
    return erase @ np.diag(np.exp(log_alpha_t))


def unified_form(q, k, v, log_alpha, beta, S0=None):
    """One sequence, one head: q, k, log_alpha [T, dk]; v [T, dv]; beta [T].

    Returns (o [T, dv], S_T [dk, dv]) computed as
        S_t = (A_t ... A_1) S0 + sum_{j<=t} (A_t ... A_{j+1}) beta_j k_j v_j^T
        o_t = S_t^T q_t
    with every ordered product formed explicitly.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    la = np.asarray(log_alpha, np.float64)
    b = np.asarray(beta, np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    A = [transition(k[i], la[i], b[i]) for i in range(T)]

    def prod(lo: int, hi: int) -> np.ndarray:
        """A_hi A_{hi-1} ... A_lo (identity when lo > hi)."""
        M = np.eye(dk)
        for i in range(lo, hi + 1):
            M = A[i] @ M
        return M

    s0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)
    o = np.zeros((T, dv))
    S_t = s0
    for t in range(T):
        S_t = prod(0, t) @ s0
        for j in range(t + 1):
            S_t = S_t + prod(j + 1, t) @ (b[j] * np.outer(k[j], v[j]))
        o[t] = S_t.T @ q[t]
    return o, S_t
