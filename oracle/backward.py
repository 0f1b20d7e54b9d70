"""fp64 adjoint of the KDA recurrence -- TEST INFRASTRUCTURE (see the package docstring).

Reverse-mode derivative of the token recurrence (the course's quiz Q9 delta rule with the
per-channel forget gate of the skill card's quick facts), per sequence and head:

    St~ = Diag(alpha_t) S_{t-1},  alpha_t = exp(g_t)
    p_t = St~^T k_t,   u_t = beta_t (v_t - p_t),   S_t = St~ + k_t u_t^T,   o_t = scale S_t^T q_t

for the scalar L = sum_t <do_t, o_t> + <dS_T, S_T>.  Walking t = T..1 with dS = dL/dS_t:

    dS    += scale q_t do_t^T            dq_t  = scale S_t do_t
    du     = dS^T k_t                    dk_t  = dS u_t + St~ dp
    dbeta  = <du, v_t - p_t>             dv_t  = beta_t du,     dp = -beta_t du
    dSt~   = dS + k_t dp^T               dg_t  = alpha_t * rowsum(dSt~ * S_{t-1})
    dS     = Diag(alpha_t) dSt~          (= dL/dS_{t-1});   dS_0 = dS after t = 1

Plain numpy per token (the forward is recomputed here, in fp64, from the same inputs).  Pinned
in tests/test_oracle_pins.py by central finite differences of L and by the closed form of the
pure-decay case.
"""
from __future__ import annotations

import numpy as np


def forward_states(q, k, v, g, beta, S0, scale):
    """One (sequence, head): all states S_0..S_T and the outputs, fp64."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    states = [S.copy()]
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        St = np.exp(g[t])[:, None] * S
        p = St.T @ k[t]
        u = beta[t] * (v[t] - p)
        S = St + np.outer(k[t], u)
        o[t] = scale * (S.T @ q[t])
        states.append(S.copy())
    return states, o


def backward(q, k, v, g, beta, cu_seqlens=None, scale=1.0, initial_state=None, do=None, dS_final=None,
             amplification=False):
    """Gradients of L = sum(do * o) + sum(dS_final * S_final) for packed varlen inputs.

    q, k, g: [T, H, dk]; v, do: [T, H, dv]; beta: [T, H]; initial_state, dS_final:
    [N, H, dk, dv] or None (zeros).  Returns (dq, dk, dv, dg, dbeta, dS0), fp64.

    amplification=True also returns amp [T, H, dk]: the sum of the magnitudes of the terms whose
    signed sum is dg, amp_t = alpha_t * rowsum(|dSt~ * S_{t-1}|) (a diagnostic: it sizes how much
    an error in the states reaches dg through the cancellation in that sum)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv_ = v.shape[2]
    cu = np.asarray(cu_seqlens if cu_seqlens is not None else [0, T], dtype=np.int64)
    N = len(cu) - 1
    do = np.zeros((T, H, dv_)) if do is None else np.asarray(do, dtype=np.float64)
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(g), np.zeros_like(beta)]
    dq_, dk_, dvv, dg_, db_ = out
    dS0 = np.zeros((N, H, dk, dv_))
    amp = np.zeros_like(g) if amplification else None
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S0 = np.zeros((dk, dv_)) if initial_state is None else np.asarray(initial_state[n, h], dtype=np.float64)
            states, _ = forward_states(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], beta[a:b, h], S0, scale)
            dS = np.zeros((dk, dv_)) if dS_final is None else np.array(dS_final[n, h], dtype=np.float64)
            for t in range(b - a - 1, -1, -1):
                tt = a + t
                S_prev, S_t = states[t], states[t + 1]
                al = np.exp(g[tt, h])
                kt, qt, vt, bt = k[tt, h], q[tt, h], v[tt, h], beta[tt, h]
                dS = dS + scale * np.outer(qt, do[tt, h])
                dq_[tt, h] = scale * (S_t @ do[tt, h])
                St = al[:, None] * S_prev
                p = St.T @ kt
                u = bt * (vt - p)
                du = dS.T @ kt
                db_[tt, h] = du @ (vt - p)
                dvv[tt, h] = bt * du
                dp = -bt * du
                dk_[tt, h] = dS @ u + St @ dp
                dSt = dS + np.outer(kt, dp)
                dg_[tt, h] = al * np.sum(dSt * S_prev, axis=1)
                if amp is not None:
                    amp[tt, h] = al * np.sum(np.abs(dSt * S_prev), axis=1)
                dS = al[:, None] * dSt
            dS0[n, h] = dS
    if amp is not None:
        return dq_, dk_, dvv, dg_, db_, dS0, amp
    return dq_, dk_, dvv, dg_, db_, dS0


def backward_fused(q, k, v, g_pre, b_pre, cu_seqlens=None, scale=1.0, initial_state=None, do=None, dS_final=None,
                   normalize=True, gate=True):
    """Gradients through the fused prologue (the operator takes, with gate, g = -5 sigmoid(a),
    beta = sigmoid(b) and, with normalize, q / |q| and k / |k| over d_k): backward() on the
    prologue's outputs, then the chain rule back to the raw inputs, per (token, head):
        dL/da = dL/dg * (-5) s (1 - s),  s = sigmoid(a);      dL/db = dL/dbeta * beta (1 - beta);
        dL/dq = (dL/dq_n - q_n <q_n, dL/dq_n>) / |q|   (0 for a zero row), the same for k.
    Without gate, g_pre and b_pre are g and beta themselves (their gradients pass unchanged).
    Returns (dq, dk, dv, da, db, dS0) for the raw q, k, v, a, b and S0, fp64."""
    from . import prologue
    qn, kn, g, beta = prologue(q, k, g_pre, b_pre, normalize)
    if not gate:
        g, beta = np.asarray(g_pre, dtype=np.float64), np.asarray(b_pre, dtype=np.float64)
    dqn, dkn, dv, dg, dbeta, dS0 = backward(qn, kn, v, g, beta, cu_seqlens, scale, initial_state, do, dS_final)
    if gate:
        s = 1.0 / (1.0 + np.exp(-np.asarray(g_pre, dtype=np.float64)))
        da = dg * (-5.0) * s * (1.0 - s)
        db = dbeta * beta * (1.0 - beta)
    else:
        da, db = dg, dbeta

    def through_unit(x, xn, dxn):
        if not normalize:
            return dxn
        x = np.asarray(x, dtype=np.float64)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        proj = dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)
        return np.divide(proj, n, out=np.zeros_like(proj), where=n > 0)

    return through_unit(q, qn, dqn), through_unit(k, kn, dkn), dv, da, db, dS0
