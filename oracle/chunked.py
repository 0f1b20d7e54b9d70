"""Chunk-parallel form of the KDA recurrence, numpy fp64 -- TEST INFRASTRUCTURE.

Written separately from the C recurrence (``kda_oracle.c``) so that each pins
the other.  It is the textbook unrolling of the recurrence over a block of C
tokens, with nothing fused or reordered beyond that algebra:

Inside a chunk whose entering state is S, with G_r = sum_{j<=r} g_j (natural
log, per channel, restarting at the chunk start):

    A_kk[r, i] = beta_r * sum_c k_rc k_ic exp(G_rc - G_ic)      (i <  r)
    A_qk[r, i] =          sum_c q_rc k_ic exp(G_rc - G_ic)      (i <= r)

The residuals u_r of the recurrence satisfy the unit lower-triangular system

    u_r + sum_{i<r} A_kk[r, i] u_i = beta_r (v_r - S^T (exp(G_r) * k_r))

(solved below by explicit forward substitution), and then

    o_r  = scale * ( S^T (exp(G_r) * q_r) + sum_{i<=r} A_qk[r, i] u_i )
    S'   = Diag(exp(G_last)) S + sum_i (exp(G_last - G_i) * k_i) u_i^T

Derivation: unrolling S_r = Diag(alpha_r) S_{r-1} + k_r u_r^T over the chunk
gives S_r = Diag(e^{G_r}) S + sum_{i<=r} Diag(e^{G_r - G_i}) k_i u_i^T; the
prediction uses the decayed state Diag(alpha_r) S_{r-1}, which is the same sum
with i < r.  This is the chunk-recurrent ("parallel inside a chunk, recurrent
across chunks") form that the course page lists under linear attention
(scripod show notes, chapter 2.1) and that the per-channel gate of the skill
card's quick facts turns into per-channel pairwise decay factors.

Pairwise exponentials are formed only for i <= r, where G_r - G_i <= 0 for a
non-positive log-decay, so nothing overflows.
"""
from __future__ import annotations

import numpy as np


def _chunk(qc, kc, vc, gc, bc, S, scale):
    """One chunk of one head.  qc,kc,gc: [n,dk]; vc: [n,dv]; bc: [n]; S: [dk,dv]."""
    n = qc.shape[0]
    G = np.cumsum(gc, axis=0)                      # [n, dk]
    A_kk = np.zeros((n, n))
    A_qk = np.zeros((n, n))
    for r in range(n):
        for i in range(r + 1):
            dec = np.exp(G[r] - G[i])              # pairwise, <= 1
            if i < r:
                A_kk[r, i] = bc[r] * np.dot(kc[r] * dec, kc[i])
            A_qk[r, i] = np.dot(qc[r] * dec, kc[i])
    eG = np.exp(G)
    rhs = bc[:, None] * (vc - (eG * kc) @ S)       # [n, dv]
    U = np.zeros_like(rhs)
    for r in range(n):                             # explicit forward substitution
        U[r] = rhs[r] - A_kk[r, :r] @ U[:r]
    O = scale * ((eG * qc) @ S + A_qk @ U)
    Glast = G[n - 1]
    S_new = np.exp(Glast)[:, None] * S + (np.exp(Glast[None, :] - G) * kc).T @ U
    return O, S_new


def forward_chunked(q, k, v, g, beta, cu_seqlens=None, scale=1.0, initial_state=None, chunk=64):
    """Same contract as ``oracle.forward`` (without checkpoints); returns (o, S_final).

    Chunks are aligned to each sequence's start; the last chunk of a sequence
    may be partial; no chunk spans two sequences.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = (np.zeros((dk, dv)) if initial_state is None
                 else np.asarray(initial_state[n, h], dtype=np.float64).copy())
            for s in range(cu[n], cu[n + 1], chunk):
                e = min(s + chunk, cu[n + 1])
                O, S = _chunk(q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h], beta[s:e, h], S, scale)
                o[s:e, h] = O
            Sf[n, h] = S
    return o, Sf
