"""CPU (numpy fp64) chunkwise form of the KDA layer -- a test artifact.

It pins the oracle from an independent algebraic direction: the chunkwise parallel
algorithm of "Decoding Hybrid Attention Architectures" (intl.cloud.baidu.com
article 9569726), section 4, and "Technical Analysis and Engineering Practices for
Novel Hybrid Linear Attention Architectures" (article 9578008), section 3 items 1-2,
must reproduce the token recurrence exactly (up to rounding).

Per chunk of n <= C tokens with entry state S (d_k x d_v), in the pages' notation:

  b_r = sum_{i<=r} g_i                 chunk-local cumulative log-decay (vector per token)
  Gamma_r = exp(b_r)                   "intra-chunk prefix cumulative decay factor"
  gamma = Gamma_n                      "chunk-level decay"
  Qbar = Gamma*Q, Kbar = Gamma*K, Ktil = K/Gamma, Khat = K*exp(b_n - b)
  A = StrictTril(Diag(beta) Kbar Ktil^T),  T = (I + A)^-1 Diag(beta)
  W = T Kbar,  U = T V                 the pages' "precomputed intermediate matrices"
  Unew = U - W S
  O = Qbar S + Tril(Qbar Ktil^T) Unew
  S_next = Diag(gamma) S + Khat^T Unew

Readings: the pages print the state term with (Gamma*K)^T; the derivation from the
recurrence needs the keys decayed to the chunk END (Khat), which is what this uses.
U and W are not defined on the pages; T = (I + A)^-1 Diag(beta) is the reading that
makes the form exact.  Tril in O is inclusive (a token sees its own write), A is
strictly lower.
"""
from __future__ import annotations

import numpy as np


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, C=64):
    q, k, v, g, bt = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        bounds = list(zip(cu[:-1], cu[1:]))
    qf, kf, vf, gf, bf = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g, bt))
    o = np.zeros((B * T, H, Dv))
    S_final = np.zeros((len(bounds), H, Dk, Dv))
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.asarray(S0[n, h], dtype=np.float64).copy()
            for c0 in range(t0, t1, C):
                sl = slice(c0, min(c0 + C, t1))
                Q, K, V, G, beta = qf[sl, h], kf[sl, h], vf[sl, h], gf[sl, h], bf[sl, h]
                nn = K.shape[0]
                b = np.cumsum(G, axis=0)
                Gam = np.exp(b)
                gam = Gam[-1]
                Qbar, Kbar = Q * Gam, K * Gam
                Ktil = K * np.exp(-b)
                Khat = K * np.exp(b[-1][None, :] - b)
                A = np.tril(beta[:, None] * (Kbar @ Ktil.T), -1)
                Tm = np.linalg.solve(np.eye(nn) + A, np.diag(beta))
                W, U = Tm @ Kbar, Tm @ V
                Unew = U - W @ S
                o[sl, h] = Qbar @ S + np.tril(Qbar @ Ktil.T) @ Unew
                S = gam[:, None] * S + Khat.T @ Unew
            S_final[n, h] = S
    return o.reshape(B, T, H, Dv), S_final
