"""Independent numpy fp64 twin of the C oracle.

TEST INFRASTRUCTURE ONLY.  Written separately from ``kda_oracle.c`` and on purpose
in the other algebraic form the pages give: the explicit transition-matrix product

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t

("Decoding Hybrid Attention Architectures", intl.cloud.baidu.com article 9569726,
section 3.4 and its variant table; "Technical Analysis and Engineering Practices for
Novel Hybrid Linear Attention Architectures", article 9578008, section 2 item 4),
transposed into the d_k x d_v state orientation.  The C oracle uses the delta form
S' = Diag(alpha) S, S = S' + beta k (v - S'^T k)^T instead; agreement of the two
pins each against the other.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def kda_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None):
    """Same contract as ``oracle.kda_fwd`` but float inputs only; returns float64
    (o [B, T, H, Dv], S_final [N, H, Dk, Dv])."""
    q, k, v, g, b = (_as_f64(x) for x in (q, k, v, log_alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        bounds = list(zip(cu[:-1], cu[1:]))
    N = len(bounds)
    qf, kf, vf, gf, bf = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g, b))
    o = np.zeros((B * T, H, Dv))
    S_final = np.zeros((N, H, Dk, Dv))
    eye = np.eye(Dk)
    for n, (t0, t1) in enumerate(bounds):
        S = np.zeros((H, Dk, Dv)) if S0 is None else _as_f64(S0[n]).copy()
        for t in range(t0, t1):
            kt = kf[t]                                                  # [H, Dk]
            erase = eye[None] - bf[t][:, None, None] * kt[:, :, None] * kt[:, None, :]
            decayed = np.exp(gf[t])[:, :, None] * S                     # Diag(alpha) S
            S = erase @ decayed + bf[t][:, None, None] * kt[:, :, None] * vf[t][:, None, :]
            o[t] = np.einsum("hcj,hc->hj", S, qf[t])                    # S^T q
        S_final[n] = S
    return o.reshape(B, T, H, Dv), S_final


def kda_step(q, k, v, log_alpha, beta, S):
    """One decode token in matrix form; returns (o [N, H, Dv], new S) without mutating S."""
    q, k, v, g, b, S = (_as_f64(x) for x in (q, k, v, log_alpha, beta, S))
    Dk = q.shape[-1]
    erase = np.eye(Dk) - b[..., None, None] * k[..., :, None] * k[..., None, :]
    S_new = erase @ (np.exp(g)[..., :, None] * S) + b[..., None, None] * k[..., :, None] * v[..., None, :]
    o = np.einsum("nhcj,nhc->nhj", S_new, q)
    return o, S_new
