"""CPU (numpy fp64) chunkwise gradient of the KDA layer -- a test artifact.

It is the algebraic model of the device backward, organised the same way, and the
tests check it against the oracle's token-by-token reverse mode (an independent
derivation).  The forward it differentiates is the chunkwise form of "Decoding
Hybrid Attention Architectures" (intl.cloud.baidu.com article 9569726), section 4,
written with midpoint-relative decays.  Per chunk of C tokens (a ragged tail chunk
is padded with zero q, k, v, beta and zero log-decay, which changes nothing), entry
state S, chunk-local cumulative log-decay b_r = sum_{i<=r} g_i and m = b at the
chunk's midpoint row:

  Q' = Q e^{b-m},  K' = K e^{b-m},  K'' = K e^{m-b},  e_m = e^{m},  e_n = e^{b_last - m}
  L = StrictTril(K' K''^T),  A = Diag(beta) L,  M = (I + A)^-1,  P = Tril(Q' K''^T)
  S_m = Diag(e_m) S,  R = V - K' S_m,  E = M Diag(beta) R
  O = Q' S_m + P E,   S_next = Diag(e_n) (S_m + K''^T E)

Gradients, given dO and dS_next (the gradient of everything after the chunk with
respect to its exit state), with dS_n = Diag(e_n) dS_next:

  dE = P^T dO + K'' dS_n,  dY = M^T dE,  dV = Diag(beta) dY
  dS (entry) = Diag(e_m) (dS_n + Q'^T dO - K'^T dV)
  dbeta = rowsum(dY * R) + rowsum(StrictTril(dA) * L),   dA = -dY E^T
  dL = Diag(beta) StrictTril(dA),  dP = Tril(dO E^T)
  dQ' = dO S_m^T + dP K'',   dK' = -dV S_m^T + dL K'',   dK'' = dP^T Q' + dL^T K' + E dS_n^T
  dq = e^{b-m} dQ',  dk = e^{b-m} dK' + e^{m-b} dK''
  db = Q' dQ' + K' dK' - K'' dK''  (elementwise), plus rowsum(dS_next * S_next) on the last row
  dlog_alpha = reverse cumulative sum of db within the chunk

The three passes are those of the device: a forward state pass that keeps every
chunk's entry state (and the final one), a reverse pass that carries dS from the
last chunk to the first and keeps every chunk's dS_next, and a per-chunk gradient
step that needs only its chunk's S, dS_next and S_next.
"""
from __future__ import annotations

import numpy as np


def _prep(Q, K, G, beta, C):
    b = np.cumsum(G, axis=0)
    m = b[C // 2 - 1]
    up, dn = np.exp(b - m), np.exp(m - b)
    Qp, Kp, Kpp = Q * up, K * up, K * dn
    L = np.tril(Kp @ Kpp.T, -1)
    M = np.linalg.inv(np.eye(C) + beta[:, None] * L)
    P = np.tril(Qp @ Kpp.T)
    return dict(b=b, m=m, up=up, dn=dn, Qp=Qp, Kp=Kp, Kpp=Kpp, L=L, M=M, P=P,
                em=np.exp(m), en=np.exp(b[-1] - m))


def chunk_bwd(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None, C=32):
    q, k, v, g, bt, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta, d_o))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        bounds = list(zip(cu[:-1], cu[1:]))
    flat = [x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g, bt, do)]
    out = dict(dq=np.zeros((B * T, H, Dk)), dk=np.zeros((B * T, H, Dk)), dv=np.zeros((B * T, H, Dv)),
               dlog_alpha=np.zeros((B * T, H, Dk)), dbeta=np.zeros((B * T, H)),
               dS0=np.zeros((len(bounds), H, Dk, Dv)))

    def padded(x, c0, t1, h):
        blk = x[c0:min(c0 + C, t1), h]
        pad = np.zeros((C,) + blk.shape[1:])
        pad[:blk.shape[0]] = blk
        return pad

    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            starts = list(range(t0, t1, C))
            ch = []
            for c0 in starts:
                Q, K, V, G, be, dO = (padded(x, c0, t1, h) for x in flat)
                p = _prep(Q, K, G, be, C)
                p.update(V=V, beta=be, dO=dO, c0=c0, nn=min(C, t1 - c0))
                ch.append(p)
            # forward state pass: entry state of every chunk, then the final state
            S = np.zeros((Dk, Dv)) if S0 is None else np.asarray(S0[n, h], dtype=np.float64).copy()
            states = [S]
            for p in ch:
                Sm = p["em"][:, None] * S
                E = p["M"] @ (p["beta"][:, None] * (p["V"] - p["Kp"] @ Sm))
                S = p["en"][:, None] * (Sm + p["Kpp"].T @ E)
                states.append(S)
            # reverse pass: dS_next of every chunk, then dS0
            dS = np.zeros((Dk, Dv)) if dS_final is None else np.asarray(dS_final[n, h], float).copy()
            dnext = [None] * len(ch)
            for c in range(len(ch) - 1, -1, -1):
                p = ch[c]
                dnext[c] = dS
                dSn = p["en"][:, None] * dS
                dE = p["P"].T @ p["dO"] + p["Kpp"] @ dSn
                dV = p["beta"][:, None] * (p["M"].T @ dE)
                dS = p["em"][:, None] * (dSn + p["Qp"].T @ p["dO"] - p["Kp"].T @ dV)
            out["dS0"][n, h] = dS
            # per-chunk gradients
            for c, p in enumerate(ch):
                Sm = p["em"][:, None] * states[c]
                dSn = p["en"][:, None] * dnext[c]
                R = p["V"] - p["Kp"] @ Sm
                E = p["M"] @ (p["beta"][:, None] * R)
                dE = p["P"].T @ p["dO"] + p["Kpp"] @ dSn
                dY = p["M"].T @ dE
                dV = p["beta"][:, None] * dY
                dA = np.tril(-dY @ E.T, -1)
                dbeta = np.sum(dY * R, axis=1) + np.sum(dA * p["L"], axis=1)
                dL = p["beta"][:, None] * dA
                dP = np.tril(p["dO"] @ E.T)
                dQp = p["dO"] @ Sm.T + dP @ p["Kpp"]
                dKp = -dV @ Sm.T + dL @ p["Kpp"]
                dKpp = dP.T @ p["Qp"] + dL.T @ p["Kp"] + E @ dSn.T
                db = p["Qp"] * dQp + p["Kp"] * dKp - p["Kpp"] * dKpp
                db[-1] += np.sum(dnext[c] * states[c + 1], axis=1)
                dg = np.cumsum(db[::-1], axis=0)[::-1]
                sl, nn = slice(p["c0"], p["c0"] + p["nn"]), p["nn"]
                out["dq"][sl, h] = (p["up"] * dQp)[:nn]
                out["dk"][sl, h] = (p["up"] * dKp + p["dn"] * dKpp)[:nn]
                out["dv"][sl, h] = dV[:nn]
                out["dlog_alpha"][sl, h] = dg[:nn]
                out["dbeta"][sl, h] = dbeta[:nn]
    for kk, shp in (("dq", (B, T, H, Dk)), ("dk", (B, T, H, Dk)), ("dv", (B, T, H, Dv)),
                    ("dlog_alpha", (B, T, H, Dk)), ("dbeta", (B, T, H))):
        out[kk] = out[kk].reshape(shp)
    return out
