"""Plain fp64 definitions of the elementwise steps either side of the layer (the fused
prologue and epilogue), for the oracle checks of the fused entry points.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings.  The pages fix none of these maps; they state the properties the layer's inputs
have.  "Decoding Hybrid Attention Architectures" (intl.cloud.baidu.com article 9569726),
section 3.2, takes the keys as normalised and the update strength beta in (0, 1];
section 3.4 has a decay vector with entries in (0, 1).  The maps below are the plainest
ones that produce exactly those properties from unconstrained values:
  * q, k: L2 normalisation over the key channels, x / sqrt(sum x^2 + 1e-12);
  * beta: the logistic sigmoid of a logit;
  * log_alpha: logsigmoid(a + bias) / scale of a logit a (scale > 0), i.e. a decay
    alpha = sigmoid(a + bias)^(1/scale) in (0, 1);
  * output gate: o * sigmoid(gate), per value channel.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-12
QK_L2NORM, BETA_SIGMOID, DECAY_LOGSIGMOID = 1, 2, 4


def l2norm(x):
    """x / sqrt(sum over the last axis of x^2 + 1e-12), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow for any x."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def logsigmoid(x):
    """log(sigmoid(x)) = min(x, 0) - log1p(e^-|x|), without overflow for any x."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def prologue(q, k, beta, log_alpha, flags, decay_bias=0.0, decay_scale=1.0):
    """The layer's inputs from raw values under the given flags (fp64 arrays)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    log_alpha = np.asarray(log_alpha, dtype=np.float64)
    if flags & QK_L2NORM:
        q, k = l2norm(q), l2norm(k)
    if flags & BETA_SIGMOID:
        beta = sigmoid(beta)
    if flags & DECAY_LOGSIGMOID:
        log_alpha = logsigmoid(log_alpha + decay_bias) / decay_scale
    return q, k, beta, log_alpha


def out_gate(o, gate):
    """o * sigmoid(gate), elementwise."""
    return np.asarray(o, dtype=np.float64) * sigmoid(gate)


def fused_backward(q, k, v, a, b, gate, d_o, S0=None, cu_seqlens=None, dS_final=None, flags=0,
                   decay_bias=0.0, decay_scale=1.0, scalar_gate=False):
    """Gradient of the fused layer with respect to its raw inputs, in fp64.

    The fused layer is the plain one (the token recurrence of "Decoding Hybrid Attention
    Architectures", section 3.4) applied to prologue(q, k, b, a) above, with the output
    multiplied by sigmoid(gate) when gate is given; its outputs are that o and the final
    states.  Given the upstream gradients d_o (of the gated o) and dS_final, this returns
    dq, dk, dv, da (the decay logits, or log_alpha itself without the decay map), db (the
    beta logits, or beta), dgate (None without a gate) and dS0.  Each map's derivative is
    written out: for x' = x / n with n = sqrt(sum x^2 + eps), dx = (dx' - x' (x' . dx')) / n;
    for sigmoid s(b), db = dbeta s (1 - s); for logsigmoid(a + c) / scale,
    da = dlog_alpha (1 - s(a + c)) / scale; for o s(g), d(o) = d_o s(g) and
    dg = d_o o s(g) (1 - s(g)).  The layer's own gradient comes from kda_bwd, and the
    ungated o for dgate from kda_fwd.  scalar_gate: a holds one decay per (token, head),
    broadcast over the key channels (its gradient sums over them)."""
    from oracle import kda_bwd, kda_fwd
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    qn, kn, beta, la = prologue(q, k, b, a, flags, decay_bias, decay_scale)
    la_full = np.ascontiguousarray(np.broadcast_to(la[..., None], q.shape)) if scalar_gate else la
    d_core = d_o
    dgate = None
    if gate is not None:
        gate = np.asarray(gate, dtype=np.float64)
        s = sigmoid(gate)
        o_core, _ = kda_fwd(qn, kn, v, la_full, beta, S0=S0, cu_seqlens=cu_seqlens, o_dtype=np.float64)
        d_core = d_o * s
        dgate = d_o * o_core * s * (1.0 - s)
    g = kda_bwd(qn, kn, v, la_full, beta, d_core, S0=S0, cu_seqlens=cu_seqlens, dS_final=dS_final)
    dq, dk, dla, dbeta = g["dq"], g["dk"], g["dlog_alpha"], g["dbeta"]
    if scalar_gate:
        dla = dla.sum(axis=-1)
    if flags & QK_L2NORM:
        for x, dx, out in ((q, dq, "dq"), (k, dk, "dk")):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)
            xn = x / n
            g[out] = (dx - xn * np.sum(xn * dx, axis=-1, keepdims=True)) / n
        dq, dk = g["dq"], g["dk"]
    if flags & BETA_SIGMOID:
        s = sigmoid(b)
        dbeta = dbeta * s * (1.0 - s)
    if flags & DECAY_LOGSIGMOID:
        dla = dla * (1.0 - sigmoid(a + decay_bias)) / decay_scale
    return {"dq": dq, "dk": dk, "dv": g["dv"], "da": dla, "db": dbeta, "dgate": dgate, "dS0": g["dS0"]}
