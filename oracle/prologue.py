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
