"""Pins for the oracle's fused prologue / epilogue definitions (oracle/prologue.py), on the
CPU.  Each map is checked against a library routine or a closed form, so that a dropped
term, a wrong sign or a swapped argument fails here:

  * l2norm: unit norm, scale invariance, direction preserved, the epsilon's effect on 0;
  * sigmoid: scipy.special.expit, the symmetry s(x) + s(-x) = 1, s(0) = 1/2, no overflow;
  * logsigmoid: scipy.special.log_expit, log(2) at 0, the asymptotes x and -e^-x;
  * prologue: flags applied one at a time and together, decays in (0, 1);
  * out_gate: o * sigmoid(g), o / 2 at g = 0;
  * fused_backward: directional derivatives of the fused layer's loss
    sum(d_o * o) + sum(dS_final * S_final) by central differences (Richardson-extrapolated),
    for every raw input, with all maps on, with none (where it must equal kda_bwd), for the
    scalar gate and for packed sequences.
The input recipe's own helpers (a separate implementation in the input generator) agree.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy import special

from oracle import prologue as P
from gated_delta_rule_62_amd import inputs


def test_l2norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7, 128)) * 3.0
    y = P.l2norm(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-12)
    assert np.allclose(P.l2norm(17.5 * x), y, atol=1e-14)
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    assert np.allclose(cos, 1.0, atol=1e-12)
    assert np.array_equal(P.l2norm(np.zeros((3, 8))), np.zeros((3, 8)))
    # epsilon under the root: a tiny vector is shrunk, not blown up
    t = np.full((1, 4), 1e-8)
    assert np.all(P.l2norm(t) < 0.5)


def test_sigmoid():
    x = np.concatenate([np.linspace(-40, 40, 2001), [-800.0, 800.0, 0.0]])
    s = P.sigmoid(x)
    assert np.allclose(s, special.expit(x), rtol=1e-15, atol=0)
    assert np.allclose(s + P.sigmoid(-x), 1.0, atol=1e-15)
    assert P.sigmoid(0.0) == 0.5
    assert P.sigmoid(800.0) == 1.0 and P.sigmoid(-800.0) == 0.0


def test_logsigmoid():
    x = np.linspace(-60, 60, 2401)
    assert np.allclose(P.logsigmoid(x), special.log_expit(x), rtol=1e-13, atol=1e-300)
    assert abs(P.logsigmoid(0.0) + np.log(2.0)) < 1e-16
    assert P.logsigmoid(-800.0) == -800.0                   # asymptote x for x -> -inf
    assert abs(P.logsigmoid(30.0) + np.exp(-30.0)) < 1e-25  # asymptote -e^-x for x -> inf
    assert np.all(P.logsigmoid(x) < 0.0)


def test_prologue_flags():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 3, 2, 16)) * 2.0, rng.standard_normal((2, 3, 2, 16)) * 2.0
    b, g = rng.standard_normal((2, 3, 2)), rng.standard_normal((2, 3, 2, 16))
    same = P.prologue(q, k, b, g, 0)
    for a, r in zip(same, (q, k, b, g)):
        assert np.array_equal(a, r)
    qn, kn, bn, gn = P.prologue(q, k, b, g, P.QK_L2NORM)
    assert np.allclose(qn, P.l2norm(q)) and np.allclose(kn, P.l2norm(k)) and np.array_equal(bn, b)
    _, _, bs, _ = P.prologue(q, k, b, g, P.BETA_SIGMOID)
    assert np.all((bs > 0) & (bs < 1)) and np.allclose(bs, special.expit(b))
    _, _, _, gl = P.prologue(q, k, b, g, P.DECAY_LOGSIGMOID, decay_bias=4.0, decay_scale=8.0)
    assert np.allclose(gl, special.log_expit(g + 4.0) / 8.0)
    a = np.exp(gl)
    assert np.all((a > 0) & (a < 1))


def test_out_gate():
    rng = np.random.default_rng(3)
    o, gt = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    assert np.allclose(P.out_gate(o, gt), o * special.expit(gt))
    assert np.allclose(P.out_gate(o, np.zeros_like(o)), o / 2)


def test_agrees_with_input_recipe():
    """The workloads' recipe draws L2-normalised q, k, sigmoid betas and logsigmoid decays
    with its own helpers; the oracle's maps give the same values from the same raw draws."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal((3, 5, 2, 64), dtype=np.float32)
    assert np.allclose(inputs._l2n(z), P.l2norm(z), atol=2e-7)
    assert np.allclose(inputs._sigmoid(z), P.sigmoid(z), atol=1e-7)
    assert np.allclose(inputs._logsigmoid(z + np.float32(4)) / np.float32(8),
                       P.logsigmoid(z.astype(np.float64) + 4) / 8, atol=1e-7)


def _fd_check(rng, flags, gate_on, scalar_gate=False, cu=None, bias=2.0, scale=4.0, B=1, T=20, H=2, D=8):
    """Compare fused_backward with central differences of the loss along a random direction
    in each raw input."""
    import oracle
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    a = rng.standard_normal((B, T, H) if scalar_gate else (B, T, H, D))
    b = rng.standard_normal((B, T, H))
    gate = rng.standard_normal((B, T, H, D)) if gate_on else None
    N = B if cu is None else len(cu) - 1
    S0 = 0.1 * rng.standard_normal((N, H, D, D))
    dO = rng.standard_normal((B, T, H, D))
    dSf = 0.1 * rng.standard_normal((N, H, D, D))
    g = P.fused_backward(q, k, v, a, b, gate, dO, S0=S0, cu_seqlens=cu, dS_final=dSf, flags=flags,
                         decay_bias=bias, decay_scale=scale, scalar_gate=scalar_gate)

    def loss(q, k, v, a, b, gate, S0):
        qn, kn, beta, la = P.prologue(q, k, b, a, flags, bias, scale)
        if scalar_gate:
            la = np.ascontiguousarray(np.broadcast_to(la[..., None], q.shape))
        o, Sf = oracle.kda_fwd(qn, kn, v, la, beta, S0=S0, cu_seqlens=cu, o_dtype=np.float64)
        if gate is not None:
            o = P.out_gate(o, gate)
        return np.sum(dO * o) + np.sum(dSf * Sf)

    args = dict(q=q, k=k, v=v, a=a, b=b, gate=gate, S0=S0)
    names = {"q": "dq", "k": "dk", "v": "dv", "a": "da", "b": "db", "gate": "dgate", "S0": "dS0"}
    for nm, gn in names.items():
        if args[nm] is None:
            assert g[gn] is None
            continue
        d = rng.standard_normal(args[nm].shape)

        def f(h):
            a2 = dict(args)
            a2[nm] = args[nm] + h * d
            return loss(**a2)
        h = 1e-4
        fd1 = (f(h) - f(-h)) / (2 * h)
        fd2 = (f(h / 2) - f(-h / 2)) / h
        fd = (4 * fd2 - fd1) / 3
        want = float(np.sum(g[gn] * d))
        assert abs(want - fd) <= 1e-8 * max(1.0, abs(fd)), (nm, want, fd)
    return g


def test_fused_backward_all_maps_and_gate():
    _fd_check(np.random.default_rng(11), P.QK_L2NORM | P.BETA_SIGMOID | P.DECAY_LOGSIGMOID, True)


def test_fused_backward_maps_one_at_a_time():
    rng = np.random.default_rng(12)
    for flags in (P.QK_L2NORM, P.BETA_SIGMOID, P.DECAY_LOGSIGMOID):
        _fd_check(rng, flags, False)


def test_fused_backward_scalar_gate_and_packed():
    rng = np.random.default_rng(13)
    _fd_check(rng, 7, True, scalar_gate=True)
    _fd_check(rng, 7, True, cu=np.array([0, 7, 7, 20], dtype=np.int32))


def test_fused_backward_without_maps_is_the_plain_gradient():
    """With no map and no gate the fused gradient is kda_bwd's, term for term."""
    import oracle
    rng = np.random.default_rng(14)
    B, T, H, D = 1, 17, 2, 8
    q, k, v, a = (rng.standard_normal((B, T, H, D)) for _ in range(4))
    a = -np.abs(a) * 0.1
    b = rng.uniform(0.1, 0.9, (B, T, H))
    dO = rng.standard_normal((B, T, H, D))
    g = P.fused_backward(q, k, v, a, b, None, dO, flags=0)
    r = oracle.kda_bwd(q, k, v, a, b, dO)
    for x, y in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("da", "dlog_alpha"), ("db", "dbeta")):
        assert np.array_equal(g[x], r[y]), x
