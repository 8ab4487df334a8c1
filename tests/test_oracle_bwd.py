"""Pins for the oracle's gradient (CPU only).

The gradient of the layer is defined by the forward recurrence of "Decoding Hybrid
Attention Architectures" (intl.cloud.baidu.com article 9569726), section 3.4, and
the pages' training motivation (section 4) is what makes it part of the path.  The
oracle computes it by reverse mode over tokens; the pins below tie it to things
other than itself:

* central finite differences of the forward oracle (every input, equal-length and
  packed batches with an empty and a one-token sequence);
* homogeneity: o is linear in q, and (o, S_final) are jointly linear in (v, S0), so
  <dq, q> = <do, o> and <dv, v> + <dS0, S0> = <do, o> + <dS_final, S_final> exactly;
* the closed form at beta = 0 and alpha = 1 (plain linear read-out of S0);
* the chunkwise gradient model (tests/chunkwise_bwd_cpu.py), derived separately
  from the chunkwise form of section 4.

``test_planted_mistakes_are_caught`` plants mistakes in the gradient code and checks
that each fails at least one pin.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from chunkwise_bwd_cpu import chunk_bwd

GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def bcase(seed, B=2, T=7, H=2, Dk=4, Dv=3, lengths=None, s=2.0, beta=None, decay=True):
    rng = np.random.default_rng(seed)
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    z = rng.standard_normal((B, T, H, Dk))
    g = (np.minimum(z, 0) - np.log1p(np.exp(-np.abs(z)))) / s if decay else np.zeros((B, T, H, Dk))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H)))) if beta is None else np.full((B, T, H), beta)
    N = B if lengths is None else len(lengths)
    S0 = rng.standard_normal((N, H, Dk, Dv))
    do = rng.standard_normal((B, T, H, Dv))
    dsf = rng.standard_normal((N, H, Dk, Dv))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, log_alpha=g, beta=b, S0=S0, d_o=do, dS_final=dsf, cu_seqlens=cu)


def grads(c, lib=None):
    return oracle.kda_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["d_o"], S0=c["S0"],
                          cu_seqlens=c["cu_seqlens"], dS_final=c["dS_final"], lib=lib)


def loss(c):
    """<do, o> + <dS_final, S_final> with the forward oracle (the default library)."""
    o, Sf = oracle.kda_fwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], S0=c["S0"],
                           cu_seqlens=c["cu_seqlens"], o_dtype=np.float64)
    return float(np.sum(o * c["d_o"]) + np.sum(Sf * c["dS_final"]))


def relerr(x, ref):
    return float(np.max(np.abs(x - ref)) / max(1e-300, np.max(np.abs(ref))))


# ------------------------------------------------------------------ pins
def pin_finite_differences(lib=None):
    """Central differences (step 1e-6) of the forward oracle, every element of every input."""
    worst = 0.0
    h = 1e-6
    for c in (bcase(31), bcase(32, H=1, Dk=3, Dv=4, lengths=[3, 0, 1, 6])):
        G = grads(c, lib)
        for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                            ("beta", "dbeta"), ("S0", "dS0")):
            x = c[name]
            num = np.zeros_like(x)
            for i in np.ndindex(x.shape):
                keep = x[i]
                x[i] = keep + h
                lp = loss(c)
                x[i] = keep - h
                lm = loss(c)
                x[i] = keep
                num[i] = (lp - lm) / (2 * h)
            worst = max(worst, relerr(G[gname], num))
    return worst


def pin_homogeneity(lib=None):
    """o is linear in q; (o, S_final) are jointly linear in (v, S0)."""
    c = bcase(33, B=2, T=40, H=2, Dk=8, Dv=6)
    G = grads(c, lib)
    o, Sf = oracle.kda_fwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], S0=c["S0"],
                           o_dtype=np.float64)
    do_o = np.sum(c["d_o"] * o)
    lhs1 = np.sum(G["dq"] * c["q"])
    lhs2 = np.sum(G["dv"] * c["v"]) + np.sum(G["dS0"] * c["S0"])
    rhs2 = do_o + np.sum(c["dS_final"] * Sf)
    scale = max(abs(do_o), abs(rhs2), 1.0)
    return float(max(abs(lhs1 - do_o), abs(lhs2 - rhs2)) / scale)


def pin_linear_readout(lib=None):
    """beta = 0, alpha = 1: S_t = S0 for all t and o_t = S0^T q_t, so
    dq_t = S0 do_t, dv = 0, dS0 = dS_final + sum_t q_t do_t^T,
    dlog_alpha_t = sum_{t' >= t} q_t' * (S0 do_t') + rowsum(S0 * dS_final),
    dk_t = dS_t e_t + S' dr = 0 (e = 0, dr = 0), and
    dbeta_t = (dS_t^T k_t) . (v_t - S0^T k_t) with dS_t = dS_final + sum_{t' >= t} q_t' do_t'^T."""
    c = bcase(34, B=1, T=9, H=1, Dk=5, Dv=4, beta=0.0, decay=False)
    G = grads(c, lib)
    q, k, v, do = (c[x][0, :, 0] for x in ("q", "k", "v", "d_o"))
    S0, dsf = c["S0"][0, 0], c["dS_final"][0, 0]
    T = q.shape[0]
    worst = relerr(G["dq"][0, :, 0], do @ S0.T)
    worst = max(worst, float(np.max(np.abs(G["dv"]))), float(np.max(np.abs(G["dk"]))))
    worst = max(worst, relerr(G["dS0"][0, 0], dsf + q.T @ do))
    dla = np.zeros_like(q)
    db = np.zeros(T)
    for t in range(T):
        dla[t] = sum(q[u] * (S0 @ do[u]) for u in range(t, T)) + np.sum(S0 * dsf, axis=1)
        dSt = dsf + sum(np.outer(q[u], do[u]) for u in range(t, T))
        db[t] = (dSt.T @ k[t]) @ (v[t] - S0.T @ k[t])
    worst = max(worst, relerr(G["dlog_alpha"][0, :, 0], dla), relerr(G["dbeta"][0, :, 0], db))
    return worst


def pin_chunkwise_model(lib=None):
    """The chunkwise gradient (separate derivation, several chunk sizes, packed
    batches with an empty sequence and ragged tails) equals the oracle's."""
    worst = 0.0
    for c, C in ((bcase(35, B=2, T=45, H=2, Dk=8, Dv=6), 8),
                 (bcase(36, H=2, Dk=8, Dv=8, lengths=[5, 0, 17, 9, 40]), 16)):
        G = grads(c, lib)
        Cb = chunk_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["d_o"], S0=c["S0"],
                       cu_seqlens=c["cu_seqlens"], dS_final=c["dS_final"], C=C)
        worst = max(worst, max(relerr(G[g], Cb[g]) for g in GRADS))
    return worst


PINS = {
    "finite_differences": (pin_finite_differences, 1e-7),
    "homogeneity": (pin_homogeneity, 1e-12),
    "linear_readout": (pin_linear_readout, 1e-12),
    "chunkwise_model": (pin_chunkwise_model, 1e-11),
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    fn, bound = PINS[name]
    err = fn()
    assert err <= bound, f"pin {name}: {err} > {bound}"


def test_zero_length_sequences_and_no_tokens():
    c = bcase(37, H=2, Dk=4, Dv=4, lengths=[0, 4, 0])
    G = grads(c)
    np.testing.assert_array_equal(G["dS0"][0], c["dS_final"][0])
    np.testing.assert_array_equal(G["dS0"][2], c["dS_final"][2])
    c = bcase(38, B=3, T=0)
    G = grads(c)
    np.testing.assert_array_equal(G["dS0"], c["dS_final"])
    assert G["dq"].size == 0


def test_bf16_inputs_are_read_exactly():
    c = bcase(39, B=1, T=12, H=1, Dk=4, Dv=4)
    bits = {}
    for kk in ("q", "k", "v", "log_alpha", "beta", "d_o"):
        f = c[kk].astype(np.float32)
        u = f.view(np.uint32)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        bits[kk] = u
        c[kk] = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Gb = oracle.kda_bwd(bits["q"], bits["k"], bits["v"], bits["log_alpha"], bits["beta"], bits["d_o"],
                        S0=c["S0"], dS_final=c["dS_final"])
    Gf = grads(c)
    for g in GRADS:
        np.testing.assert_array_equal(Gb[g], Gf[g])


# ------------------------------------------------------------------ planted mistakes
MUTANTS = {
    "no_output_to_state": (
        "for (int j = 0; j < Dv; ++j) dS[(size_t)c * Dv + j] += qc * load_elem(d_o, do_dtype, vi + j);",
        "for (int j = 0; j < Dv; ++j) (void)qc;"),
    "dq_before_write": ("acc += (Sp[(size_t)c * Dv + j] + kc * e[j]) * load_elem(d_o, do_dtype, vi + j);",
                        "acc += Sp[(size_t)c * Dv + j] * load_elem(d_o, do_dtype, vi + j);"),
    "no_read_path_in_dk": ("        dk[xi + c] += acc;\n", "        (void)acc;\n"),
    "dr_sign": ("dr[j] = -bt * de[j];", "dr[j] = bt * de[j];"),
    "decay_grad_from_old_state": ("acc += dS[(size_t)c * Dv + j] * Sp[(size_t)c * Dv + j];",
                                  "acc += dS[(size_t)c * Dv + j] * Sprev[(size_t)c * Dv + j];"),
    "no_decay_of_state_grad": ("            dS[(size_t)c * Dv + j] *= a;\n", ""),
    "dbeta_without_erase": ("db += de[j] * (load_elem(v, in_dtype, vi + j) - r[j]);",
                            "db += de[j] * load_elem(v, in_dtype, vi + j);"),
}


def test_planted_mistakes_are_caught():
    src_path = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")
    src = open(src_path).read()
    tmp = tempfile.mkdtemp(prefix="oracle_bwd_mutants_")
    try:
        shutil.copy(os.path.join(os.path.dirname(src_path), "kda_oracle.h"), tmp)
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, f"mutant {name}: anchor text not unique in the oracle source"
            path = os.path.join(tmp, f"m_{name}.c")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            lib_path = os.path.join(tmp, f"libm_{name}.so")
            subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib_path, path, "-lm"],
                           check=True)
            lib = oracle.load_library(lib_path)
            failed = []
            for pname, (fn, bound) in PINS.items():
                with np.errstate(all="ignore"):
                    err = fn(lib)
                if not (err <= bound):
                    failed.append(pname)
            assert failed, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_scalar_gate_gradient_is_the_channel_sum():
    """A scalar gate is the per-channel rule with one log-decay broadcast over the key
    channels ("Decoding Hybrid Attention Architectures", section 3.3), so its gradient is
    the per-channel dlog_alpha summed over the channels: checked against central
    differences in the scalar log-decay."""
    c = bcase(40, B=1, T=9, H=2, Dk=4, Dv=3)
    gs = c["log_alpha"][..., 0].copy()                       # [B, T, H]
    c["log_alpha"] = np.ascontiguousarray(np.broadcast_to(gs[..., None], c["q"].shape))
    want = grads(c)["dlog_alpha"].sum(axis=-1)
    num = np.zeros_like(gs)
    h = 1e-6
    for i in np.ndindex(gs.shape):
        for sign in (1, -1):
            x = gs.copy()
            x[i] += sign * h
            c["log_alpha"] = np.ascontiguousarray(np.broadcast_to(x[..., None], c["q"].shape))
            num[i] += sign * loss(c) / (2 * h)
    assert relerr(want, num) < 1e-7
