"""Backward parity on the GPU: kda_chunk_bwd (HIP, through the C ABI) vs the oracle's
exact gradient (fp64 reverse mode over tokens) on the same seeded inputs.

Shapes span several chunks and ragged tails, packed batches with empty and one-token
sequences, both head sizes, both input dtypes, fast-decay mixtures, calls without an
initial state or a final-state gradient, and the training-prefill workload at full
size (4 x 4096 tokens, 16 heads; the oracle checks two of the heads).  The forward
being differentiated is the chunkwise KDA layer of "Decoding Hybrid Attention
Architectures" (intl.cloud.baidu.com article 9569726), sections 3.4 and 4.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_delta_rule_62_amd import inputs
from gpu_util import TOL_BF16, TOL_F32, o_metric, state_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS
GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def gpu_bwd(d, g, grad_dtype=torch.float32, want_dS0=True):
    kda = _kda()
    fn = kda.gdn_chunk_bwd if d.get("scalar_gate") else kda.kda_chunk_bwd
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    cu = to_dev(d["cu_seqlens"]) if d["cu_seqlens"] is not None else None
    dsf = to_dev(g["dS_final"]) if g["dS_final"] is not None else None
    out = fn(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], to_dev(g["d_o"]),
             S0, cu, dsf, grad_dtype=grad_dtype, want_dS0=want_dS0)
    torch.cuda.synchronize()
    return {kk: to_host(t) for kk, t in out.items() if t is not None}


def oracle_bwd(d, g, heads=None):
    """The oracle's gradient.  A scalar gate is the per-channel rule with the decay
    broadcast over the key channels, so its dlog_alpha is the per-channel one summed over
    them (the chain rule through the broadcast)."""
    sel = slice(None) if heads is None else heads
    args = [d[kk][:, :, sel] for kk in ("q", "k", "v", "log_alpha", "beta")]
    if d.get("scalar_gate"):
        la = inputs.to_float(args[3]).astype(np.float64)
        args[3] = np.ascontiguousarray(np.broadcast_to(la[..., None], args[0].shape))
        args = [inputs.to_float(x).astype(np.float64) for x in args[:3]] + [args[3]] + \
            [inputs.to_float(args[4]).astype(np.float64)]
    S0 = None if d["S0"] is None else d["S0"][:, sel]
    dsf = None if g["dS_final"] is None else g["dS_final"][:, sel]
    do = g["d_o"][:, :, sel]
    if d.get("scalar_gate"):
        do = inputs.to_float(do).astype(np.float64)
    out = oracle.kda_bwd(*args, do, S0=S0, cu_seqlens=d["cu_seqlens"], dS_final=dsf)
    if d.get("scalar_gate"):
        out["dlog_alpha"] = out["dlog_alpha"].sum(axis=-1)
    return out


def metrics(got, ref, cu, heads=None):
    sel = slice(None) if heads is None else heads
    err = {}
    for name in ("dq", "dk", "dv", "dlog_alpha"):
        x, y = got[name][:, :, sel], ref[name]
        if x.ndim == 3:   # scalar-gate dlog_alpha [B, T, H]
            x, y = x[..., None], y[..., None]
        err[name] = o_metric(x, y, cu)
    err["dbeta"] = o_metric(got["dbeta"][:, :, sel, None], ref["dbeta"][..., None], cu)
    if "dS0" in got:
        err["dS0"] = state_metric(got["dS0"][:, sel], ref["dS0"])
    return err


def check(d, g, label, heads=None, tol=None):
    print(f"[backward] {label}: B={d['B']} T={d['T']} H={d['H']} D={d['D']} N={d['N']} dtype={d['dtype']} "
          f"S0={'yes' if d['S0'] is not None else 'no'} dS_final={'yes' if g['dS_final'] is not None else 'no'}",
          flush=True)
    got = gpu_bwd(d, g)
    ref = oracle_bwd(d, g, heads)
    for name, x in got.items():
        assert np.all(np.isfinite(x)), f"{name} has non-finite values"
    err = metrics(got, ref, d["cu_seqlens"], heads)
    tol = tol if tol is not None else (TOL_F32 if d["dtype"] == "f32" else TOL_BF16)
    print("[backward]   " + "  ".join(f"{kk} {vv:.2e}" for kk, vv in err.items()) + f"  (tol {tol})", flush=True)
    for name, e in err.items():
        assert e <= tol, f"{label}: {name} error {e:.3e} > {tol}"
    return err


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_ragged_with_state(D):
    d = inputs.make_prefill(W[0], seed=101, B=2, T=45, H=2, D=D, s0=True, mu=0.0, s=2.0)
    check(d, inputs.make_output_grads(d, seed=201), f"fp32 ragged D={D}")


def test_fp32_several_chunks_d128():
    d = inputs.make_prefill(W[0], seed=102, B=1, T=200, H=3, D=128, s0=True)
    check(d, inputs.make_output_grads(d, seed=202), "fp32 several chunks")


@pytest.mark.parametrize("D", [64, 128])
def test_packed_with_empty_and_one_token_sequences(D):
    d = inputs.make_prefill(W[1], seed=103, H=2, D=D, s0=True, lengths=[5, 0, 70, 33, 1, 64, 0])
    check(d, inputs.make_output_grads(d, seed=203), f"packed D={D}")


def test_no_initial_state_and_no_final_state_gradient():
    d = inputs.make_prefill(W[1], seed=104, B=2, T=77, H=2, D=128, s0=False)
    g = inputs.make_output_grads(d, seed=204, dS_final=False)
    check(d, g, "no S0, no dS_final")


def test_fast_decay_mixture_packed():
    d = inputs.make_prefill(W[4], seed=105, H=2, lengths=[200, 37, 129])
    check(d, inputs.make_output_grads(d, seed=205), "mixture decay")


def test_long_context_decay_recipe():
    d = inputs.make_prefill(W[2], seed=106, B=1, T=700, H=2)
    check(d, inputs.make_output_grads(d, seed=206), "long-context recipe, T=700")


def test_bf16_gradients_are_rne_of_fp32_gradients():
    d = inputs.make_prefill(W[1], seed=107, B=1, T=96, H=2, D=128, s0=True)
    g = inputs.make_output_grads(d, seed=207)
    g32 = gpu_bwd(d, g, grad_dtype=torch.float32)
    g16 = gpu_bwd(d, g, grad_dtype=torch.bfloat16)
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        want = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(g32[name]))
        np.testing.assert_array_equal(g16[name], want, err_msg=name)
    np.testing.assert_array_equal(g16["dS0"], g32["dS0"])


def test_run_to_run_bitwise_deterministic():
    d = inputs.make_prefill(W[1], seed=108, H=2, D=128, s0=True, lengths=[90, 3, 41])
    g = inputs.make_output_grads(d, seed=208)
    a, b = gpu_bwd(d, g), gpu_bwd(d, g)
    for name in GRADS:
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_zero_tokens_and_empty_sequences():
    d = inputs.make_prefill(W[1], seed=109, H=2, D=64, s0=True, lengths=[0, 0])
    g = inputs.make_output_grads(d, seed=209)
    got = gpu_bwd(d, g)
    np.testing.assert_array_equal(got["dS0"], g["dS_final"])
    # equal-length batch with no tokens: dS0 = dS_final, and zeros without dS_final
    d = inputs.make_prefill(W[1], seed=110, B=3, T=0, H=2, D=128, s0=True)
    g = inputs.make_output_grads(d, seed=210)
    got = gpu_bwd(d, g)
    np.testing.assert_array_equal(got["dS0"], g["dS_final"])
    g["dS_final"] = None
    got = gpu_bwd(d, g)
    assert not np.any(got["dS0"])


def test_full_size_train_prefill_sampled_heads():
    """Training prefill at full size: B=4 sequences of 4096 tokens, 16 heads, d=128,
    bf16; the oracle checks heads 0 and 11 of every sequence."""
    d = inputs.make_prefill(W[1])
    g = inputs.make_output_grads(d, seed=210)
    check(d, g, "train prefill full size", heads=[0, 11])


def test_matches_forward_directional_derivative():
    """<grad, delta> equals the central difference of the library's own forward along
    a random direction delta of every input (fp32, steps 1e-2 and 5e-3 with Richardson
    extrapolation; this ties the backward to the forward kernels, the oracle ties both
    to the definition)."""
    kda = _kda()
    d = inputs.make_prefill(W[0], seed=111, B=1, T=100, H=2, D=64, s0=True, mu=0.0, s=4.0)
    g = inputs.make_output_grads(d, seed=211)
    rng = np.random.default_rng(311)
    names = ("q", "k", "v", "log_alpha", "beta")
    delta = {kk: rng.standard_normal(d[kk].shape).astype(np.float32) for kk in names}
    delta["S0"] = rng.standard_normal(d["S0"].shape).astype(np.float32)
    do = to_dev(g["d_o"]).double()
    dsf = to_dev(g["dS_final"]).double()

    def loss(eps):
        x = {kk: to_dev(d[kk].astype(np.float64) + eps * delta[kk]) for kk in names + ("S0",)}
        o, Sf = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"], None)
        return float((o.double() * do).sum() + (Sf.double() * dsf).sum())

    got = gpu_bwd(d, g)
    gname = dict(q="dq", k="dk", v="dv", log_alpha="dlog_alpha", beta="dbeta", S0="dS0")
    want = sum(float(np.sum(got[gname[kk]].astype(np.float64) * delta[kk])) for kk in gname)
    h = 1e-2
    fd1 = (loss(h) - loss(-h)) / (2 * h)
    fd2 = (loss(h / 2) - loss(-h / 2)) / h
    fd = (4 * fd2 - fd1) / 3        # Richardson: removes the h^2 term of the central difference
    print(f"[backward] directional derivative: grad {want:.6f}  central differences {fd1:.6f} {fd2:.6f} "
          f"extrapolated {fd:.6f}", flush=True)
    assert abs(want - fd) <= 1e-3 * max(1.0, abs(fd))


# ------------------------------------------------------------------ windowed plan (memory control)
WINDOW_CASES = [   # (label, make_prefill overrides, limit in bytes, expected windows of W chunks)
    ("bf16 d128 ragged", dict(w=1, B=2, T=1000, H=2, s0=True), 4 << 20, (4, 8)),
    ("fp32 d64 ragged", dict(w=0, B=2, T=1000, H=3, D=64, s0=True), 3 << 20, None),
    ("bf16 d128 two windows", dict(w=2, B=1, T=2000, H=2, s0=True), 20 << 20, None),
    ("bf16 d128 no S0", dict(w=1, B=2, T=1500, H=2, s0=False), 8 << 20, None),
    ("bf16 d64 scalar gate", dict(w=1, B=2, T=700, H=2, D=64, s0=True, scalar_gate=True), 2 << 20, None),
    ("fp32 d128 scalar gate", dict(w=0, B=1, T=900, H=2, D=128, s0=True, scalar_gate=True), 6 << 20, None),
]


@pytest.mark.parametrize("label,kw,limit,win", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_windowed_backward(label, kw, limit, win, monkeypatch):
    """Past the workspace limit an equal-length backward runs window by window (a forward sweep
    keeps each window's entry state, then the windows run from last to first, each carrying the
    state gradient to the one before).  fp32 inputs: the checkpoints come from the backward's own
    forward state pass, so every chunk's arithmetic is that of the one-pass plan and the gradients
    are bitwise equal to it.  bf16 inputs: where their scratch fits, the checkpoints come from
    the prefill's segment summaries and combine, whose fp32 rounding differs; then the gradients
    agree with the one-pass plan to 1e-4 of each tensor's largest magnitude.  Both are checked
    against the oracle to the parity bound."""
    kda = _kda()
    kw = dict(kw)
    w = W[kw.pop("w")]
    d = inputs.make_prefill(w, seed=241, **kw)
    g = inputs.make_output_grads(d, seed=242)
    B, T, H, D = d["B"], d["T"], d["H"], d["D"]
    one = kda.kda_chunk_bwd_workspace_bytes(B, T, H, D, D, B, False)
    print(f"[backward] windowed {label}: B={B} T={T} H={H} D={D}, limit {limit}", flush=True)
    ref_one = gpu_bwd(d, g)
    monkeypatch.setenv("KDA_BWD_WORKSPACE_LIMIT", str(limit))
    ws = kda.kda_chunk_bwd_workspace_bytes(B, T, H, D, D, B, False)
    assert ws < one
    if win is not None:   # W chunks per window, n windows: W + 1 states and n - 1 checkpoints
        Wc, n = win
        assert (T + 31) // 32 > Wc * (n - 1)
    got = gpu_bwd(d, g)
    for name in ref_one:
        if w.dtype == "f32":
            assert np.array_equal(got[name], ref_one[name]), f"{label}: {name} differs from the one-pass plan"
        else:
            scale = max(float(np.abs(ref_one[name]).max()), 1e-30)
            err = float(np.abs(got[name].astype(np.float64) - ref_one[name]).max()) / scale
            assert err <= 1e-4, f"{label}: {name} differs from the one-pass plan by {err:.3g}"
    check(d, g, f"windowed {label}")
    monkeypatch.delenv("KDA_BWD_WORKSPACE_LIMIT")


def test_long_context_full_size_windowed_sampled_head():
    """Long-context workload at full size (B=1, T=65536, H=32, d=128, bf16, S0 != 0): the
    default plan runs 6 windows of 342 chunks in a 2.13 GB workspace (one pass would take 12.7
    GB); head 9 against the oracle's gradient."""
    kda = _kda()
    x = inputs.device_prefill(W[2])
    g = inputs.device_output_grads(x, seed=213)
    B, T, H, D = x["B"], x["T"], x["H"], x["D"]
    assert kda.kda_chunk_bwd_workspace_bytes(B, T, H, D, D, 1, False) <= 2 << 30
    print(f"[backward] long context full size, windowed: T={T} H={H}", flush=True)
    gr = kda.kda_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], g["d_o"], x["S0"], None,
                           g["dS_final"])
    torch.cuda.synchronize()
    h = [9]
    from gated_delta_rule_62_amd.inputs import host_bits
    args = [host_bits(x[kk][:, :, h]) for kk in ("q", "k", "v", "log_alpha", "beta")]
    ref = oracle.kda_bwd(*args, host_bits(g["d_o"][:, :, h]), S0=x["S0"][:, h].cpu().numpy(), cu_seqlens=None,
                         dS_final=g["dS_final"][:, h].cpu().numpy())
    got = {kk: to_host(t[:, :, h]) if kk != "dS0" else to_host(t[:, h]) for kk, t in gr.items()}
    err = {}
    for name in ("dq", "dk", "dv", "dlog_alpha"):
        err[name] = o_metric(got[name], ref[name])
    err["dbeta"] = o_metric(got["dbeta"][..., None], ref["dbeta"][..., None])
    err["dS0"] = state_metric(got["dS0"], ref["dS0"])
    print("[backward]   head 9: " + "  ".join(f"{kk} {vv:.2e}" for kk, vv in err.items()), flush=True)
    for name, e in err.items():
        assert e <= TOL_BF16, f"{name} error {e:.3e}"


# ------------------------------------------------------------------ scalar gate (gdn_chunk_bwd)
@pytest.mark.parametrize("D", [64, 128])
def test_scalar_gate_fp32_ragged(D):
    d = inputs.make_prefill(W[0], seed=121, B=2, T=45, H=2, D=D, s0=True, mu=0.0, s=2.0, scalar_gate=True)
    check(d, inputs.make_output_grads(d, seed=221), f"scalar gate fp32 ragged D={D}")


def test_scalar_gate_packed_long_context_recipe():
    d = inputs.make_prefill(W[6], seed=122, H=2, lengths=[300, 0, 41, 1, 96])
    check(d, inputs.make_output_grads(d, seed=222), "scalar gate packed, long-context recipe")


def test_long_context_full_size_identities():
    """Long-context workload at full size (B=1, T=65536, H=32, d=128, bf16, S0 != 0), where
    the oracle would take hours: properties that hold at any size.  o is linear in q, and
    (o, S_final) are jointly linear in (v, S0), so with this library's forward outputs
    <dq, q> = <dO, o> and <dv, v> + <dS0, S0> = <dO, o> + <dS_final, S_final> (per head,
    fp64 sums of the fp32 results)."""
    kda = _kda()
    x = inputs.device_prefill(W[2])
    g = inputs.device_output_grads(x, seed=212)
    print(f"[backward] long context full size: T={x['T']} H={x['H']}", flush=True)
    o, Sf = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"], None,
                              out_dtype=torch.float32)
    gr = kda.kda_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], g["d_o"], x["S0"], None,
                           g["dS_final"])
    torch.cuda.synchronize()
    f64 = lambda t: t.double()
    dims = (0, 1, 3)   # sum over batch, tokens, channels: one value per head
    do_o = (f64(g["d_o"]) * f64(o)).sum(dim=dims)
    lhs1 = (f64(gr["dq"]) * f64(x["q"])).sum(dim=dims)
    lhs2 = (f64(gr["dv"]) * f64(x["v"])).sum(dim=dims) + (f64(gr["dS0"]) * f64(x["S0"])).sum(dim=(0, 2, 3))
    rhs2 = do_o + (f64(g["dS_final"]) * f64(Sf)).sum(dim=(0, 2, 3))
    scale1 = (f64(g["d_o"]).abs() * f64(o).abs()).sum(dim=dims)
    scale2 = scale1 + (f64(g["dS_final"]).abs() * f64(Sf).abs()).sum(dim=(0, 2, 3))
    e1 = ((lhs1 - do_o).abs() / scale1).max().item()
    e2 = ((lhs2 - rhs2).abs() / scale2).max().item()
    print(f"[backward]   identity errors (relative to the sum of |terms|): q {e1:.2e}  v,S0 {e2:.2e}", flush=True)
    for t in gr.values():
        assert torch.isfinite(t).all()
    assert e1 < 1e-4 and e2 < 1e-4


def test_chunk_64_forward_gets_the_same_gradient():
    """kda_chunk_bwd for a forward run with 64-token chunks: the layer, and so its gradient, does
    not depend on the chunk length, and the backward evaluates it with 32-token chunks, so the
    result equals the chunk-32 call bit for bit (and the oracle within the bound)."""
    kda = _kda()
    d = inputs.make_prefill(W[1], seed=251, B=2, T=300, H=2, s0=True)
    g = inputs.make_output_grads(d, seed=252)
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    args = (dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], to_dev(g["d_o"]), to_dev(d["S0"]), None,
            to_dev(g["dS_final"]))
    a = kda.kda_chunk_bwd(*args, chunk=32)
    b = kda.kda_chunk_bwd(*args, chunk=64)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name
    check(d, g, "chunk 64 forward")
