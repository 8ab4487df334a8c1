"""Fused prologue / epilogue on the GPU: kda_chunk_fwd_fused and kda_recurrent_step_fused,
and their scalar-gate forms gdn_chunk_fwd_fused and gdn_recurrent_step_fused (HIP, through the
C ABI), vs the fp64 oracle applied to the oracle's own prologue maps (oracle/prologue.py:
L2-normalised q and k, sigmoid beta, logsigmoid decay, sigmoid output gate; a scalar decay is
broadcast over the key channels).  Raw inputs are unnormalised keys and queries and N(0,1)
logits.  Cases: every flag alone and all together, both head sizes and input dtypes, the
segmented two-pass path, packed sequences with empty members (one batch cut into segments per
sequence), short batches, decode steps, and the no-flag call matching the plain entry point bit
for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle import prologue as P
from gated_delta_rule_62_amd import inputs
from gpu_util import TOL_BF16, TOL_F32, o_metric, state_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "log_alpha", "beta")
BIAS, SCALE = 4.0, 8.0


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def flags_of(qk, beta, decay):
    return (P.QK_L2NORM if qk else 0) | (P.BETA_SIGMOID if beta else 0) | (P.DECAY_LOGSIGMOID if decay else 0)


def run(d, flags, gate, chunk=0, recurrent=False):
    """GPU call; inputs a flag does not transform are given already transformed (fp32/bf16 of
    the same map), so every case exercises exactly its flags."""
    kda = _kda()
    f = {kk: inputs.to_float(d[kk]) for kk in KEYS}
    if not flags & P.DECAY_LOGSIGMOID:
        f["log_alpha"] = P.logsigmoid(f["log_alpha"]).astype(np.float32)
    if not flags & P.BETA_SIGMOID:
        f["beta"] = P.sigmoid(f["beta"]).astype(np.float32)
    if not flags & P.QK_L2NORM:
        # unnormalised keys make the recurrence blow up: give them normalised
        f["q"], f["k"] = P.l2norm(f["q"]).astype(np.float32), P.l2norm(f["k"]).astype(np.float32)
    cast = (lambda x: inputs.f32_to_bf16_bits(x)) if d["dtype"] == "bf16" else (lambda x: x.astype(np.float32))
    dev = {kk: to_dev(cast(f[kk])) for kk in KEYS}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    cu = to_dev(d["cu_seqlens"]) if d["cu_seqlens"] is not None else None
    kw = dict(qk_l2norm=bool(flags & P.QK_L2NORM), beta_logits=bool(flags & P.BETA_SIGMOID),
              decay_logits=(BIAS, SCALE) if flags & P.DECAY_LOGSIGMOID else None,
              out_gate=to_dev(d["gate"]) if gate else None, out_dtype=torch.float32)
    if recurrent:
        fn = kda.gdn_recurrent_fwd_fused if d.get("scalar_gate") else kda.kda_recurrent_fwd_fused
    else:
        fn = kda.gdn_chunk_fwd_fused if d.get("scalar_gate") else kda.kda_chunk_fwd_fused
        kw["chunk"] = chunk
    o, Sf = fn(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, cu, **kw)
    torch.cuda.synchronize()
    # the reference must see the same (rounded) inputs the GPU saw
    d2 = dict(d, **{kk: cast(f[kk]) for kk in KEYS})
    return to_host(o), to_host(Sf), d2


def check(d, flags, gate, label, recurrent=False):
    print(f"[fused] {label}: flags={flags} gate={gate} B={d['B']} T={d['T']} H={d['H']} D={d['D']} "
          f"dtype={d['dtype']} scalar_gate={bool(d.get('scalar_gate'))} recurrent={recurrent}", flush=True)
    o, Sf, d2 = run(d, flags, gate, recurrent=recurrent)
    # the reference reads the raw values of the transformed inputs, the transformed values of the rest
    o_ref, S_ref = reference_seen(d2, flags, gate)
    eo, es = o_metric(o, o_ref, d["cu_seqlens"]), state_metric(Sf, S_ref)
    tol = TOL_F32 if d["dtype"] == "f32" else TOL_BF16
    print(f"[fused]   worst o {eo:.3e}  S_final {es:.3e}  (tol {tol})", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    assert eo <= tol and es <= tol


def reference_seen(d2, flags, gate):
    """Oracle on exactly the buffers the GPU read: flagged inputs are raw, the others final."""
    f = [inputs.to_float(d2[kk]).astype(np.float64) for kk in KEYS]
    q, k, beta, g = P.prologue(f[0], f[1], f[4], f[3], flags, BIAS, SCALE)
    if d2.get("scalar_gate"):   # one decay per token and head, the same for every key channel
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], q.shape))
    o, S = oracle.kda_fwd(q, k, f[2], g, beta, S0=d2["S0"], cu_seqlens=d2["cu_seqlens"], o_dtype=np.float64)
    if gate:
        o = P.out_gate(o, inputs.to_float(d2["gate"]))
    return o, S


ALL = flags_of(True, True, True)


@pytest.mark.parametrize("flags,gate", [(ALL, True), (flags_of(True, False, False), False),
                                        (flags_of(False, True, False), False), (flags_of(False, False, True), False),
                                        (0, True)])
def test_each_flag_and_all(flags, gate):
    d = inputs.make_raw_prefill(701, B=2, T=300, H=2, D=128)
    check(d, flags, gate, "ragged")


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "f32")])
def test_head_sizes_and_dtypes(D, dtype):
    d = inputs.make_raw_prefill(702, B=1, T=200, H=2, D=D, dtype=dtype)
    check(d, ALL, True, f"D={D} {dtype}")


def test_segmented_two_pass_path():
    kda = _kda()
    assert kda.kda_chunk_fwd_workspace_bytes(1, 1000, 2, 128, 128, 1, False) > 0
    d = inputs.make_raw_prefill(703, B=1, T=1000, H=2, D=128)
    check(d, ALL, True, "segmented")


@pytest.mark.parametrize("sg", [False, True])
def test_chunk_64_is_evaluated_with_32_token_chunks(sg):
    """The fused maps run on the 32-token kernel: a 64-token request gives the 32-token call's
    outputs bit for bit (equal-length segmented and packed batches), and both are within the
    parity bound of the oracle."""
    for d, label in ((inputs.make_raw_prefill(713, B=1, T=1000, H=2, D=128, scalar_gate=sg), "segmented"),
                     (inputs.make_raw_prefill(714, H=3, D=64, lengths=[70, 0, 1, 64, 129], scalar_gate=sg),
                      "packed")):
        o32, S32, _ = run(d, ALL, True, chunk=32)
        o64, S64, _ = run(d, ALL, True, chunk=64)
        assert np.array_equal(o32, o64) and np.array_equal(S32, S64), label
    check(d, ALL, True, "chunk 64 packed")


def test_varlen_and_short():
    d = inputs.make_raw_prefill(704, H=3, D=128, lengths=[70, 0, 1, 64, 129])
    check(d, ALL, True, "varlen")
    d = inputs.make_raw_prefill(705, B=4, T=3, H=2, D=128)
    check(d, ALL, True, "T=3")


def test_no_flags_matches_plain_bitwise():
    kda = _kda()
    d = inputs.make_prefill(inputs.WORKLOADS[1], seed=706, B=1, T=130, H=2, s0=True)
    dev = {kk: to_dev(d[kk]) for kk in KEYS}
    S0 = to_dev(d["S0"])
    a = kda.kda_chunk_fwd(*(dev[kk] for kk in KEYS), S0, out_dtype=torch.float32)
    b = kda.kda_chunk_fwd_fused(*(dev[kk] for kk in KEYS), S0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("D", [64, 128])
def test_decode_steps(D):
    kda = _kda()
    rng = np.random.default_rng(707)
    N, H = 3, 2
    S = (0.02 * rng.standard_normal((N, H, D, D))).astype(np.float32)
    S_dev = to_dev(S).clone()
    S_ref = S.astype(np.float64)
    worst = 0.0
    for _ in range(30):
        raw = {"q": 3 * rng.standard_normal((N, H, D)), "k": 3 * rng.standard_normal((N, H, D)),
               "v": rng.standard_normal((N, H, D)), "log_alpha": rng.standard_normal((N, H, D)),
               "beta": rng.standard_normal((N, H)), "gate": rng.standard_normal((N, H, D))}
        bits = {kk: inputs.f32_to_bf16_bits(x.astype(np.float32)) for kk, x in raw.items()}
        o, _ = kda.kda_recurrent_step_fused(*(to_dev(bits[kk]) for kk in KEYS), S_dev, qk_l2norm=True,
                                            beta_logits=True, decay_logits=(BIAS, SCALE),
                                            out_gate=to_dev(bits["gate"]), out_dtype=torch.float32)
        f = {kk: inputs.to_float(x).astype(np.float64) for kk, x in bits.items()}
        q, k, beta, g = P.prologue(f["q"], f["k"], f["beta"], f["log_alpha"], ALL, BIAS, SCALE)
        o_ref = oracle.kda_step(q, k, f["v"], g, beta, S_ref, o_dtype=np.float64)
        o_ref = P.out_gate(o_ref, f["gate"])
        torch.cuda.synchronize()
        worst = max(worst, o_metric(to_host(o)[:, None], o_ref[:, None]))
    es = state_metric(to_host(S_dev), S_ref)
    print(f"[fused] decode D={D}: worst o {worst:.3e} S {es:.3e}", flush=True)
    assert worst <= TOL_BF16 and es <= TOL_BF16


# ------------------------------------------------------------------ scalar gate (gdn_*_fused)
@pytest.mark.parametrize("flags,gate", [(ALL, True), (flags_of(True, False, False), False),
                                        (flags_of(False, True, False), False), (flags_of(False, False, True), False),
                                        (0, True)])
def test_scalar_gate_each_flag_and_all(flags, gate):
    d = inputs.make_raw_prefill(711, B=2, T=300, H=2, D=128, scalar_gate=True)
    check(d, flags, gate, "scalar gate ragged")


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "f32")])
def test_scalar_gate_head_sizes_and_dtypes(D, dtype):
    d = inputs.make_raw_prefill(712, B=1, T=200, H=2, D=D, dtype=dtype, scalar_gate=True)
    check(d, ALL, True, f"scalar gate D={D} {dtype}")


def test_scalar_gate_schedules():
    """Segmented equal-length batch (split schedule), a packed batch cut into segments per
    sequence, and a packed batch of short sequences."""
    d = inputs.make_raw_prefill(713, B=1, T=1000, H=2, D=128, scalar_gate=True)
    check(d, ALL, True, "scalar gate segmented")
    d = inputs.make_raw_prefill(714, H=4, D=128, lengths=[3000, 700, 40, 0], scalar_gate=True)
    check(d, ALL, True, "scalar gate packed, cut")
    d = inputs.make_raw_prefill(715, H=3, D=128, lengths=[70, 0, 1, 64, 129], scalar_gate=True)
    check(d, ALL, True, "scalar gate packed")


def test_scalar_gate_no_flags_matches_plain_bitwise():
    kda = _kda()
    d = inputs.make_prefill(inputs.WORKLOADS[6], seed=716, B=1, T=130, H=2, s0=True, mu=4.0, s=8.0)
    dev = {kk: to_dev(d[kk]) for kk in KEYS}
    S0 = to_dev(d["S0"])
    a = kda.gdn_chunk_fwd(*(dev[kk] for kk in KEYS), S0, out_dtype=torch.float32)
    b = kda.gdn_chunk_fwd_fused(*(dev[kk] for kk in KEYS), S0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("D", [64, 128])
def test_scalar_gate_decode_steps(D):
    kda = _kda()
    rng = np.random.default_rng(717)
    N, H = 3, 2
    S = (0.02 * rng.standard_normal((N, H, D, D))).astype(np.float32)
    S_dev = to_dev(S).clone()
    S_ref = S.astype(np.float64)
    worst = 0.0
    for _ in range(30):
        raw = {"q": 3 * rng.standard_normal((N, H, D)), "k": 3 * rng.standard_normal((N, H, D)),
               "v": rng.standard_normal((N, H, D)), "log_alpha": rng.standard_normal((N, H)),
               "beta": rng.standard_normal((N, H)), "gate": rng.standard_normal((N, H, D))}
        bits = {kk: inputs.f32_to_bf16_bits(x.astype(np.float32)) for kk, x in raw.items()}
        o, _ = kda.gdn_recurrent_step_fused(*(to_dev(bits[kk]) for kk in KEYS), S_dev, qk_l2norm=True,
                                            beta_logits=True, decay_logits=(BIAS, SCALE),
                                            out_gate=to_dev(bits["gate"]), out_dtype=torch.float32)
        f = {kk: inputs.to_float(x).astype(np.float64) for kk, x in bits.items()}
        q, k, beta, g = P.prologue(f["q"], f["k"], f["beta"], f["log_alpha"], ALL, BIAS, SCALE)
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], q.shape))
        o_ref = oracle.kda_step(q, k, f["v"], g, beta, S_ref, o_dtype=np.float64)
        o_ref = P.out_gate(o_ref, f["gate"])
        torch.cuda.synchronize()
        worst = max(worst, o_metric(to_host(o)[:, None], o_ref[:, None]))
    es = state_metric(to_host(S_dev), S_ref)
    print(f"[fused] scalar gate decode D={D}: worst o {worst:.3e} S {es:.3e}", flush=True)
    assert worst <= TOL_BF16 and es <= TOL_BF16


# ------------------------------------------------------------------ token by token (kda/gdn_recurrent_fwd_fused)
@pytest.mark.parametrize("sg", [False, True], ids=["kda", "gdn"])
def test_token_by_token_fused(sg):
    """The fused maps in the token-by-token forward: packed sequences with empty and one-token
    members and fp32 inputs through kda/gdn_recurrent_fwd_fused, and equal-length batches of at
    most 4 tokens through kda/gdn_chunk_fwd_fused (which take this kernel for them)."""
    d = inputs.make_raw_prefill(721, H=3, D=128, lengths=[70, 0, 1, 64, 129], scalar_gate=sg)
    check(d, ALL, True, "token by token, packed", recurrent=True)
    for flags, gate in [(flags_of(True, False, False), False), (flags_of(False, True, True), True)]:
        check(d, flags, gate, "token by token, packed", recurrent=True)
    d = inputs.make_raw_prefill(722, B=2, T=40, H=2, D=64, dtype="f32", scalar_gate=sg)
    check(d, ALL, True, "token by token, fp32 d64", recurrent=True)
    for T in (1, 4):
        d = inputs.make_raw_prefill(723 + T, B=5, T=T, H=2, D=128, scalar_gate=sg)
        check(d, ALL, True, f"chunk entry point, T={T}")
