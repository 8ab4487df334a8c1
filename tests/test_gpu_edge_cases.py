"""Prefill parity on the method's special cases: the chunkwise kernels (32-token pipelined and
64-token single-buffered, both head sizes, fp32 and bf16 inputs) against the fp64 oracle on
inputs that sit on the edges of the rule's domain.

  * beta = 0: nothing is written.  With S0 = 0 the outputs are exactly zero; with S0 != 0 the
    state only decays ("Decoding Hybrid Attention Architectures", sections 3.3 and 3.5).
  * beta = 1 with unit keys and q_t = k_t: the write replaces the slot, so o_t = v_t for any
    decay and any earlier state; with alpha = 1 and orthonormal keys every written value reads
    back from the final state (section 3.2 of the same page, the overwrite behaviour).
  * log_alpha = 0 exactly: the plain delta rule (DeltaNet, section 3.2 and the variant table).
  * a chunk of identical keys: the strictly lower block of beta K K^T is dense, the hardest
    case for the (I + A) solve (section 4).
  * steep per-channel decays: chunk log-decay sums of -40, -80 and -150 on half the channels
    (fast forgetting, sections 3.3 and 3.5; "Technical Analysis and Engineering Practices for
    Novel Hybrid Linear Attention Architectures", section 2 items 2-3), with a ragged tail.

Every case compares element by element with the oracle at the parity bound (1e-4 for fp32
inputs, 2e-3 for bf16 inputs, per (sequence, head) slice); the closed forms are checked as well
where the case has one.  Inputs are the seeded workload recipe with the named fields replaced.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_delta_rule_62_amd import inputs
from gpu_util import TOL_BF16, TOL_F32, o_metric, slice_metric, state_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS
GRID = [(c, D, dt) for c in (32, 64) for D in (64, 128) for dt in ("f32", "bf16")]
IDS = [f"C{c}-D{D}-{dt}" for c, D, dt in GRID]


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def _cast(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _f(x):
    return inputs.to_float(x).astype(np.float64)


def run(d, chunk, fn="kda_chunk_fwd"):
    kda = _kda()
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    cu = to_dev(d["cu_seqlens"]) if d.get("cu_seqlens") is not None else None
    o, Sf = getattr(kda, fn)(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, cu,
                             out_dtype=torch.float32, chunk=chunk)
    torch.cuda.synchronize()
    return to_host(o), to_host(Sf)


def against_oracle(d, chunk, label, scalar_gate=False):
    print(f"[edge] {label}: B={d['B']} T={d['T']} H={d['H']} D={d['D']} {d['dtype']} chunk={chunk}", flush=True)
    o, Sf = run(d, chunk, "gdn_chunk_fwd" if scalar_gate else "kda_chunk_fwd")
    g = d["log_alpha"]
    if scalar_gate:   # the scalar gate is the per-channel rule with the decay broadcast over channels
        g = np.ascontiguousarray(np.repeat(g[..., None], d["D"], axis=-1))
    o_ref, S_ref = oracle.kda_fwd(d["q"], d["k"], d["v"], g, d["beta"], S0=d["S0"],
                                  cu_seqlens=d.get("cu_seqlens"), o_dtype=np.float64)
    tol = TOL_F32 if d["dtype"] == "f32" else TOL_BF16
    eo, es = o_metric(o, o_ref, d.get("cu_seqlens")), state_metric(Sf, S_ref)
    print(f"[edge]   worst o {eo:.3e}  S_final {es:.3e}  (tol {tol})", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    assert eo <= tol and es <= tol
    return o, Sf, o_ref, S_ref


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_beta_zero_zero_state_gives_exact_zeros(chunk, D, dtype):
    """beta = 0 and S0 = 0: no write ever happens, so o and S_final are exactly zero."""
    d = inputs.make_prefill(W[1], seed=501, B=2, T=3 * chunk + 7, H=2, D=D, dtype=dtype)
    d["beta"] = _cast(np.zeros(d["beta"].shape), dtype)
    o, Sf = run(d, chunk)
    assert np.count_nonzero(o) == 0 and np.count_nonzero(Sf) == 0


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_beta_zero_with_state_is_pure_decay(chunk, D, dtype):
    """beta = 0 and S0 != 0: S_t = Diag(exp(sum_{i<=t} log_alpha_i)) S0 and o_t = S_t^T q_t."""
    d = inputs.make_prefill(W[1], seed=502, B=1, T=3 * chunk + 11, H=2, D=D, dtype=dtype, s0=True)
    d["beta"] = _cast(np.zeros(d["beta"].shape), dtype)
    o, Sf, _, _ = against_oracle(d, chunk, "beta=0, S0")
    # the closed form, evaluated independently of the oracle
    cum = np.cumsum(_f(d["log_alpha"]), axis=1)                       # [B, T, H, D]
    S0 = d["S0"].astype(np.float64)                                   # [1, H, D, D]
    closed_S = np.exp(cum[0, -1])[:, :, None] * S0[0]                 # [H, D, D]
    closed_o = np.einsum("thc,thcj->thj", _f(d["q"])[0], np.exp(cum[0])[:, :, :, None] * S0[0][None])
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert state_metric(Sf, closed_S[None]) <= tol
    assert slice_metric(o[0], closed_o, axes=(0, 2)) <= tol


def _signed_basis_keys(rng, T, D):
    """T keys, each +-e_i, cycling through a random permutation of the D basis vectors."""
    perm = rng.permutation(D)
    sign = rng.choice([-1.0, 1.0], size=T)
    k = np.zeros((T, D), dtype=np.float32)
    k[np.arange(T), perm[np.arange(T) % D]] = sign
    return k


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_overwrite_reads_back_every_value(chunk, D, dtype):
    """beta = 1, q_t = k_t, unit keys: o_t = v_t whatever the decay and the earlier state."""
    rng = np.random.default_rng(503)
    T, H = 2 * D + 5, 2   # every basis key written twice, then a few more: later writes replace earlier ones
    d = inputs.make_prefill(W[1], seed=503, B=1, T=T, H=H, D=D, dtype=dtype, s0=True)
    k = np.stack([_signed_basis_keys(rng, T, D) for _ in range(H)], axis=1)[None]   # [1, T, H, D]
    d["k"] = _cast(k, dtype)
    d["q"] = d["k"].copy()
    d["beta"] = _cast(np.ones(d["beta"].shape), dtype)
    o, Sf, _, _ = against_oracle(d, chunk, "beta=1, q=k")
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert slice_metric(o, _f(d["v"]), axes=(1, 3)) <= tol


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_orthonormal_keys_without_decay_read_back_from_the_final_state(chunk, D, dtype):
    """beta = 1, alpha = 1, orthonormal keys: after all writes S_T^T k_i = v_i for the last write
    of every key (half the basis is written twice; the later write replaces the earlier one)."""
    rng = np.random.default_rng(504)
    T, H = D + D // 2, 2   # the first half of the basis is written twice
    d = inputs.make_prefill(W[1], seed=504, B=1, T=T, H=H, D=D, dtype=dtype, s0=True)
    k = np.stack([_signed_basis_keys(rng, T, D) for _ in range(H)], axis=1)[None]
    d["k"] = _cast(k, dtype)
    d["beta"] = _cast(np.ones(d["beta"].shape), dtype)
    d["log_alpha"] = _cast(np.zeros(d["log_alpha"].shape), dtype)
    o, Sf, _, _ = against_oracle(d, chunk, "orthonormal keys, alpha=1")
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    kf, vf = _f(d["k"])[0], _f(d["v"])[0]
    for h in range(H):
        read = kf[:, h] @ Sf[0, h]              # row t: S_T^T k_t
        last = {}
        for t in range(T):
            last[int(np.argmax(np.abs(kf[t, h])))] = t
        rows = np.array(sorted(last.values()))
        assert rows.size == D
        assert slice_metric(read[rows], vf[rows, h], axes=(0, 1)) <= tol


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_no_decay_is_the_delta_rule(chunk, D, dtype):
    """log_alpha = 0 exactly (DeltaNet)."""
    d = inputs.make_prefill(W[1], seed=505, B=2, T=4 * chunk - 3, H=2, D=D, dtype=dtype, s0=True)
    d["log_alpha"] = _cast(np.zeros(d["log_alpha"].shape), dtype)
    against_oracle(d, chunk, "log_alpha=0")


@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_repeated_identical_keys_in_a_chunk(chunk, D, dtype):
    """Tokens [chunk, 2 chunk) all share one key (and the last chunk half of another)."""
    rng = np.random.default_rng(506)
    T, H = 3 * chunk + chunk // 2, 2
    d = inputs.make_prefill(W[1], seed=506, B=1, T=T, H=H, D=D, dtype=dtype, s0=True)
    k = inputs.to_float(d["k"]).copy()
    for h in range(H):
        u = rng.standard_normal(D)
        k[0, chunk:2 * chunk, h] = u / np.linalg.norm(u)
        w = rng.standard_normal(D)
        k[0, 3 * chunk:, h] = w / np.linalg.norm(w)
    d["k"] = _cast(k, dtype)
    against_oracle(d, chunk, "repeated keys")


@pytest.mark.parametrize("X", [40, 80, 150])
@pytest.mark.parametrize("chunk,D,dtype", GRID, ids=IDS)
def test_steep_decay_channels(chunk, D, dtype, X):
    """Half the key channels decay by exp(-X) over every chunk (log_alpha = -X / chunk per
    token), the rest follow the recipe; a ragged last chunk and a nonzero S0."""
    d = inputs.make_prefill(W[1], seed=507 + X, B=2, T=3 * chunk + 9, H=2, D=D, dtype=dtype, s0=True)
    g = inputs.to_float(d["log_alpha"]).copy()
    steep = np.random.default_rng(508).permutation(D)[: D // 2]
    g[..., steep] = -float(X) / chunk
    d["log_alpha"] = _cast(g, dtype)
    against_oracle(d, chunk, f"steep decay, chunk sum -{X}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_gate_edge_cases(D, dtype):
    """The scalar-gate kernel (gdn_chunk_fwd) on beta = 0 (exact zeros with S0 = 0), log_alpha = 0
    and a steep decay of -150 per 32-token chunk."""
    T = 3 * 32 + 5
    d = inputs.make_prefill(W[1], seed=509, B=2, T=T, H=2, D=D, dtype=dtype, scalar_gate=True)
    d["beta"] = _cast(np.zeros(d["beta"].shape), dtype)
    o, Sf = run(d, 32, "gdn_chunk_fwd")
    assert np.count_nonzero(o) == 0 and np.count_nonzero(Sf) == 0
    d = inputs.make_prefill(W[1], seed=510, B=2, T=T, H=2, D=D, dtype=dtype, scalar_gate=True, s0=True)
    d["log_alpha"] = _cast(np.zeros(d["log_alpha"].shape), dtype)
    against_oracle(d, 32, "scalar gate, log_alpha=0", scalar_gate=True)
    d = inputs.make_prefill(W[1], seed=511, B=2, T=T, H=2, D=D, dtype=dtype, scalar_gate=True, s0=True)
    d["log_alpha"] = _cast(np.full(d["log_alpha"].shape, -150.0 / 32), dtype)
    against_oracle(d, 32, "scalar gate, chunk sum -150", scalar_gate=True)


@pytest.mark.parametrize("chunk", [32, 64])
def test_edge_cases_in_a_packed_batch(chunk):
    """The cases above side by side in one packed batch (each sequence its own case), with
    empty and one-token sequences between them."""
    lengths = [chunk + 3, 0, 2 * chunk, 1, chunk + chunk // 2, 2 * chunk + 1]
    D, H = 128, 2
    d = inputs.make_prefill(W[4], seed=512, H=H, D=D, lengths=lengths)
    cu = d["cu_seqlens"]
    beta = inputs.to_float(d["beta"]).copy()
    g = inputs.to_float(d["log_alpha"]).copy()
    k = inputs.to_float(d["k"]).copy()
    beta[:, cu[0]:cu[1]] = 0.0                                # no write
    g[:, cu[2]:cu[3]] = 0.0                                   # no decay
    k[:, cu[4]:cu[5]] = k[:, cu[4]:cu[4] + 1]                 # one repeated key
    g[:, cu[5]:cu[6], :, : D // 2] = -80.0 / chunk            # steep channels
    beta[:, cu[5]:cu[6]] = 1.0
    d["beta"], d["log_alpha"], d["k"] = _cast(beta, "bf16"), _cast(g, "bf16"), _cast(k, "bf16")
    d["S0"] = (0.02 * np.random.default_rng(513).standard_normal((d["N"], H, D, D))).astype(np.float32)
    against_oracle(d, chunk, "packed edge cases")
