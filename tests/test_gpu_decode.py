"""Decode-step parity on the GPU: kda_recurrent_step (HIP, through the C ABI) vs
the fp64 CPU oracle on the same seeded inputs.

Pages: the recurrent (constant-state) decode of "Decoding Hybrid Attention
Architectures" (intl.cloud.baidu.com article 9569726) section 1 and the rule of its
section 3.4.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_delta_rule_62_amd import inputs
from gpu_util import TOL_BF16, TOL_F32, slice_metric, to_dev, to_host

pytestmark = pytest.mark.gpu


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def run_steps(N, H, D, dtype, steps, seed, check_every=1, sample=None):
    """Run `steps` decode steps on the GPU and on the oracle (optionally only for
    the sequences in `sample`), comparing o every `check_every` steps and S at the end."""
    kda = _kda()
    print(f"[decode] N={N} H={H} D={D} dtype={dtype} steps={steps} seed={seed}", flush=True)
    ds = inputs.DecodeStream(inputs.WORKLOADS[3], seed=seed, num_seqs=N, H=H, D=D, dtype=dtype)
    S_gpu = to_dev(ds.state())
    sel = np.arange(N) if sample is None else np.asarray(sample)
    S_ref = np.ascontiguousarray(ds.state()[sel].astype(np.float64))
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    worst_o = 0.0
    for s in range(steps):
        x = ds.step()
        dev = {kk: to_dev(vv) for kk, vv in x.items()}
        o, _ = kda.kda_recurrent_step(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                                      S_gpu, out_dtype=torch.float32)
        o_ref = oracle.kda_step(*(x[kk][sel] for kk in ("q", "k", "v", "log_alpha", "beta")), S_ref,
                                o_dtype=np.float64)
        if s % check_every == 0 or s == steps - 1:
            torch.cuda.synchronize()
            worst_o = max(worst_o, slice_metric(to_host(o)[sel], o_ref, axes=(2,)))
    torch.cuda.synchronize()
    worst_s = slice_metric(to_host(S_gpu)[sel], S_ref, axes=(2, 3))
    print(f"[decode]   worst o {worst_o:.3e}  S {worst_s:.3e}  tol {tol}", flush=True)
    assert worst_o <= tol and worst_s <= tol
    return worst_o, worst_s


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(D, dtype):
    run_steps(N=5, H=3, D=D, dtype=dtype, steps=24, seed=101 + D)


def test_decode_full_shape_sampled():
    """The decode workload's launch shape (256 sequences x 32 heads, d=128, bf16),
    oracle-checked on 8 sampled sequences at every step."""
    run_steps(N=256, H=32, D=128, dtype="bf16", steps=48, seed=4, sample=[0, 1, 2, 3, 100, 200, 254, 255])


def test_decode_1024_steps_all_heads():
    """1024 sequential steps (the decode workload's step count) on 32 sequences x 32 heads,
    d=128, bf16: o checked at every step for sequences 0-7 and at the last step for all,
    the final state for every head, all against the fp64 oracle run on every head."""
    kda = _kda()
    N, H, D, steps = 32, 32, 128, 1024
    ds = inputs.DecodeStream(inputs.WORKLOADS[3], seed=4, num_seqs=N, H=H, D=D, dtype="bf16")
    S_gpu = to_dev(ds.state())
    S_ref = np.ascontiguousarray(ds.state().astype(np.float64))
    worst_o = 0.0
    for s in range(steps):
        x = ds.step()
        dev = {kk: to_dev(vv) for kk, vv in x.items()}
        o, _ = kda.kda_recurrent_step(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                                      S_gpu, out_dtype=torch.float32)
        o_ref = oracle.kda_step(*(x[kk] for kk in ("q", "k", "v", "log_alpha", "beta")), S_ref,
                                o_dtype=np.float64)
        rows = slice(None) if s == steps - 1 else slice(0, 8)
        worst_o = max(worst_o, slice_metric(to_host(o)[rows], o_ref[rows], axes=(2,)))
        if s % 256 == 0:
            print(f"[decode] step {s}: worst o so far {worst_o:.3e}", flush=True)
    torch.cuda.synchronize()
    worst_s = slice_metric(to_host(S_gpu), S_ref, axes=(2, 3))
    print(f"[decode]   1024 steps: worst o {worst_o:.3e}  S {worst_s:.3e}  tol {TOL_BF16}", flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


@pytest.mark.timeout(900)
def test_decode_workload_full_1024_steps_every_head():
    """The decode workload itself: 256 sequences x 32 heads, d=128, bf16 inputs, 1024 sequential
    steps on an fp32 state S0 ~ 0.02 N(0,1).  o is checked at every step for sequences 0-7 and
    at the last step for all 8192 heads, and the final state of every head, all against the
    fp64 oracle run on every head (the constant-size recurrent state of "Decoding Hybrid
    Attention Architectures" section 1).  Inputs are drawn on the device with the workload's
    recipe and copied to the host, so both sides read the same bf16 values."""
    kda = _kda()
    w = inputs.WORKLOADS[3]
    print("[decode] full workload: 256 x 32 heads, 1024 steps", flush=True)
    S_init, steps_in = inputs.device_decode_steps(w, w.steps, seed=44)
    S_gpu = S_init.clone()
    S_ref = np.ascontiguousarray(to_host(S_init).astype(np.float64))
    worst_o = 0.0
    for s in range(w.steps):
        x = steps_in[s]
        o, _ = kda.kda_recurrent_step(*x, S_gpu, out_dtype=torch.float32)
        hx = [inputs.host_bits(t) for t in x]
        o_ref = oracle.kda_step(*hx, S_ref, o_dtype=np.float64)
        rows = slice(None) if s == w.steps - 1 else slice(0, 8)
        worst_o = max(worst_o, slice_metric(to_host(o)[rows], o_ref[rows], axes=(2,)))
        steps_in[s] = None
        if s % 128 == 0:
            print(f"[decode] step {s}: worst o so far {worst_o:.3e}", flush=True)
    torch.cuda.synchronize()
    worst_s = slice_metric(to_host(S_gpu), S_ref, axes=(2, 3))
    print(f"[decode]   full workload: worst o {worst_o:.3e}  S {worst_s:.3e}  tol {TOL_BF16}", flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


def test_decode_inplace_and_out_of_place_agree_and_bf16_output_is_rne():
    kda = _kda()
    ds = inputs.DecodeStream(inputs.WORKLOADS[3], seed=7, num_seqs=3, H=2, D=128)
    x = {kk: to_dev(vv) for kk, vv in ds.step().items()}
    S0 = to_dev(ds.state())
    S_a = S0.clone()
    o_a, _ = kda.kda_recurrent_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S_a,
                                    out_dtype=torch.float32)
    S_b = torch.empty_like(S0)
    o_b, _ = kda.kda_recurrent_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S0.clone(), S_b,
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(S_a, S_b)
    assert torch.equal(o_a.to(torch.bfloat16), o_b)   # torch's cast is round-to-nearest-even


def test_decode_rejects_bad_arguments():
    kda = _kda()
    ds = inputs.DecodeStream(inputs.WORKLOADS[3], seed=8, num_seqs=2, H=2, D=128)
    x = {kk: to_dev(vv) for kk, vv in ds.step().items()}
    S = to_dev(ds.state())
    with pytest.raises(kda.KDAError) as e:      # unsupported head size
        kda.kda_recurrent_step(x["q"][..., :96].contiguous(), x["k"][..., :96].contiguous(),
                               x["v"][..., :96].contiguous(), x["log_alpha"][..., :96].contiguous(),
                               x["beta"], S[..., :96, :96].contiguous())
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    with pytest.raises(kda.KDAError) as e:      # partial overlap of S_in and S_out
        flat = torch.empty(S.numel() + 64, device="cuda")
        kda.kda_recurrent_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                               flat[:S.numel()].view_as(S), flat[64:].view_as(S))
    assert e.value.status == kda.KDA_ERR_INVALID_ARGUMENT
