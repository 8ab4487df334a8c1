"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times: inputs are drawn on the GPU (seeded), the HIP path runs on the whole batch,
and the fp64 oracle recomputes every (sequence, head) unit from the same bf16 values
copied back to the host (in groups of heads or one sequence at a time, so the host
holds one group's arrays at once).

  workload 1  B=4, H=16, T=4096, d=128     all 64 units, chunk 32 and 64
  workload 2  B=1, H=32, T=65536, d=128    all 32 heads
  workload 4  64 packed sequences, 525,197 tokens, H=32, d=128   all 64 x 32 units
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_delta_rule_62_amd import inputs
from gated_delta_rule_62_amd.inputs import host_bits
from gpu_util import TOL_BF16, o_metric, state_metric, to_host

pytestmark = pytest.mark.gpu


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def run_full(x, chunk=0):
    kda = _kda()
    o, Sf = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"], x["cu_seqlens"],
                              out_dtype=torch.float32, chunk=chunk)
    torch.cuda.synchronize()
    return o, Sf


def sampled_oracle(x, heads):
    """Oracle on the given heads of an equal-length batch (same bf16 values)."""
    args = [host_bits(x[kk][:, :, heads]) for kk in ("q", "k", "v", "log_alpha", "beta")]
    S0 = None if x["S0"] is None else x["S0"][:, heads].cpu().numpy()
    return oracle.kda_fwd(*args, S0=S0, o_dtype=np.float64)


@pytest.mark.parametrize("chunk", [32, 64])
def test_workload1_full(chunk):
    w = inputs.WORKLOADS[1]
    print(f"[full] workload 1 {w} chunk {chunk}", flush=True)
    x = inputs.device_prefill(w)
    o, Sf = run_full(x, chunk)
    heads = list(range(w.H))
    o_ref, S_ref = sampled_oracle(x, heads)
    eo, es = o_metric(to_host(o), o_ref), state_metric(to_host(Sf), S_ref)
    print(f"[full]   worst o {eo:.3e} S_final {es:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_workload2_full_all_heads():
    w = inputs.WORKLOADS[2]
    print(f"[full] workload 2 {w}", flush=True)
    x = inputs.device_prefill(w)
    o, Sf = run_full(x)
    worst_o = worst_s = 0.0
    for h0 in range(0, w.H, 8):
        heads = list(range(h0, h0 + 8))
        o_ref, S_ref = sampled_oracle(x, heads)
        eo = o_metric(to_host(o[:, :, heads]), o_ref)
        es = state_metric(to_host(Sf[:, heads]), S_ref)
        print(f"[full]   heads {h0}..{h0 + 7}: worst o {eo:.3e} S_final {es:.3e}", flush=True)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


def test_workload4_full_all_sequences():
    w = inputs.WORKLOADS[4]
    x = inputs.device_prefill(w)
    cu = x["cu_host"]
    lens = np.diff(cu)
    print(f"[full] workload 4: {len(lens)} sequences, {int(cu[-1])} tokens", flush=True)
    o, Sf = run_full(x)
    worst_o = worst_s = 0.0
    for n in range(len(lens)):
        tok = slice(int(cu[n]), int(cu[n + 1]))
        args = [host_bits(x[kk][:, tok]) for kk in ("q", "k", "v", "log_alpha", "beta")]
        o_ref, S_ref = oracle.kda_fwd(*args, o_dtype=np.float64)
        eo = o_metric(to_host(o[:, tok]), o_ref)
        es = state_metric(to_host(Sf[n:n + 1]), S_ref)
        print(f"[full]   sequence {n} (len {lens[n]}): worst o {eo:.3e} S_final {es:.3e}", flush=True)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16
