"""Prefill parity over a sweep of shapes that reach every schedule the planner picks:
one pass, the plain two-segment schedule, and split schedules of 3 to 26 segments
(segment 0's output pass in the same launch as the other summaries, lengthened when
segments are long) with ragged last segments and chunks; both chunk lengths, both head sizes, fp32 and bf16 inputs,
the fast-decay mixture and packed batches.  Each case is compared with the fp64
oracle on the same seeded inputs.  Pages: "Decoding Hybrid Attention Architectures"
(intl.cloud.baidu.com article 9569726) sections 3.4 and 4.
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

# (B, T, H, D, chunk, dtype, mixture, S0); the comment names the plan for these sizes
CASES = [
    (1, 2000, 1, 64, 32, "bf16", False, True),     # 1 unit: 13 segments of 5 chunks
    (1, 1500, 3, 64, 32, "f32", True, True),       # 3 units: 10 segments, fp32 inputs
    (2, 900, 5, 128, 32, "bf16", True, False),     # 10 units: 6 segments, zero S0
    (1, 3000, 7, 64, 32, "bf16", False, True),     # 7 units: 19 segments
    (2, 700, 8, 64, 32, "bf16", True, True),       # 16 units: 5 segments, ragged last chunk
    (1, 1200, 48, 64, 32, "bf16", False, True),    # 48 units: 6 segments (240 workgroups per pass)
    (4, 300, 25, 64, 32, "bf16", True, True),      # 100 units: plain two-segment schedule
    (1, 700, 129, 64, 32, "bf16", False, True),    # 129 units: plain two segments
    (3, 1000, 2, 128, 64, "bf16", True, True),     # 64-token chunks: plain schedule, 4 segments
    (1, 64, 2, 64, 32, "bf16", False, True),       # one pass
    (1, 4100, 1, 128, 32, "bf16", True, True),     # 1 unit, d = 128: 26 segments
    (1, 10300, 64, 64, 32, "bf16", True, True),    # 64 units: 5 segments of 65 chunks; segment 0
                                                   # lengthened to 70, the others 63, ragged chunk
]


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}D{c[3]}C{c[4]}{c[5]}" for c in CASES])
def test_prefill_schedule_sweep(case):
    B, T, H, D, chunk, dtype, mix, s0 = case
    kda = _kda()
    d = inputs.make_prefill(W[1], seed=300 + T + H, B=B, T=T, H=H, D=D, dtype=dtype, mix=mix, s0=s0)
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    print(f"[sweep] B={B} T={T} H={H} D={D} chunk={chunk} {dtype} mix={mix} S0={s0} "
          f"workspace={kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, B, False, chunk)}", flush=True)
    o, Sf = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, None,
                              out_dtype=torch.float32, chunk=chunk)
    torch.cuda.synchronize()
    o, Sf = to_host(o), to_host(Sf)
    o_ref, S_ref = oracle.kda_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0=d["S0"],
                                  cu_seqlens=None, o_dtype=np.float64)
    eo, es = o_metric(o, o_ref), state_metric(Sf, S_ref)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    print(f"[sweep]   worst o {eo:.3e}  S_final {es:.3e}  (tol {tol})", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    assert eo <= tol and es <= tol


def test_two_calls_on_two_streams_interleave():
    """Two segmented calls enqueued on two streams at once, each running all of its kernels on
    its own stream; both results must match one call alone."""
    kda = _kda()
    d1 = inputs.make_prefill(W[1], seed=401, B=1, T=1500, H=3, D=64, s0=True)
    d2 = inputs.make_prefill(W[1], seed=402, B=1, T=1200, H=5, D=64, s0=True, mix=True)
    args = []
    for d in (d1, d2):
        args.append(([to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")], to_dev(d["S0"])))
    ref = []
    for (x, S0) in args:
        ref.append([to_host(t) for t in kda.kda_chunk_fwd(*x, S0, None, out_dtype=torch.float32)])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        outs = []
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream())
        s1.wait_event(ev)
        s2.wait_event(ev)
        for (x, S0), st in zip(args, (s1, s2)):
            with torch.cuda.stream(st):
                outs.append(kda.kda_chunk_fwd(*x, S0, None, out_dtype=torch.float32, stream=st))
        torch.cuda.synchronize()
        for (o, Sf), (o_ref, S_ref) in zip(outs, ref):
            assert np.array_equal(to_host(o), o_ref) and np.array_equal(to_host(Sf), S_ref)
