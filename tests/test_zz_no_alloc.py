"""The no-allocation prefill entry point (kda_chunk_fwd_noalloc) on the GPU, through the C ABI:
its outputs equal kda_chunk_fwd's on the same inputs, bit for bit (the same kernels run on the
library's fixed scratch array instead of a caller workspace), on two calls in a row, the second
with a smaller input, so the second call runs on scratch that still holds the first call's
contents.  Both are also within the parity bound of the fp64 oracle.  Pages: "Decoding Hybrid
Attention Architectures" (intl.cloud.baidu.com article 9569726) sections 3.4 and 4.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_delta_rule_62_amd import inputs
from gpu_util import TOL_BF16, o_metric, state_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _kda():
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    return kda


def _both(d):
    kda = _kda()
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    cu = to_dev(d["cu_seqlens"]) if d["cu_seqlens"] is not None else None
    B, T, H, D, N = d["B"], d["T"], d["H"], d["D"], d["N"]
    o_ref, S_ref = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, cu,
                                     out_dtype=torch.float32)
    o = torch.full((B, T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    Sf = torch.full((N, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    kda.kda_chunk_fwd_noalloc(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, cu, o=o, S_final=Sf)
    torch.cuda.synchronize()
    return to_host(o), to_host(Sf), to_host(o_ref), to_host(S_ref)


@pytest.mark.parametrize("case", ["equal-length", "packed", "packed, cut into segments"])
def test_noalloc_matches_the_workspace_entry_point(case):
    if case == "equal-length":
        # segmented schedule (summaries and entry states in the scratch), then a smaller call
        big = inputs.make_prefill(W[2], seed=701, B=1, T=3000, H=4, s0=True)
        small = inputs.make_prefill(W[2], seed=702, B=1, T=1100, H=2, s0=True)
    elif case == "packed":
        big = inputs.make_prefill(W[4], seed=703, H=3, lengths=[400, 0, 1, 257, 96, 31])
        small = inputs.make_prefill(W[4], seed=704, H=2, lengths=[65, 3])
    else:
        # few long sequences: the segment table, summaries and entry states in the scratch
        big = inputs.make_prefill(W[4], seed=705, H=4, lengths=[3000, 700, 40, 0])
        small = inputs.make_prefill(W[4], seed=706, H=2, lengths=[900, 5])
    for label, d in (("first", big), ("second, smaller", small)):
        print(f"[noalloc] {case} {label}: B={d['B']} T={d['T']} H={d['H']} N={d['N']}", flush=True)
        o, Sf, o_ref, S_ref = _both(d)
        assert np.array_equal(o, o_ref) and np.array_equal(Sf, S_ref)
        o64, S64 = oracle.kda_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0=d["S0"],
                                  cu_seqlens=d["cu_seqlens"], o_dtype=np.float64)
        assert o_metric(o, o64, d["cu_seqlens"]) <= TOL_BF16 and state_metric(Sf, S64) <= TOL_BF16
