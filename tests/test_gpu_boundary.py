"""The C ABI's contract on the GPU: streams, the workspace's status word and the failure path of
the kernels' bounded ordering waits.

  * A call enqueued on a stream other than torch's current one, followed at once by new
    allocations and writes on the current stream, still returns the oracle's result: every
    tensor the binding allocates for the call is kept alive for the call's stream.
  * Every kernel of a prefill call runs on the caller's stream (the library creates no stream
    of its own): a call on a fresh stream is ordered after earlier work on it and before later
    work on it, with no synchronisation in between.
  * The status word at the start of the workspace is 0 after a normal call.  With the poll
    limit of the ordering waits forced to 0 from the host (KDA_DEBUG_WAIT_POLLS=0), the waits
    give up at once: every kernel still runs to its end, the outputs are NaN, and the status
    word is set.  A normal call on the same workspace clears it again.
Pages: "Decoding Hybrid Attention Architectures" (intl.cloud.baidu.com article 9569726) sections
3.4 and 4.
"""
from __future__ import annotations

import os

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


def _oracle(d):
    return oracle.kda_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0=d["S0"],
                          cu_seqlens=d["cu_seqlens"], o_dtype=np.float64)


def test_call_on_another_stream_keeps_its_buffers():
    kda = _kda()
    d = inputs.make_prefill(W[2], seed=601, B=1, T=2000, H=4, s0=True)   # segmented schedule
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("[boundary] prefill on a side stream, then allocations on the current stream", flush=True)
    o, Sf = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0,
                              out_dtype=torch.float32, stream=side)
    # the binding's workspace is released when the call returns; new tensors written on the
    # current stream must not land in it while the side stream still runs
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    o_ref, S_ref = _oracle(d)
    assert o_metric(to_host(o), o_ref) <= TOL_BF16
    assert state_metric(to_host(Sf), S_ref) <= TOL_BF16


def test_all_work_stays_on_the_callers_stream():
    """A call on a fresh stream reads inputs written just before it on that stream and its
    outputs are read by work enqueued right after it, all without synchronisation."""
    kda = _kda()
    d = inputs.make_prefill(W[2], seed=602, B=1, T=3000, H=2, s0=True)
    host = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0h = to_dev(d["S0"])
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        dev = {kk: torch.empty_like(t) for kk, t in host.items()}
        S0 = torch.empty_like(S0h)
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for kk in dev:
            dev[kk].copy_(host[kk])
        S0.copy_(S0h)
        o, Sf = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0,
                                  out_dtype=torch.float32, stream=st)
        o2, Sf2 = o.clone(), Sf.clone()
    st.synchronize()
    o_ref, S_ref = _oracle(d)
    assert o_metric(to_host(o2), o_ref) <= TOL_BF16
    assert state_metric(to_host(Sf2), S_ref) <= TOL_BF16


CASES = [
    ("segmented", dict(B=1, T=3000, H=2, s0=True)),          # single-launch pass 1, combine, pass 2
    ("one pass", dict(B=8, T=200, H=40, s0=True)),           # enough units for one pass
    ("packed", dict(lengths=[300, 0, 1, 129, 64], H=3)),     # packed sequences
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_status_word_reports_a_broken_ordering(label, kw, monkeypatch):
    kda = _kda()
    w = W[4] if "lengths" in kw else W[2]
    d = inputs.make_prefill(w, seed=603, **kw)
    dev = {kk: to_dev(d[kk]) for kk in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(d["S0"]) if d["S0"] is not None else None
    cu = to_dev(d["cu_seqlens"]) if d["cu_seqlens"] is not None else None
    B, T, H, D, N = d["B"], d["T"], d["H"], d["D"], d["N"]
    ws = torch.full((kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, N, cu is not None),), 0x5A,
                    dtype=torch.uint8, device="cuda")

    def call():
        o, Sf = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S0, cu,
                                  out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        return to_host(o), to_host(Sf)

    print(f"[boundary] {label}: normal call", flush=True)
    o, Sf = call()
    assert kda.workspace_status(ws) == 0
    o_ref, S_ref = _oracle(d)
    assert o_metric(o, o_ref, d["cu_seqlens"]) <= TOL_BF16 and state_metric(Sf, S_ref) <= TOL_BF16

    print(f"[boundary] {label}: poll limit 0 (every ordering wait gives up at once)", flush=True)
    monkeypatch.setenv("KDA_DEBUG_WAIT_POLLS", "0")
    o_bad, Sf_bad = call()
    assert kda.workspace_status(ws) != 0
    real = np.ones(T, dtype=bool) if cu is None else np.repeat(np.diff(d["cu_seqlens"]) > 0, np.diff(d["cu_seqlens"]))
    assert np.isnan(o_bad[:, real]).any()
    monkeypatch.delenv("KDA_DEBUG_WAIT_POLLS")

    print(f"[boundary] {label}: normal call again on the same workspace", flush=True)
    o2, Sf2 = call()
    assert kda.workspace_status(ws) == 0
    assert np.array_equal(o2, o) and np.array_equal(Sf2, Sf)
