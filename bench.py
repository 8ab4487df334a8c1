#!/usr/bin/env python3
"""Benchmark of the KDA layer on one MI355X.

A step is one prefill call (``kda_chunk_fwd``) on the long-context workload:
B=1, H=32, T=65536, d_k=d_v=128, bf16 q/k/v/log_alpha/beta, fp32 initial state
S0 ~ 0.02*N(0,1), bf16 o and fp32 S_final, chunk 32 (the library default).
``value`` is prefill tokens/s (sequence tokens, not token-heads) with the inputs
resident in HBM.

The same JSON line also reports the decode workload (256 sequences x 32 heads,
d=128, 1024 sequential ``kda_recurrent_step`` calls on an fp32 state) as
``decode``, the same prefill with the fused prologue / epilogue as
``fused_prologue``, the scalar-gated variant (Gated DeltaNet) at the long-context shape
as ``gdn``, a few new tokens per sequence on top of a carried state as
``continuation``, the gradient (``kda_chunk_bwd``) on the training-prefill
workload as ``backward``, the roofline of each path's dominant launch measured with HIP events
on the launch stream, and the fp64 CPU oracle timed on a bounded sample of the
same workloads on this host (``cpu_baseline``).  ``prefill_workloads`` gives the
forward of the other prefill workloads the same way: the tiny fp32 one (B=1, H=2,
T=256, d=64, chunk 64), the training shape (B=4, H=16, T=4096, d=128) at chunk 64
as the workload names it and at the default chunk 32, and the packed varlen one
(64 sequences, 525,197 tokens, H=32, d=128).  Every prefill line gives the median
and the minimum of individually timed calls (HIP events around each call).

Inputs are synthetic and seeded, drawn on the GPU with the workloads' recipe
(q, k L2-normalised normals, v normal, beta = sigmoid(normal), log_alpha =
logsigmoid(normal + mu)/s); the parity tests draw the same recipe on the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H32,d128,T64K) + decode steps/s and HBM GB/s"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
CHUNK = 32                       # chunk length passed to kda_chunk_fwd (the library default)


def prefill_alg_flops_per_token_head(d: int, C: int = CHUNK) -> int:
    """Flops the chunkwise method needs per (token, head), counting only the
    needed triangles: A (C-1)d, P (C+1)d, W and U 2(C+1)d, P*Unew (C+1)d,
    and 6d^2 for K S, Q S and Khat^T Unew.  The (I+A)^-1 solve is excluded."""
    return 6 * d * d + (C - 1) * d + 4 * (C + 1) * d


def prefill_tile_flops_per_token_head(d: int, C: int = CHUNK) -> int:
    """Flops the full C x C tiles would issue: 6d^2 + 6Cd (A, P, W, U, P*Unew
    as dense products) + 4Cd."""
    return 6 * d * d + 10 * C * d


def prefill_alg_bytes(T: int, H: int, d: int, n_seqs: int, has_s0: bool) -> int:
    """q, k, v, log_alpha, beta read once, o written once (bf16), S0 read and
    S_final written once (fp32)."""
    per_token_head = 4 * d * 2 + 2 + d * 2
    states = n_seqs * H * d * d * 4 * (2 if has_s0 else 1)
    return T * H * per_token_head + states


def backward_alg_flops_per_token_head(d: int, C: int = CHUNK) -> int:
    """Flops of the chunkwise gradient per (token, head): ten d x d contractions per
    token (the state pass K' S_m and K''^T E, the reverse pass K'' dS_n, Q'^T dO and
    K'^T dV, then R, dE, dQ', dK', dK'' in the gradient step), 2 d^2 flops each, and
    sixteen C-deep ones over d (L, P, M Y, M^T dE, P^T dO twice, dP, dA, dP K'',
    dL K'', dP^T Q', dL^T K' and the C-sized parts of the state passes), 2 C d each."""
    return 20 * d * d + 32 * C * d


def backward_alg_bytes(T: int, H: int, d: int, n_seqs: int) -> int:
    """q, k, v, log_alpha, d_o and beta read once, dq, dk, dv, dlog_alpha and dbeta
    written once (bf16), dS_final read and dS0 written (fp32)."""
    return T * H * (5 * d * 2 + 2 + 4 * d * 2 + 2) + 2 * n_seqs * H * d * d * 4


def decode_alg_bytes(N: int, H: int, d: int) -> int:
    """State read and written once (fp32), q, k, v, log_alpha and o (bf16), beta."""
    return 2 * N * H * d * d * 4 + 4 * N * H * d * 2 + N * H * 2 + N * H * d * 2


def counted_traffic(kind: str):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (profiles/traffic.json), or None once the kernel source has changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[kind]
    except (OSError, KeyError, ValueError):
        return None
    files = {"decode": ["kda_decode.hip", "kda_device.h", "kda_launch.h"],
             "prefill": ["kda_prefill.hip", "kda_device.h", "kda_launch.h"],
             "backward": ["kda_backward.hip", "kda_backward.h", "kda_device.h"]}[kind]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_62_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def counted_workload(key: str):
    """Counter figures of one bench workload's call (profiles/traffic.json "workloads"): HBM bytes
    from FETCH_SIZE/WRITE_SIZE and the matrix-core / vector-ALU busy fractions, or None once the
    prefill kernel source has changed since they were taken."""
    import hashlib
    try:
        tj = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        rec = tj["workloads"][key]
        want = tj["prefill"]["source_sha256"]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ("kda_prefill.hip", "kda_device.h", "kda_launch.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_62_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != want:
        return None
    return {"traffic": rec["read_bytes"] + rec["write_bytes"], "mfma_busy": rec["mfma_busy"],
            "valu_busy": rec["valu_busy"], "kernels": rec["kernels"]}


# floats per (chunk, head) record of the backward at d = 128: M, P, L (32 x 32 each), e_m, e_n
# (128 each), beta (32), the decay exponents (32 x 128)
Rec128 = 3 * 32 * 32 + 2 * 128 + 32 + 32 * 128


def timed_calls(torch, fn, stream, warmup: int, n: int) -> dict:
    """warmup untimed calls, then n calls each bracketed by HIP events on `stream`:
    median, min and mean milliseconds per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": ms[len(ms) // 2], "min": ms[0], "mean": sum(ms) / len(ms), "calls": n}


def prefill_line(label, tokens, H, d, n_seqs, has_s0, C, t, in_bytes=2, out_bytes=2):
    """Throughput and roofline fields of one prefill workload from its call times t (ms)."""
    per_token_head = 4 * d * in_bytes + in_bytes + d * out_bytes
    byts = tokens * H * per_token_head + n_seqs * H * d * d * 4 * (2 if has_s0 else 1)
    flops = prefill_alg_flops_per_token_head(d, C) * tokens * H
    tile = prefill_tile_flops_per_token_head(d, C) * tokens * H
    sec = t["median"] / 1e3
    return {"workload": label, "tokens": tokens, "value": tokens / sec, "unit": "tokens/s",
            "ms_per_call_median": t["median"], "ms_per_call_min": t["min"], "ms_per_call_mean": t["mean"],
            "roofline": {"bound": "hbm", "achieved": byts / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": byts / sec / 1e9 / HBM_PEAK_GBS, "bytes_per_call": byts,
                         "mfma_frac": flops / sec / 1e12 / BF16_PEAK_TFLOPS,
                         "mfma_frac_dense_tile": tile / sec / 1e12 / BF16_PEAK_TFLOPS,
                         "flop_convention": f"algorithmic {prefill_alg_flops_per_token_head(d, C)} / dense-tile "
                                            f"{prefill_tile_flops_per_token_head(d, C)} per token-head at C={C}"}}


def cpu_baseline_batch(torch, x, target_s=6.0):
    """The fp64 oracle on a bounded sample of a device batch x (inputs.device_prefill layout):
    equal-length batches run the first Ts tokens of every sequence, packed batches their first
    sequences; the sample is sized from a calibration run to about target_s seconds."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    H = x["H"]
    units_per_seq = H
    keys = ("q", "k", "v", "log_alpha", "beta")
    if x["cu_seqlens"] is None:
        B, T = x["B"], x["T"]
        threads = min(cores, oracle.max_threads(), B * H)

        def run(Ts):
            args = [bf16_to_bits(torch, x[kk][:, :Ts]) if x[kk].dtype == torch.bfloat16
                    else x[kk][:, :Ts].contiguous().cpu().numpy() for kk in keys]
            s0 = None if x["S0"] is None else x["S0"].cpu().numpy()
            t0 = time.perf_counter()
            oracle.kda_fwd(*args, S0=s0, num_threads=threads)
            return time.perf_counter() - t0

        cal = min(T, 512)
        dt = run(cal)
        Ts = int(min(T, max(cal, cal * target_s / max(dt, 1e-6))))
        dt = run(Ts) if Ts != cal else dt
        return {"value": B * Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"first {Ts} of {T} tokens of all {B} sequences, all {H} heads (fp64 token "
                          f"recurrence, OpenMP over (sequence, head)), {dt:.1f} s"}
    cu = np.asarray(x["cu_host"], dtype=np.int64)
    N = len(cu) - 1
    threads = min(cores, oracle.max_threads())

    def run(m):
        sl = slice(0, int(cu[m]))
        args = [bf16_to_bits(torch, x[kk][:, sl]) for kk in keys]
        t0 = time.perf_counter()
        oracle.kda_fwd(*args, cu_seqlens=cu[: m + 1].astype(np.int32), num_threads=threads)
        return time.perf_counter() - t0

    m = min(N, max(1, threads // units_per_seq))
    dt = run(m)
    while m < N and dt < target_s / 2:
        m = min(N, 2 * m)
        dt = run(m)
    return {"value": int(cu[m]) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {m} of {N} packed sequences ({int(cu[m])} tokens), all {H} heads "
                      f"(fp64 token recurrence, OpenMP over (sequence, head)), {dt:.1f} s"}


def bf16_to_bits(torch, t):
    from gated_delta_rule_62_amd.inputs import host_bits
    return host_bits(t)


def cpu_baseline_prefill(torch, q, k, v, la, beta, S0, target_s=10.0):
    """Time the fp64 CPU oracle on the first T_s tokens (all heads) of the same
    inputs; T_s is sized from a short calibration run to about target_s seconds."""
    import oracle
    T = q.shape[1]
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    H = q.shape[2]
    threads = min(cores, oracle.max_threads(), H)

    def run(Ts):
        args = [bf16_to_bits(torch, x[:, :Ts]) for x in (q, k, v, la, beta)]
        s0 = S0.detach().cpu().numpy()
        t0 = time.perf_counter()
        oracle.kda_fwd(*args, S0=s0, num_threads=threads)
        return time.perf_counter() - t0

    cal = min(T, 1024)
    dt = run(cal)
    Ts = int(min(T, max(cal, cal * target_s / max(dt, 1e-6))))
    Ts = max(CHUNK, (Ts // CHUNK) * CHUNK)
    dt = run(Ts)
    return {"value": Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {Ts} of {T} tokens, all {H} heads (fp64 token recurrence, "
                      f"OpenMP over heads), {dt:.1f} s"}


def cpu_baseline_decode(torch, steps_inputs, S, target_s=8.0):
    """Time the oracle's decode step on all sequences of the decode workload for
    as many of the same steps as fit in about target_s seconds of oracle time."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = min(cores, oracle.max_threads())
    S64 = S.detach().cpu().numpy().astype(np.float64)
    done, total = 0, 0.0
    while total < target_s and done < len(steps_inputs):
        x = [bf16_to_bits(torch, t) for t in steps_inputs[done]]
        ts = time.perf_counter()
        oracle.kda_step(*x, S64, num_threads=threads)
        total += time.perf_counter() - ts
        done += 1
    return {"value": done / total, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {done} steps of the decode workload, all {S.shape[0]}x{S.shape[1]} heads "
                      f"(fp64, OpenMP over heads), {total:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA layer here is built and timed on a single MI355X; "
              "--gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_62_amd import kda
    kda.load_library()
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ prefill (headline)
    from gated_delta_rule_62_amd import inputs
    w2 = inputs.WORKLOADS[2]
    B, T, H, d = w2.B, w2.T, w2.H, w2.D
    x = inputs.device_prefill(w2)
    q, k, v, la, beta, S0 = x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"]
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    ws_bytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, d, d, B, False, CHUNK)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        kda.kda_chunk_fwd(q, k, v, la, beta, S0, None, o=o, S_final=Sf, workspace=ws, chunk=CHUNK, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = time.perf_counter()
    torch.cuda.synchronize()
    e_all0 = torch.cuda.Event(enable_timing=True)
    e_all1 = torch.cuda.Event(enable_timing=True)
    e_all0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    e_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_total = e_all0.elapsed_time(e_all1)
    ms_step = ms_total / args.steps
    call_ms = sorted(a.elapsed_time(b) for a, b in ev)
    call_avg_ms = sum(call_ms) / len(call_ms)
    call_med_ms, call_min_ms = call_ms[len(call_ms) // 2], call_ms[0]
    tokens = B * T
    value = tokens / (ms_step / 1e3)
    flops = prefill_alg_flops_per_token_head(d) * tokens * H
    tile_flops = prefill_tile_flops_per_token_head(d) * tokens * H
    byts = prefill_alg_bytes(tokens, H, d, B, True)
    tflops = flops / (call_avg_ms / 1e3) / 1e12
    tile_tflops = tile_flops / (call_avg_ms / 1e3) / 1e12
    gbs = byts / (call_avg_ms / 1e3) / 1e9

    # ------------------------------------------------------------------ the other prefill workloads
    # The forward of the remaining prefill workloads, each timed call by call (median and min of
    # `steps` calls after `warmup`), with its own roofline and oracle sample.
    del o
    prefill_workloads = {}

    def other_prefill(key, w, C, label, in_bytes=2, out_bytes=2, as_packed=False):
        xw = inputs.device_prefill(w)
        if as_packed:   # the equal-length batch passed as packed sequences (cu_seqlens)
            xw["cu_seqlens"] = torch.arange(0, xw["B"] * xw["T"] + 1, xw["T"], dtype=torch.int32, device="cuda")
        Bw, Tw, Hw, dw, Nw = xw["B"], xw["T"], xw["H"], xw["D"], xw["N"]
        odt = torch.bfloat16 if out_bytes == 2 else torch.float32
        ow = torch.empty((Bw, Tw, Hw, dw), dtype=odt, device="cuda")
        Sw = torch.empty((Nw, Hw, dw, dw), dtype=torch.float32, device="cuda")
        wsw = torch.empty(kda.kda_chunk_fwd_workspace_bytes(Bw, Tw, Hw, dw, dw, Nw, xw["cu_seqlens"] is not None, C),
                          dtype=torch.uint8, device="cuda")

        def run():
            kda.kda_chunk_fwd(xw["q"], xw["k"], xw["v"], xw["log_alpha"], xw["beta"], xw["S0"], xw["cu_seqlens"],
                              o=ow, S_final=Sw, workspace=wsw, chunk=C, stream=stream)
        t = timed_calls(torch, run, stream, max(3, args.warmup // 2), args.steps)
        line = prefill_line(label, Bw * Tw, Hw, dw, Nw, xw["S0"] is not None, C, t, in_bytes, out_bytes)
        line["config"] = {"workload": w.name, "B": Bw, "T": Tw, "H": Hw, "d_k": dw, "d_v": dw, "chunk": C,
                          "sequences": Nw, "in_dtype": w.dtype, "out_dtype": "bf16" if out_bytes == 2 else "fp32",
                          "packed": xw["cu_seqlens"] is not None}
        if as_packed:
            line["cpu_baseline"] = "the headline line's (same batch)"
        elif not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_batch(torch, xw)
        cw = counted_workload(key)
        if cw is not None:
            line["roofline"]["traffic"] = cw["traffic"]
            line["roofline"]["traffic_vs_algorithmic"] = cw["traffic"] / line["roofline"]["bytes_per_call"]
            line["counters"] = {"mfma_busy": cw["mfma_busy"], "valu_busy": cw["valu_busy"], "kernels": cw["kernels"]}
        prefill_workloads[key] = line
        del xw, ow, Sw, wsw
        torch.cuda.empty_cache()

    other_prefill("tiny_fp32", inputs.WORKLOADS[0], 64,
                  "tiny fp32 prefill: B=1, T=256, H=2, d=64, fp32 in/out, chunk 64", in_bytes=4, out_bytes=4)
    other_prefill("train_prefill_c64", inputs.WORKLOADS[1], 64,
                  "training-shape prefill: B=4, T=4096, H=16, d=128, bf16, chunk 64 (as the workload states)")
    other_prefill("train_prefill_c32", inputs.WORKLOADS[1], 32,
                  "training-shape prefill: B=4, T=4096, H=16, d=128, bf16, chunk 32 (the library default)")
    other_prefill("varlen_packed", inputs.WORKLOADS[4], 32,
                  "packed varlen prefill: 64 sequences U{512..16384} (525,197 tokens), H=32, d=128, bf16, "
                  "per-element decay mixture, chunk 32")
    other_prefill("long_context_packed", inputs.WORKLOADS[2], 32,
                  "long-context prefill passed as one packed sequence (cu_seqlens = [0, 65536]): B=1, "
                  "T=65536, H=32, d=128, bf16, S0 != 0, chunk 32", as_packed=True)
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")

    # ------------------------------------------------------------------ decode
    w3 = inputs.WORKLOADS[3]
    N, Hd = w3.num_seqs, w3.H
    S_init, steps_in = inputs.device_decode_steps(w3, args.decode_steps)
    S = torch.empty_like(S_init)
    od = torch.empty((N, Hd, d), dtype=torch.bfloat16, device="cuda")
    S.copy_(S_init)
    for i in range(8):
        kda.kda_recurrent_step(*steps_in[i], S, o=od, stream=stream)
    # The steps run back to back between two events on the launch stream; the average launch
    # duration is the bracketed time over the step count (an event recorded after every step adds
    # 2-3% to each 0.19 ms launch, so the per-step events are not used for the roofline).
    dec_ms = []
    for rep in range(3):
        S.copy_(S_init)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            kda.kda_recurrent_step(*steps_in[i], S, o=od, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms.append(e0.elapsed_time(e1))
    dec_ms.sort()
    dec_med = dec_ms[len(dec_ms) // 2]
    step_avg = dec_med / args.decode_steps
    dbytes = decode_alg_bytes(N, Hd, d)
    # the same steps captured once as a HIP graph and replayed (no host work per step)
    dg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dg):
        for i in range(args.decode_steps):
            kda.kda_recurrent_step(*steps_in[i], S, o=od)
    graph_ms = []
    for rep in range(3):
        S.copy_(S_init)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        dg.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms.append(g0.elapsed_time(g1))
    graph_ms.sort()
    graph_med = graph_ms[len(graph_ms) // 2]
    del dg
    decode = {
        "value": args.decode_steps / (dec_med / 1e3), "unit": "steps/s",
        "ms_per_step": dec_med / args.decode_steps,
        "hbm_gbs": dbytes / (step_avg / 1e3) / 1e9,
        "config": {"workload": "decode", "sequences": N, "H": Hd, "d_k": d, "d_v": d,
                   "steps": args.decode_steps, "in_dtype": "bf16", "out_dtype": "bf16", "state": "fp32"},
        "roofline": {"bound": "hbm", "achieved": dbytes / (step_avg / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dbytes / (step_avg / 1e3) / 1e9 / HBM_PEAK_GBS, "traffic": counted_traffic("decode"),
                     "kernel": "decode_step_kernel<128,BF16,bf16 out>", "avg_launch_us": step_avg * 1e3,
                     "bytes_per_launch": dbytes},
        "graph": {"what": f"the {args.decode_steps} steps replayed from one captured HIP graph",
                  "value": args.decode_steps / (graph_med / 1e3), "unit": "steps/s",
                  "ms_per_step": graph_med / args.decode_steps,
                  "hbm_frac": dbytes / (graph_med / args.decode_steps / 1e3) / 1e9 / HBM_PEAK_GBS},
    }

    # ------------------------------------------------------------------ fused prologue / epilogue
    # The headline call with every fused step on: q, k normalised in the kernels, beta and
    # log_alpha taken as logits (sigmoid; logsigmoid(a + 6) / 16), an output gate of N(0,1)
    # logits (one more bf16 tensor of o's shape to read).
    gate = torch.randn((B, T, H, d), device="cuda").to(torch.bfloat16)

    def call_fused():
        kda.kda_chunk_fwd_fused(q, k, v, la, beta, S0, None, qk_l2norm=True, beta_logits=True,
                                decay_logits=(6.0, 16.0), out_gate=gate, o=o, S_final=Sf, workspace=ws,
                                stream=stream)
    for _ in range(3):
        call_fused()
    torch.cuda.synchronize()
    ef0, ef1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ef0.record(stream)
    for _ in range(args.steps):
        call_fused()
    ef1.record(stream)
    torch.cuda.synchronize()
    fused_ms = ef0.elapsed_time(ef1) / args.steps

    # The same work unfused: the prologue and the output gate as separate elementwise passes over
    # HBM (torch's kernels, bf16 in and out) around the plain call.
    F = torch.nn.functional
    qn, kn, bn, lan = (torch.empty_like(t) for t in (q, k, beta, la))

    def call_unfused():
        qn.copy_(F.normalize(q, dim=-1))
        kn.copy_(F.normalize(k, dim=-1))
        torch.sigmoid(beta, out=bn)
        lan.copy_(F.logsigmoid(la.float() + 6.0) / 16.0)
        kda.kda_chunk_fwd(qn, kn, v, lan, bn, S0, None, o=o, S_final=Sf, workspace=ws, chunk=CHUNK, stream=stream)
        o.mul_(torch.sigmoid(gate))
    for _ in range(3):
        call_unfused()
    torch.cuda.synchronize()
    eu0, eu1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eu0.record(stream)
    for _ in range(args.steps):
        call_unfused()
    eu1.record(stream)
    torch.cuda.synchronize()
    unfused_ms = eu0.elapsed_time(eu1) / args.steps
    fused = {"counters": counted_workload("fused"),
             "workload": "long_context_prefill with q/k L2 norm, sigmoid beta, logsigmoid decay and an output "
                         "gate inside the kernels (kda_chunk_fwd_fused)",
             "ms_per_call": fused_ms, "vs_plain_call": fused_ms / ms_step,
             "tokens_per_s": tokens / (fused_ms / 1e3),
             "unfused_ms_per_call": unfused_ms,
             "unfused": "the same maps as separate elementwise passes (torch, bf16) around kda_chunk_fwd",
             "saving_ms": unfused_ms - fused_ms,
             # what separate passes cost at best: read and write q, k, log_alpha, beta once (bf16), and
             # read o and the gate and write o once, at the HBM peak
             "unfused_extra_hbm_floor_ms": tokens * H * ((3 * d + 1) * 2 * 2 + 3 * d * 2) / (HBM_PEAK_GBS * 1e9) * 1e3,
             "fused_extra_ms": fused_ms - ms_step}
    del gate, qn, kn, bn, lan

    # ------------------------------------------------------------------ scalar gate (Gated DeltaNet)
    # Workload 2's shape with one decay per (token, head): gdn_chunk_fwd.
    w6 = inputs.WORKLOADS[6]
    xg = inputs.device_prefill(w6)
    og = torch.empty((w6.B, w6.T, w6.H, d), dtype=torch.bfloat16, device="cuda")
    Sg = torch.empty((w6.B, w6.H, d, d), dtype=torch.float32, device="cuda")

    def call_gdn():
        kda.gdn_chunk_fwd(xg["q"], xg["k"], xg["v"], xg["log_alpha"], xg["beta"], xg["S0"], None, o=og, S_final=Sg,
                          workspace=ws, stream=stream)
    for _ in range(args.warmup):
        call_gdn()
    torch.cuda.synchronize()
    eg0, eg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eg0.record(stream)
    for _ in range(args.steps):
        call_gdn()
    eg1.record(stream)
    torch.cuda.synchronize()
    gdn_ms = eg0.elapsed_time(eg1) / args.steps
    # bytes: q, k, v and o (bf16 rows of d), one log_alpha and one beta per token-head, S0 and S_final
    gdn_bytes = w6.B * w6.T * w6.H * (4 * d * 2 + 2 + 2) + 2 * w6.B * w6.H * d * d * 4
    gdn_counters = counted_workload("gdn")
    gdn = {"counters": gdn_counters,
           "workload": "long_context_prefill, scalar gate: B=1, T=65536, H=32, d=128, bf16, "
                       "log_alpha [B,T,H] = logsigmoid(N(0,1)+6)/16",
           "value": w6.B * w6.T / (gdn_ms / 1e3), "unit": "tokens/s", "ms_per_call": gdn_ms,
           "roofline": {"bound": "hbm", "achieved": gdn_bytes / (gdn_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": gdn_bytes / (gdn_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                        "bytes_per_launch": gdn_bytes, "launch": "gdn_chunk_fwd (all prefill kernels of one call)"}}
    # The same call with every fused step on (q, k normalised in the kernels, beta and the one
    # log_alpha per token-head taken as logits, an output gate of N(0,1) logits).
    gate_g = torch.randn((w6.B, w6.T, w6.H, d), device="cuda").to(torch.bfloat16)

    def call_gdn_fused():
        kda.gdn_chunk_fwd_fused(xg["q"], xg["k"], xg["v"], xg["log_alpha"], xg["beta"], xg["S0"], None,
                                qk_l2norm=True, beta_logits=True, decay_logits=(6.0, 16.0), out_gate=gate_g,
                                o=og, S_final=Sg, workspace=ws, stream=stream)
    tgf = timed_calls(torch, call_gdn_fused, stream, 3, args.steps)
    gdn["fused"] = {"workload": "the same with the fused prologue and an output gate (gdn_chunk_fwd_fused)",
                    "ms_per_call_median": tgf["median"], "ms_per_call_min": tgf["min"],
                    "vs_plain_call": tgf["median"] / gdn_ms, "counters": counted_workload("gdn_fused")}
    del xg, og, Sg, gate_g

    # ------------------------------------------------------------------ continuation (serving shapes)
    # New tokens on top of a carried state: 256 sequences x 32 heads.  "verify4": 4 tokens each
    # (speculative verification; equal lengths, so kda_chunk_fwd runs them token by token);
    # "packed": workload 5, 1..32 tokens per sequence packed by cu_seqlens (chunked path).
    import dataclasses

    def cont_case(w, label):
        xc = inputs.device_prefill(w)
        Nc, Tc = xc["N"], xc["B"] * xc["T"]
        oc = torch.empty((xc["B"], xc["T"], w.H, w.D), dtype=torch.bfloat16, device="cuda")
        Sc = torch.empty_like(xc["S0"])

        def run():
            kda.kda_chunk_fwd(xc["q"], xc["k"], xc["v"], xc["log_alpha"], xc["beta"], xc["S0"], xc["cu_seqlens"],
                              o=oc, S_final=Sc, stream=stream)
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        # the call captured once as a HIP graph (workspace allocated beforehand), replayed reps times
        wsc = torch.empty(max(kda.kda_chunk_fwd_workspace_bytes(xc["B"], xc["T"], w.H, w.D, w.D, Nc, True), 256),
                          dtype=torch.uint8, device="cuda")
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            kda.kda_chunk_fwd(xc["q"], xc["k"], xc["v"], xc["log_alpha"], xc["beta"], xc["S0"], xc["cu_seqlens"],
                              o=oc, S_final=Sc, workspace=wsc)
        cg.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            cg.replay()
        e1.record()
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) / reps * 1e3
        del cg
        cb = prefill_alg_bytes(Tc, w.H, w.D, Nc, True)
        return {"workload": label, "sequences": Nc, "tokens": Tc, "H": w.H, "d": w.D, "us_per_call": us,
                "tokens_per_s": Tc / (us / 1e6), "bytes_per_call": cb, "hbm_gbs": cb / (us / 1e6) / 1e9,
                "frac_hbm": cb / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
                "us_per_call_graph_replay": us_graph, "tokens_per_s_graph_replay": Tc / (us_graph / 1e6)}

    w5 = inputs.WORKLOADS[5]
    continuation = {
        "verify4": cont_case(dataclasses.replace(w5, B=256, T=4, len_range=()),
                             "256 sequences x 4 new tokens (token-by-token kernel)"),
        "packed": cont_case(w5, "256 sequences x U{1..32} new tokens, packed (chunked kernel)"),
    }

    # ------------------------------------------------------------------ backward (training)
    # kda_chunk_bwd on the training-prefill workload (4 x 4096 tokens, 16 heads, d=128, bf16
    # inputs, bf16 gradients, fp32 dS0), upstream gradients d_o ~ N(0,1), dS_final ~ 0.02 N(0,1).
    w1 = inputs.WORKLOADS[1]
    xb = inputs.device_prefill(w1)
    gb = inputs.device_output_grads(xb, seed=1001)
    Bb, Tb, Hb = xb["B"], xb["T"], xb["H"]
    grads = {nm: torch.empty((Bb, Tb, Hb, d), dtype=torch.bfloat16, device="cuda")
             for nm in ("dq", "dk", "dv", "dlog_alpha")}
    grads["dbeta"] = torch.empty((Bb, Tb, Hb), dtype=torch.bfloat16, device="cuda")
    grads["dS0"] = torch.empty((Bb, Hb, d, d), dtype=torch.float32, device="cuda")
    wsb = torch.empty(kda.kda_chunk_bwd_workspace_bytes(Bb, Tb, Hb, d, d, Bb, False), dtype=torch.uint8,
                      device="cuda")

    def call_bwd():
        kda.kda_chunk_bwd(xb["q"], xb["k"], xb["v"], xb["log_alpha"], xb["beta"], gb["d_o"], None, None,
                          gb["dS_final"], grads=grads, workspace=wsb, stream=stream)
    for _ in range(3):
        call_bwd()
    torch.cuda.synchronize()
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record(stream)
    for _ in range(args.steps):
        call_bwd()
    eb1.record(stream)
    torch.cuda.synchronize()
    bwd_ms = eb0.elapsed_time(eb1) / args.steps
    bwd_flops = backward_alg_flops_per_token_head(d) * Bb * Tb * Hb
    bwd_bytes = backward_alg_bytes(Bb * Tb, Hb, d, Bb)
    backward = {
        "workload": "train_prefill backward: B=4, T=4096, H=16, d=128, bf16 inputs and gradients, "
                    "fp32 dS0, kda_chunk_bwd (all kernels of one call)",
        "value": Bb * Tb / (bwd_ms / 1e3), "unit": "tokens/s", "ms_per_call": bwd_ms,
        # The method's intensity (about 199 flop/B) is below MI355X's ridge (2500 TFLOP/s / 8 TB/s
        # = 312 flop/B), so HBM bounds it.  The MFMA fractions are side figures: against the bf16
        # peak, and against a third of it (each product here is three split-bf16 MFMAs).
        "roofline": {"bound": "hbm", "achieved": bwd_bytes / (bwd_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": bwd_bytes / (bwd_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "bytes_per_call": bwd_bytes, "traffic": counted_traffic("backward"),
                     "mfma_tflops": bwd_flops / (bwd_ms / 1e3) / 1e12,
                     "mfma_frac": bwd_flops / (bwd_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                     "mfma_frac_split_peak": bwd_flops / (bwd_ms / 1e3) / 1e12 / (BF16_PEAK_TFLOPS / 3),
                     "flops_per_call": bwd_flops,
                     "flop_convention": f"{backward_alg_flops_per_token_head(d)} per token-head "
                                        "(20 d^2 + 32 C d), each product as three bf16 MFMAs"},
        "workspace_bytes": wsb.numel(),
    }

    # The fused layer's gradient on the same shape (kda_chunk_bwd_fused): raw q, k ~ 3 N(0,1),
    # beta and decay logits, an output gate of N(0,1) logits; the maps' chain rule around the
    # rule's gradient, with the ungated output recomputed for the gate's gradient.
    gen = torch.Generator(device="cuda").manual_seed(1003)
    rn = lambda *shape, s=1.0: (s * torch.randn(shape, device="cuda", generator=gen)).to(torch.bfloat16)
    raw = {"q": rn(Bb, Tb, Hb, d, s=3.0), "k": rn(Bb, Tb, Hb, d, s=3.0), "la": rn(Bb, Tb, Hb, d),
           "b": rn(Bb, Tb, Hb)}
    gf = rn(Bb, Tb, Hb, d)
    fgrads = dict(grads)
    fgrads["dgate"] = torch.empty((Bb, Tb, Hb, d), dtype=torch.bfloat16, device="cuda")
    wsf = torch.empty(kda.kda_chunk_bwd_fused_workspace_bytes(Bb, Tb, Hb, d, d, Bb, False, has_out_gate=True),
                      dtype=torch.uint8, device="cuda")

    def call_bwd_fused():
        kda.kda_chunk_bwd_fused(raw["q"], raw["k"], xb["v"], raw["la"], raw["b"], gb["d_o"], None, None,
                                gb["dS_final"], qk_l2norm=True, beta_logits=True, decay_logits=(6.0, 16.0),
                                out_gate=gf, grads=fgrads, workspace=wsf, stream=stream)
    tbf = timed_calls(torch, call_bwd_fused, stream, 3, args.steps)
    backward["fused"] = {
        "workload": "the same shape through kda_chunk_bwd_fused: q/k L2 norm, sigmoid beta, logsigmoid decay "
                    "and an output gate (bf16 raw inputs and gradients)",
        "ms_per_call_median": tbf["median"], "ms_per_call_min": tbf["min"],
        "value": Bb * Tb / (tbf["median"] / 1e3), "unit": "tokens/s",
        "vs_plain_call": tbf["median"] / bwd_ms, "workspace_bytes": wsf.numel()}
    del xb, gb, grads, wsb, gf, raw, fgrads, wsf
    torch.cuda.empty_cache()

    # The long-context shape's backward (1 x 65,536 tokens, 32 heads): past the workspace limit
    # it runs in windows of chunks (8 of 256 here), a forward sweep keeping each window's entry
    # state and the windows from last to first; timed over a few calls.
    x2 = inputs.device_prefill(inputs.WORKLOADS[2])
    g2 = inputs.device_output_grads(x2, seed=1002)
    B2, T2, H2 = x2["B"], x2["T"], x2["H"]
    grads2 = {nm: torch.empty((B2, T2, H2, d), dtype=torch.bfloat16, device="cuda")
              for nm in ("dq", "dk", "dv", "dlog_alpha")}
    grads2["dbeta"] = torch.empty((B2, T2, H2), dtype=torch.bfloat16, device="cuda")
    grads2["dS0"] = torch.empty((B2, H2, d, d), dtype=torch.float32, device="cuda")
    ws2 = torch.empty(kda.kda_chunk_bwd_workspace_bytes(B2, T2, H2, d, d, B2, False), dtype=torch.uint8,
                      device="cuda")

    def call_bwd2():
        kda.kda_chunk_bwd(x2["q"], x2["k"], x2["v"], x2["log_alpha"], x2["beta"], g2["d_o"], x2["S0"], None,
                          g2["dS_final"], grads=grads2, workspace=ws2, stream=stream)
    t2 = timed_calls(torch, call_bwd2, stream, 1, 3)
    b2_bytes = backward_alg_bytes(B2 * T2, H2, d, B2)
    backward["long_context"] = {
        "workload": "long_context backward: B=1, T=65536, H=32, d=128, bf16 inputs and gradients, S0 != 0, "
                    "kda_chunk_bwd", "value": B2 * T2 / (t2["median"] / 1e3), "unit": "tokens/s",
        "ms_per_call_median": t2["median"], "ms_per_call_min": t2["min"],
        "hbm_frac": b2_bytes / (t2["median"] / 1e3) / 1e9 / HBM_PEAK_GBS,
        "workspace_bytes": ws2.numel(),
        "workspace_bytes_one_pass": 2048 * H2 * 4 * (Rec128 + 2 * d * d + 2 * 32 * d) + H2 * 4 * d * d,
    }
    del x2, g2, grads2, ws2
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ CPU baselines (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(torch, q, k, v, la, beta, S0)
        S.copy_(S_init)
        decode["cpu_baseline"] = cpu_baseline_decode(torch, steps_in, S_init)

    plan_G = "segments" if ws_bytes > 0 else "single pass"
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long_context_prefill", "B": B, "T": T, "H": H, "d_k": d, "d_v": d,
                   "chunk": CHUNK, "in_dtype": "bf16", "out_dtype": "bf16", "state": "fp32", "S0": "0.02*N(0,1)",
                   "log_alpha": "logsigmoid(N(0,1)+6)/16",
                   "precision": "split-bf16 MFMA operands (hi+lo), fp32 accumulation and state",
                   "schedule": plan_G},
        # Arithmetic intensity of the method (about 93 flop/B here) is below MI355X's ridge
        # (2500 TFLOP/s / 8 TB/s = 312 flop/B), so HBM bounds it; the MFMA fractions follow.
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": counted_traffic("prefill"),
                     "launch": "kda_chunk_fwd (all prefill kernels of one call)",
                     "avg_launch_us": call_avg_ms * 1e3, "median_launch_us": call_med_ms * 1e3,
                     "min_launch_us": call_min_ms * 1e3, "bytes_per_launch": byts,
                     "mfma_tflops": tflops, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
                     "mfma_frac_dense_tile": tile_tflops / BF16_PEAK_TFLOPS,
                     "flop_convention": f"algorithmic {prefill_alg_flops_per_token_head(d)} / dense-tile "
                                        f"{prefill_tile_flops_per_token_head(d)} per token-head at C={CHUNK}",
                     "flops_per_launch": flops,
                     # matrix-core and vector-ALU busy fractions of the call's kernels (rocprofv3
                     # counters, profiles/kernel_counters.md), or null once the kernels changed
                     "counters": counted_workload("long_context")},
        "cpu_baseline": cpu,
        "prefill_workloads": prefill_workloads,
        "decode": decode,
        "fused_prologue": fused,
        "gdn": gdn,
        "continuation": continuation,
        "backward": backward,
        "wall_s": wall,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
