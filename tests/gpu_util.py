"""Helpers for the GPU tests: host<->device marshalling and the parity metric.

Parity metric (per (sequence, head) slice, as stated for the KDA parity bar):
with s = rms(ref_slice), a slice passes iff max_i |x_i - ref_i| / (|ref_i| + s) <= tol.
The bound is 1e-4 for fp32-input workloads and 2e-3 for bf16-input / fp32-state
workloads.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16 = 2e-3


def to_dev(x, device="cuda"):
    """numpy float32 or bf16-bit (uint16) array -> torch tensor on the GPU."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if x.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return (t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.detach().cpu().numpy()


def slice_metric(x, ref, axes):
    """Worst per-slice normalised error; ``axes`` are the axes reduced inside a slice."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    s = np.sqrt(np.mean(ref ** 2, axis=axes, keepdims=True))
    s = np.where(s > 0, s, 1e-30)
    return float(np.max(np.abs(x - ref) / (np.abs(ref) + s))) if ref.size else 0.0


def o_metric(o, o_ref, cu_seqlens=None):
    """o: [B, T, H, Dv].  Slices are (sequence, head)."""
    B, T, H, Dv = o_ref.shape
    if cu_seqlens is None:
        return slice_metric(o, o_ref, axes=(1, 3))
    worst = 0.0
    cu = [int(c) for c in cu_seqlens]
    for n in range(len(cu) - 1):
        if cu[n + 1] > cu[n]:
            worst = max(worst, slice_metric(o[:, cu[n]:cu[n + 1]], o_ref[:, cu[n]:cu[n + 1]], axes=(1, 3)))
    return worst


def state_metric(S, S_ref):
    """S: [N, H, Dk, Dv].  Slices are (sequence, head)."""
    return slice_metric(S, S_ref, axes=(2, 3))
