"""Seeded synthetic inputs for the KDA layer (host-side, numpy).

This module is the one piece shared by the HIP path's callers and by the oracle's
tests: it draws and shapes random inputs and holds none of the method's arithmetic
(no decay, no delta update, no chunking).  It imports numpy; the on-device draws
for full-size workloads import torch lazily.

Workloads (the five shapes the layer is measured and checked on):

  0  tiny fp32 prefill      B=1,  H=2,  T=256,    d=64,  fp32 in/out, S0=0
  1  training-shape prefill B=4,  H=16, T=4096,   d=128, bf16 in, S0=0
  2  long-context prefill   B=1,  H=32, T=65536,  d=128, bf16 in, S0 ~ 0.02*N(0,1)
  3  decode                 N=256 sequences, H=32, d=128, 1024 steps, bf16 in,
                            S ~ 0.02*N(0,1)
  4  packed varlen prefill  64 sequences, lengths U{512..16384}, H=32, d=128, bf16
  5  continuation           256 sequences of U{1..32} new tokens each on top of a carried
                            state (speculative verification / chunked continuation),
                            packed, H=32, d=128, bf16, S0 ~ 0.02*N(0,1)
  6  scalar-gate prefill    workload 2's shape with one decay per (token, head) (Gated
                            DeltaNet): log_alpha [B, T, H] = logsigmoid(N(0,1) + 6) / 16

Distributions: q, k ~ N(0,1) then L2-normalised per (token, head); v ~ N(0,1);
beta = sigmoid(N(0,1)); log_alpha = logsigmoid(N(0,1) + mu) / s per channel with
(mu, s) = (4, 8) except workload 2 (6, 16); workload 4 draws each element from an
even mixture of logsigmoid(N+4)/8 and logsigmoid(N)/2.  numpy PCG64
``default_rng(seed)``; draws are float32 and happen in the order lengths (4 only),
q, k, v, z_beta, z_alpha, z_alpha2 and mixture mask (4 only), S0.  Decode draws S0
first and then each step's q, k, v, z_beta, z_alpha in step order, so steps can be
streamed.  bf16 inputs are the round-to-nearest-even bf16 of the float32 value and
are carried as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_DEFAULT = 128


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str                 # "prefill" or "decode"
    B: int = 1
    T: int = 0
    H: int = 32
    D: int = 128
    dtype: str = "bf16"       # input dtype: "bf16" or "f32"
    mu: float = 4.0
    s: float = 8.0
    s0: bool = False
    mix: bool = False
    num_seqs: int = 0         # varlen sequences / decode sequences
    len_range: tuple = ()     # varlen length bounds (inclusive)
    steps: int = 0            # decode steps
    chunk: int = 64
    scalar_gate: bool = False # log_alpha drawn [B, T, H] (one decay per token and head)
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return self.index + 1


WORKLOADS = {
    0: Workload(0, "tiny_fp32_prefill", "prefill", B=1, T=256, H=2, D=64, dtype="f32"),
    1: Workload(1, "train_prefill", "prefill", B=4, T=4096, H=16, D=128),
    2: Workload(2, "long_context_prefill", "prefill", B=1, T=65536, H=32, D=128,
                mu=6.0, s=16.0, s0=True),
    3: Workload(3, "decode", "decode", H=32, D=128, s0=True, num_seqs=256, steps=1024),
    4: Workload(4, "varlen_packed_prefill", "prefill", H=32, D=128, mix=True,
                num_seqs=64, len_range=(512, 16384)),
    5: Workload(5, "continuation", "prefill", H=32, D=128, s0=True,
                num_seqs=256, len_range=(1, 32)),
    6: Workload(6, "gdn_long_context_prefill", "prefill", B=1, T=65536, H=32, D=128,
                mu=6.0, s=16.0, s0=True, scalar_gate=True),
}


# ---------------------------------------------------------------- bf16 bit helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bit patterns
    (finite inputs only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(x: np.ndarray) -> np.ndarray:
    """Exact float32 view of an input array (bf16 bits widen exactly)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# ---------------------------------------------------------------- transforms
def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _logsigmoid(x):
    x = x.astype(np.float64)
    return (np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


# ---------------------------------------------------------------- prefill
def make_prefill(w: Workload, seed: int | None = None, *, B=None, T=None, H=None, D=None,
                 num_seqs=None, len_range=None, s0=None, dtype=None, mu=None, s=None,
                 mix=None, lengths=None, scalar_gate=None):
    """Draw one prefill batch.  Keyword overrides shrink a workload for tests while
    keeping its recipe.  Returns a dict with q, k, v, log_alpha, beta (float32 or
    bf16 bits), S0 (float32 [N, H, D, D] or None), cu_seqlens (int32 [N+1] or None),
    and the shape fields."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    H = w.H if H is None else H
    D = w.D if D is None else D
    dtype = w.dtype if dtype is None else dtype
    mu = w.mu if mu is None else mu
    s = w.s if s is None else s
    mix = w.mix if mix is None else mix
    s0 = w.s0 if s0 is None else s0
    scalar_gate = w.scalar_gate if scalar_gate is None else scalar_gate
    varlen = bool(w.len_range) or lengths is not None or num_seqs is not None and len_range is not None
    if varlen:
        if lengths is None:
            lo, hi = len_range if len_range is not None else w.len_range
            n = num_seqs if num_seqs is not None else w.num_seqs
            lengths = rng.integers(lo, hi, endpoint=True, size=n)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(lengths.size + 1, dtype=np.int64)
        np.cumsum(lengths, out=cu[1:])
        B, T, N = 1, int(cu[-1]), int(lengths.size)
    else:
        B = w.B if B is None else B
        T = w.T if T is None else T
        N, cu = B, None
    shp = (B, T, H, D)
    q = _l2n(_normal(rng, shp))
    k = _l2n(_normal(rng, shp))
    v = _normal(rng, shp)
    beta = _sigmoid(_normal(rng, (B, T, H)))
    gshp = (B, T, H) if scalar_gate else shp
    g = _logsigmoid(_normal(rng, gshp) + np.float32(mu)) / np.float32(s)
    if mix:
        g_fast = _logsigmoid(_normal(rng, gshp)) / np.float32(2.0)
        pick = rng.random(gshp, dtype=np.float32) < 0.5
        g = np.where(pick, g_fast, g)
    S0 = (np.float32(0.02) * _normal(rng, (N, H, D, D))) if s0 else None
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                log_alpha=_cast(g, dtype), beta=_cast(beta, dtype), S0=S0,
                cu_seqlens=None if cu is None else cu.astype(np.int32),
                B=B, T=T, H=H, D=D, N=N, dtype=dtype, scalar_gate=scalar_gate)


def make_output_grads(d: dict, seed: int, *, dS_final: bool = True, scale: float = 1.0):
    """Upstream gradients for a prefill batch ``d`` (from ``make_prefill``): d_o ~ N(0,1)
    [B, T, H, D] in the batch's dtype and, if asked, dS_final ~ 0.02 N(0,1) [N, H, D, D]
    float32 (the scale of the recipe's S0).  Drawn from their own stream (``seed``) so
    the inputs of the batch stay as they are."""
    rng = np.random.default_rng(seed)
    shp = (d["B"], d["T"], d["H"], d["D"])
    do = np.float32(scale) * _normal(rng, shp)
    dsf = (np.float32(0.02) * _normal(rng, (d["N"], d["H"], d["D"], d["D"]))) if dS_final else None
    return dict(d_o=_cast(do, d["dtype"]), dS_final=dsf)


def make_raw_prefill(seed: int, *, B=1, T=64, H=2, D=128, dtype="bf16", num_seqs=None, lengths=None,
                     qk_scale=3.0, s0=True, scalar_gate=False):
    """Unconstrained inputs for the fused prologue: q, k ~ qk_scale * N(0,1) (not normalised),
    beta and log_alpha logits ~ N(0,1) (log_alpha [B, T, H, D], or [B, T, H] with scalar_gate),
    output-gate logits ~ N(0,1), v ~ N(0,1), S0 ~ 0.02 N(0,1); drawn in that order.  Same dict
    layout as make_prefill plus ``gate``."""
    rng = np.random.default_rng(seed)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(lengths.size + 1, dtype=np.int64)
        np.cumsum(lengths, out=cu[1:])
        B, T, N = 1, int(cu[-1]), int(lengths.size)
    else:
        N, cu = B, None
    shp = (B, T, H, D)
    q = np.float32(qk_scale) * _normal(rng, shp)
    k = np.float32(qk_scale) * _normal(rng, shp)
    v = _normal(rng, shp)
    beta = _normal(rng, (B, T, H))
    g = _normal(rng, (B, T, H) if scalar_gate else shp)
    gate = _normal(rng, shp)
    S0 = (np.float32(0.02) * _normal(rng, (N, H, D, D))) if s0 else None
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), log_alpha=_cast(g, dtype),
                beta=_cast(beta, dtype), gate=_cast(gate, dtype), S0=S0,
                cu_seqlens=None if cu is None else cu.astype(np.int32),
                B=B, T=T, H=H, D=D, N=N, dtype=dtype, scalar_gate=scalar_gate)


# ---------------------------------------------------------------- decode
class DecodeStream:
    """Seeded decode workload: ``state()`` gives the initial state, then ``step()``
    returns each step's inputs in order (so 1024 steps never need to be resident
    on the host at once)."""

    def __init__(self, w: Workload, seed: int | None = None, *, num_seqs=None, H=None, D=None,
                 dtype=None, mu=None, s=None, scalar_gate=False):
        self.rng = np.random.default_rng(w.seed if seed is None else seed)
        self.N = w.num_seqs if num_seqs is None else num_seqs
        self.H = w.H if H is None else H
        self.D = w.D if D is None else D
        self.dtype = w.dtype if dtype is None else dtype
        self.mu = w.mu if mu is None else mu
        self.s = w.s if s is None else s
        self.scalar_gate = scalar_gate
        self._S0 = np.float32(0.02) * _normal(self.rng, (self.N, self.H, self.D, self.D))

    def state(self) -> np.ndarray:
        return self._S0

    def step(self):
        shp = (self.N, self.H, self.D)
        q = _l2n(_normal(self.rng, shp))
        k = _l2n(_normal(self.rng, shp))
        v = _normal(self.rng, shp)
        beta = _sigmoid(_normal(self.rng, (self.N, self.H)))
        gshp = (self.N, self.H) if self.scalar_gate else shp
        g = _logsigmoid(_normal(self.rng, gshp) + np.float32(self.mu)) / np.float32(self.s)
        dt = self.dtype
        return dict(q=_cast(q, dt), k=_cast(k, dt), v=_cast(v, dt), log_alpha=_cast(g, dt),
                    beta=_cast(beta, dt))


# ---------------------------------------------------------------- on-device draws
# The full-size workloads (up to 2^31 elements per tensor) are drawn directly on
# the GPU with torch's seeded generator, same recipe, then the sampled slices a
# test checks are copied to the host so both sides read identical bf16 values.

def varlen_lengths(w: Workload, seed: int | None = None) -> np.ndarray:
    """Sequence lengths of a packed workload: integers(lo, hi, endpoint=True) from
    default_rng(seed) (seed 5 gives 525,197 tokens for workload 4)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lo, hi = w.len_range
    return rng.integers(lo, hi, endpoint=True, size=w.num_seqs)


def device_prefill(w: Workload, seed: int | None = None, device="cuda", *, lengths=None):
    """Full-size prefill batch of workload w drawn on the device (bf16 inputs).
    Returns a dict like make_prefill but with torch tensors; cu_seqlens is int32."""
    import torch
    F = torch.nn.functional
    seed = w.seed if seed is None else seed
    if w.len_range:
        lengths = varlen_lengths(w, seed) if lengths is None else np.asarray(lengths)
        cu = np.zeros(lengths.size + 1, dtype=np.int64)
        np.cumsum(lengths, out=cu[1:])
        B, T, N = 1, int(cu[-1]), int(lengths.size)
    else:
        B, T, N, cu = w.B, w.T, w.B, None
    H, D = w.H, w.D
    g = torch.Generator(device=device).manual_seed(seed)
    shp = (B, T, H, D)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def normal(shape):
        return torch.randn(shape, device=device, generator=g)

    q = F.normalize(normal(shp), dim=-1).to(dt)
    k = F.normalize(normal(shp), dim=-1).to(dt)
    v = normal(shp).to(dt)
    beta = torch.sigmoid(normal((B, T, H))).to(dt)
    gshp = (B, T, H) if w.scalar_gate else shp
    la = F.logsigmoid(normal(gshp) + w.mu) / w.s
    if w.mix:
        fast = F.logsigmoid(normal(gshp)) / 2.0
        pick = torch.rand(gshp, device=device, generator=g) < 0.5
        la = torch.where(pick, fast, la)
        del fast, pick
    la = la.to(dt)
    S0 = 0.02 * normal((N, H, D, D)) if w.s0 else None
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, S0=S0,
                cu_seqlens=None if cu is None else torch.tensor(cu, dtype=torch.int32, device=device),
                cu_host=cu, B=B, T=T, H=H, D=D, N=N, dtype=w.dtype, scalar_gate=w.scalar_gate)


def device_output_grads(x: dict, seed: int, device="cuda", *, dS_final: bool = True):
    """Upstream gradients for a device batch ``x`` (from ``device_prefill``), the recipe
    of ``make_output_grads``: d_o ~ N(0,1) in the batch's dtype, dS_final ~ 0.02 N(0,1)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    do = torch.randn((x["B"], x["T"], x["H"], x["D"]), device=device, generator=g).to(dt)
    dsf = 0.02 * torch.randn((x["N"], x["H"], x["D"], x["D"]), device=device, generator=g) if dS_final else None
    return dict(d_o=do, dS_final=dsf)


def device_decode_steps(w: Workload, steps: int, seed: int | None = None, device="cuda"):
    """Initial state and `steps` per-step input tuples (q, k, v, log_alpha, beta) of
    a decode workload, drawn on the device."""
    import torch
    F = torch.nn.functional
    g = torch.Generator(device=device).manual_seed(w.seed if seed is None else seed)
    N, H, D = w.num_seqs, w.H, w.D
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    S0 = 0.02 * torch.randn((N, H, D, D), device=device, generator=g)
    out = []
    for _ in range(steps):
        q = F.normalize(torch.randn((N, H, D), device=device, generator=g), dim=-1).to(dt)
        k = F.normalize(torch.randn((N, H, D), device=device, generator=g), dim=-1).to(dt)
        v = torch.randn((N, H, D), device=device, generator=g).to(dt)
        beta = torch.sigmoid(torch.randn((N, H), device=device, generator=g)).to(dt)
        la = (F.logsigmoid(torch.randn((N, H, D), device=device, generator=g) + w.mu) / w.s).to(dt)
        out.append((q, k, v, la, beta))
    return S0, out


def host_bits(t) -> np.ndarray:
    """Device tensor -> host numpy array (bf16 as uint16 bit patterns, else float32)."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
