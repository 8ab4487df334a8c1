"""Plain fp64 CPU oracle for the KDA gated delta rule.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path
(``gated_delta_rule_62_amd``) never does, and this package imports nothing from it.

* ``kda_fwd`` / ``kda_step`` call the C oracle (``kda_oracle.c``), a token-by-token
  fp64 recurrence, OpenMP-parallel over independent (sequence, head) units.
* ``kda_bwd`` calls the C oracle's gradient: reverse mode of the same token
  recurrence, the chain rule applied to each step of a token in reverse order.
* ``twin`` is a second, independently written numpy implementation that uses the
  pages' matrix-product form instead of the delta form.

The recurrence is the fine-grained gated delta rule of "Decoding Hybrid Attention
Architectures" (intl.cloud.baidu.com article 9569726), section 3.4, in the delta
form of its section 3.2; see ``kda_oracle.h`` for the readings taken.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_kda.so")
SOURCES = [os.path.join(_HERE, "kda_oracle.c")]

F64, F32, BF16 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``liboracle_kda.so`` (plain gcc, OpenMP, no -ffast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp] + SOURCES + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load_library(path: str):
    """ctypes handle on a built oracle library (the default one, or a variant the
    tests compile from a modified copy of the source)."""
    lib = ctypes.CDLL(path)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
    lib.oracle_kda_fwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64p,
                                   i32, i32, i32, i32, i32, i32, vp, i32, vp, i32]
    lib.oracle_kda_fwd.restype = i32
    lib.oracle_kda_step.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, vp, i32, i32]
    lib.oracle_kda_step.restype = i32
    lib.oracle_kda_bwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64p,
                                   i32, i32, i32, i32, i32, i32, vp, i32, vp, i32,
                                   vp, vp, vp, vp, vp, vp, i32]
    lib.oracle_kda_bwd.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load_library(LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle inputs must be float64, float32 or bf16 bits (uint16), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, o_dtype=np.float32,
            num_threads: int = 0, lib=None):
    """Token recurrence over whole sequences.

    q, k, log_alpha: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H]; all of one
    dtype (float64, float32, or uint16 holding bf16 bits).  S0: [N, H, Dk, Dv] or
    None.  cu_seqlens: int sequence offsets (N+1) with B == 1, or None (N = B).
    Returns (o [B, T, H, Dv] in o_dtype, S_final [N, H, Dk, Dv] float64).
    """
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, log_alpha, beta)]
    dt = _dtype_code(arrs[0])
    if any(_dtype_code(a) != dt for a in arrs):
        raise TypeError("q, k, v, log_alpha, beta must share one dtype")
    q, k, v, log_alpha, beta = arrs
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (B, T, H, Dv) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.size - 1
    else:
        N = B
    s0 = None if S0 is None else np.ascontiguousarray(S0)
    if s0 is not None and s0.shape != (N, H, Dk, Dv):
        raise ValueError("S0 shape mismatch")
    od = np.dtype(o_dtype)
    o = np.zeros((B, T, H, Dv), dtype=od)
    Sf = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    rc = (lib or _load()).oracle_kda_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), dt,
        _ptr(s0), _dtype_code(s0) if s0 is not None else F64,
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if cu is not None else None,
        B, T, H, Dk, Dv, N, _ptr(o), F64 if od == np.float64 else F32, _ptr(Sf), int(num_threads))
    if rc != 0:
        raise ValueError("oracle_kda_fwd rejected its arguments")
    return o, Sf


def kda_step(q, k, v, log_alpha, beta, S, o_dtype=np.float32, num_threads: int = 0, lib=None):
    """One decode token.  q, k, log_alpha: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H].
    S: float64 [N, H, Dk, Dv], updated IN PLACE.  Returns o [N, H, Dv]."""
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, log_alpha, beta)]
    dt = _dtype_code(arrs[0])
    q, k, v, log_alpha, beta = arrs
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if S.dtype != np.float64 or not S.flags["C_CONTIGUOUS"] or S.shape != (N, H, Dk, Dv):
        raise ValueError("S must be a C-contiguous float64 [N, H, Dk, Dv] array")
    od = np.dtype(o_dtype)
    o = np.zeros((N, H, Dv), dtype=od)
    rc = (lib or _load()).oracle_kda_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), dt,
                                 _ptr(S), N, H, Dk, Dv, _ptr(o),
                                 F64 if od == np.float64 else F32, int(num_threads))
    if rc != 0:
        raise ValueError("oracle_kda_step rejected its arguments")
    return o


def kda_bwd(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None,
            num_threads: int = 0, lib=None):
    """Gradient of ``kda_fwd``'s (o, S_final) against the upstream gradients d_o
    [B, T, H, Dv] and dS_final [N, H, Dk, Dv] (None = zero).  Inputs as for
    ``kda_fwd``; d_o and dS_final may be float64, float32 or bf16 bits.  Returns a
    dict of float64 arrays dq, dk, dv, dlog_alpha, dbeta, dS0 shaped like q, k, v,
    log_alpha, beta and S0 ([N, H, Dk, Dv])."""
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, log_alpha, beta)]
    dt = _dtype_code(arrs[0])
    if any(_dtype_code(a) != dt for a in arrs):
        raise TypeError("q, k, v, log_alpha, beta must share one dtype")
    q, k, v, log_alpha, beta = arrs
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (B, T, H, Dv) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    d_o = np.ascontiguousarray(d_o)
    if d_o.shape != (B, T, H, Dv):
        raise ValueError("d_o shape mismatch")
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.size - 1
    else:
        N = B
    s0 = None if S0 is None else np.ascontiguousarray(S0)
    dsf = None if dS_final is None else np.ascontiguousarray(dS_final)
    for a in (s0, dsf):
        if a is not None and a.shape != (N, H, Dk, Dv):
            raise ValueError("state shape mismatch")
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
               dlog_alpha=np.zeros((B, T, H, Dk)), dbeta=np.zeros((B, T, H)),
               dS0=np.zeros((N, H, Dk, Dv)))
    rc = (lib or _load()).oracle_kda_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), dt,
        _ptr(s0), _dtype_code(s0) if s0 is not None else F64,
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if cu is not None else None,
        B, T, H, Dk, Dv, N, _ptr(d_o), _dtype_code(d_o),
        _ptr(dsf), _dtype_code(dsf) if dsf is not None else F64,
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
        _ptr(out["dbeta"]), _ptr(out["dS0"]), int(num_threads))
    if rc != 0:
        raise ValueError("oracle_kda_bwd rejected its arguments")
    return out
