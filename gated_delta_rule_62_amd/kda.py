"""Thin Python binding over libkda.so (argument marshalling only).

The functions carry the C ABI's names (include/kda.h) and take torch tensors that
live on the GPU; torch provides device memory and streams, every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, these raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

(KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_HIP,
 KDA_ERR_SCRATCH_LIMIT) = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES
KDA_F32, KDA_BF16 = 0, 1
CHUNK = 0          # library default chunk length (32 tokens); 32 and 64 are built

EXPORTED = ("kda_status_string", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_recurrent_step",
            "kda_recurrent_fwd", "gdn_chunk_fwd", "gdn_recurrent_step", "gdn_recurrent_fwd",
            "kda_chunk_fwd_fused", "kda_recurrent_step_fused", "kda_chunk_bwd_workspace_bytes",
            "kda_chunk_bwd", "gdn_chunk_bwd", "kda_chunk_fwd_noalloc", "gdn_chunk_fwd_fused",
            "gdn_recurrent_step_fused", "kda_recurrent_fwd_fused", "gdn_recurrent_fwd_fused",
            "kda_chunk_bwd_fused_workspace_bytes", "kda_chunk_bwd_fused", "gdn_chunk_bwd_fused_workspace_bytes",
            "gdn_chunk_bwd_fused")
KDA_FUSE_QK_L2NORM, KDA_FUSE_BETA_SIGMOID, KDA_FUSE_DECAY_LOGSIGMOID = 1, 2, 4


class Fusion(ctypes.Structure):
    """kda_fusion of include/kda.h."""
    _fields_ = [("flags", ctypes.c_int), ("decay_bias", ctypes.c_float), ("decay_scale", ctypes.c_float),
                ("out_gate", ctypes.c_void_p)]

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)}")


def load_library(path: str = LIB_PATH):
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_62_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i32] * 8
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp] * 7 + [i32] * 7 + [i32, i32] + [vp, vp] + [vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp] * 7 + [i32] * 7 + [i32, i32] + [vp, vp] + [vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_recurrent_step.argtypes = [vp] * 7 + [i32] * 4 + [i32, i32] + [vp, vp]
    lib.kda_recurrent_step.restype = i32
    lib.kda_recurrent_fwd.argtypes = [vp] * 7 + [i32] * 6 + [i32, i32] + [vp, vp, vp]
    lib.kda_recurrent_fwd.restype = i32
    fp = ctypes.POINTER(Fusion)
    lib.kda_chunk_fwd_fused.argtypes = [vp] * 7 + [i32] * 7 + [i32, i32] + [vp, vp] + [vp, sz, fp, vp]
    lib.kda_chunk_fwd_fused.restype = i32
    lib.kda_recurrent_step_fused.argtypes = [vp] * 7 + [i32] * 4 + [i32, i32] + [vp, fp, vp]
    lib.kda_recurrent_step_fused.restype = i32
    lib.gdn_chunk_fwd_fused.argtypes = lib.kda_chunk_fwd_fused.argtypes
    lib.gdn_chunk_fwd_fused.restype = i32
    lib.gdn_recurrent_step_fused.argtypes = lib.kda_recurrent_step_fused.argtypes
    lib.gdn_recurrent_step_fused.restype = i32
    for name in ("kda_recurrent_fwd_fused", "gdn_recurrent_fwd_fused"):
        getattr(lib, name).argtypes = [vp] * 7 + [i32] * 6 + [i32, i32] + [vp, vp, fp, vp]
        getattr(lib, name).restype = i32
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32] * 8
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp] * 9 + [i32] * 7 + [i32, i32] + [vp] * 6 + [vp, sz, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.gdn_chunk_bwd.argtypes = lib.kda_chunk_bwd.argtypes
    lib.gdn_chunk_bwd.restype = i32
    for pre in ("kda", "gdn"):
        getattr(lib, f"{pre}_chunk_bwd_fused_workspace_bytes").argtypes = [i32] * 9
        getattr(lib, f"{pre}_chunk_bwd_fused_workspace_bytes").restype = sz
        getattr(lib, f"{pre}_chunk_bwd_fused").argtypes = [vp] * 9 + [i32] * 7 + [i32, i32] + [vp] * 7 + [vp, sz, fp, vp]
        getattr(lib, f"{pre}_chunk_bwd_fused").restype = i32
    for pre in ("kda", "gdn"):
        getattr(lib, f"{pre}_chunk_fwd").argtypes = lib.kda_chunk_fwd.argtypes
        getattr(lib, f"{pre}_chunk_fwd").restype = i32
        getattr(lib, f"{pre}_recurrent_step").argtypes = lib.kda_recurrent_step.argtypes
        getattr(lib, f"{pre}_recurrent_step").restype = i32
        getattr(lib, f"{pre}_recurrent_fwd").argtypes = lib.kda_recurrent_fwd.argtypes
        getattr(lib, f"{pre}_recurrent_fwd").restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _keep_for(stream, *ts):
    """Tensors this wrapper allocated are used by work on ``stream``: when that is not the
    current stream, tell the caching allocator, so that their memory is not handed to other
    work before the library's kernels on ``stream`` are done with it."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in ts:
        if t is not None:
            t.record_stream(stream)


def workspace_status(workspace) -> int:
    """The status word a prefill call left at the start of its workspace (waits for the device):
    0 when every ordering wait inside the kernels completed, nonzero when some workgroup gave
    up a wait and wrote NaN to what it stored from then on."""
    return int(workspace[:4].view(torch.int32).item())


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs, has_cu_seqlens, chunk=CHUNK) -> int:
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs,
                                                            int(bool(has_cu_seqlens)), chunk))


def kda_chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, out_dtype=None, o=None,
                  S_final=None, workspace=None, chunk=CHUNK, stream=None, want_final=True, _fn="kda_chunk_fwd"):
    """Prefill.  q, k, log_alpha [B, T, H, Dk]; v [B, T, H, Dv]; beta [B, T, H]
    (one dtype: float32 or bfloat16); S0 [N, H, Dk, Dv] float32 or None;
    cu_seqlens int32 [N+1] on the GPU (B == 1) or None.  Returns (o, S_final)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o_new, sf_new = o is None, S_final is None and want_final
    if o_new:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    if sf_new:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check_dev(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_final, workspace)
    ws_need = kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, chunk)
    own = [o if o_new else None, S_final if sf_new else None]
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, Dk, Dv, N, chunk, _dtype_code(q.dtype), _dtype_code(o.dtype),
        _ptr(o), _ptr(S_final), _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, *own)
    return o, S_final


def kda_chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, o, S_final=None,
                          chunk=CHUNK, stream=None):
    """kda_chunk_fwd through the entry point that allocates nothing: the outputs are the
    caller's (o required, S_final optional) and the scratch is the library's fixed array."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check_dev(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_final)
    st = load_library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, Dk, Dv, N, chunk, _dtype_code(q.dtype), _dtype_code(o.dtype),
        _ptr(o), _ptr(S_final), _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return o, S_final


def kda_recurrent_step(q, k, v, log_alpha, beta, S_in, S_out=None, *, out_dtype=None, o=None,
                       stream=None, _fn="kda_recurrent_step"):
    """Decode one token.  q, k, log_alpha [N, H, Dk]; v [N, H, Dv]; beta [N, H];
    S_in [N, H, Dk, Dv] float32; S_out defaults to S_in (in place).  Returns (o, S_out)."""
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o_new = o is None
    if o_new:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=q.device)
    if S_out is None:
        S_out = S_in
    _check_dev(q, k, v, log_alpha, beta, S_in, S_out, o)
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S_in), _ptr(S_out),
        N, H, Dk, Dv, _dtype_code(q.dtype), _dtype_code(o.dtype), _ptr(o), _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, o if o_new else None)
    return o, S_out


def kda_recurrent_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, out_dtype=None, o=None,
                      S_final=None, stream=None, want_final=True, _fn="kda_recurrent_fwd", _fusion_arg=None):
    """Token-by-token forward over each sequence (the multi-token continuation of decode).
    Same tensors as kda_chunk_fwd; S_final may be S0 (in place).  Returns (o, S_final)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o_new, sf_new = o is None, S_final is None and want_final
    if o_new:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    if sf_new:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check_dev(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_final)
    extra = () if _fusion_arg is None else (ctypes.byref(_fusion_arg),)
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, Dk, Dv, N, _dtype_code(q.dtype), _dtype_code(o.dtype), _ptr(o), _ptr(S_final),
        *extra, _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, o if o_new else None, S_final if sf_new else None)
    return o, S_final


# Scalar-gated variant (Gated DeltaNet): log_alpha is [B, T, H] ([N, H] for a decode step);
# everything else as in the kda_ function of the same suffix.
def gdn_chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, **kw):
    return kda_chunk_fwd(q, k, v, log_alpha, beta, S0, cu_seqlens, _fn="gdn_chunk_fwd", **kw)


def gdn_recurrent_step(q, k, v, log_alpha, beta, S_in, S_out=None, **kw):
    return kda_recurrent_step(q, k, v, log_alpha, beta, S_in, S_out, _fn="gdn_recurrent_step", **kw)


def gdn_recurrent_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, **kw):
    return kda_recurrent_fwd(q, k, v, log_alpha, beta, S0, cu_seqlens, _fn="gdn_recurrent_fwd", **kw)


def kda_recurrent_fwd_fused(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, qk_l2norm=False,
                            beta_logits=False, decay_logits=None, out_gate=None, _fn="kda_recurrent_fwd_fused", **kw):
    """kda_recurrent_fwd with the fused prologue / epilogue (see kda_chunk_fwd_fused)."""
    if out_gate is not None:
        _check_dev(out_gate)
    f = _fusion(qk_l2norm, beta_logits, decay_logits, out_gate)
    o, Sf = kda_recurrent_fwd(q, k, v, log_alpha, beta, S0, cu_seqlens, _fn=_fn, _fusion_arg=f, **kw)
    return o, Sf


def gdn_recurrent_fwd_fused(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, **kw):
    """gdn_recurrent_fwd with the fused prologue / epilogue (log_alpha [B, T, H])."""
    return kda_recurrent_fwd_fused(q, k, v, log_alpha, beta, S0, cu_seqlens, _fn="gdn_recurrent_fwd_fused", **kw)


def _fusion(qk_l2norm=False, beta_logits=False, decay_logits=None, out_gate=None):
    f = Fusion()
    f.flags = (KDA_FUSE_QK_L2NORM if qk_l2norm else 0) | (KDA_FUSE_BETA_SIGMOID if beta_logits else 0) | \
        (KDA_FUSE_DECAY_LOGSIGMOID if decay_logits is not None else 0)
    f.decay_bias, f.decay_scale = (decay_logits if decay_logits is not None else (0.0, 1.0))
    f.out_gate = None if out_gate is None else out_gate.data_ptr()
    return f


def kda_chunk_fwd_fused(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, qk_l2norm=False,
                        beta_logits=False, decay_logits=None, out_gate=None, out_dtype=None, o=None,
                        S_final=None, workspace=None, chunk=CHUNK, stream=None, want_final=True,
                        _fn="kda_chunk_fwd_fused"):
    """Prefill with the fused prologue / epilogue: q, k unnormalised (qk_l2norm), beta as
    logits (beta_logits), log_alpha as logits a with decay_logits = (bias, scale) giving
    logsigmoid(a + bias) / scale, and an optional output gate (logits shaped like o)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o_new, sf_new = o is None, S_final is None and want_final
    if o_new:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    if sf_new:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_final, workspace, out_gate)
    ws_need = kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, chunk)
    own = [o if o_new else None, S_final if sf_new else None]
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    f = _fusion(qk_l2norm, beta_logits, decay_logits, out_gate)
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, Dk, Dv, N, chunk, _dtype_code(q.dtype), _dtype_code(o.dtype),
        _ptr(o), _ptr(S_final), _ptr(workspace), ws_bytes, ctypes.byref(f), _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, *own)
    return o, S_final


def kda_recurrent_step_fused(q, k, v, log_alpha, beta, S_in, S_out=None, *, qk_l2norm=False, beta_logits=False,
                             decay_logits=None, out_gate=None, out_dtype=None, o=None, stream=None,
                             _fn="kda_recurrent_step_fused"):
    """Decode one token with the fused prologue / epilogue (see kda_chunk_fwd_fused)."""
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o_new = o is None
    if o_new:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=q.device)
    if S_out is None:
        S_out = S_in
    _check_dev(q, k, v, log_alpha, beta, S_in, S_out, o, out_gate)
    f = _fusion(qk_l2norm, beta_logits, decay_logits, out_gate)
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S_in), _ptr(S_out),
        N, H, Dk, Dv, _dtype_code(q.dtype), _dtype_code(o.dtype), _ptr(o), ctypes.byref(f), _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, o if o_new else None)
    return o, S_out


def gdn_chunk_fwd_fused(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, **kw):
    """gdn_chunk_fwd with the fused prologue / epilogue (log_alpha [B, T, H]; see kda_chunk_fwd_fused)."""
    return kda_chunk_fwd_fused(q, k, v, log_alpha, beta, S0, cu_seqlens, _fn="gdn_chunk_fwd_fused", **kw)


def gdn_recurrent_step_fused(q, k, v, log_alpha, beta, S_in, S_out=None, **kw):
    """gdn_recurrent_step with the fused prologue / epilogue (log_alpha [N, H])."""
    return kda_recurrent_step_fused(q, k, v, log_alpha, beta, S_in, S_out, _fn="gdn_recurrent_step_fused", **kw)


def kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs, has_cu_seqlens, chunk=CHUNK) -> int:
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs,
                                                            int(bool(has_cu_seqlens)), chunk))


def kda_chunk_bwd(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None, *,
                  grad_dtype=torch.float32, grads=None, want_dS0=True, workspace=None, chunk=CHUNK,
                  stream=None, _fn="kda_chunk_bwd"):
    """Gradient of kda_chunk_fwd.  Inputs as for kda_chunk_fwd plus d_o [B, T, H, Dv]
    (the inputs' dtype) and dS_final [N, H, Dk, Dv] float32 or None.  Returns a dict
    dq, dk, dv, dlog_alpha, dbeta (grad_dtype) and dS0 (float32, or None when
    want_dS0 is False); ``grads`` may supply preallocated outputs under those names."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if d_o.dtype != q.dtype:
        raise TypeError("d_o must have the inputs' dtype")
    g = dict(grads or {})
    dev = q.device
    own = []
    for name, shape in (("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("dlog_alpha", log_alpha.shape),
                        ("dbeta", beta.shape)):
        if g.get(name) is None:
            g[name] = torch.empty(shape, dtype=grad_dtype, device=dev)
            own.append(g[name])
    if g.get("dS0") is None and want_dS0:
        g["dS0"] = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
        own.append(g["dS0"])
    _check_dev(q, k, v, log_alpha, beta, d_o, S0, cu_seqlens, dS_final, workspace, *g.values())
    ws_need = kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, chunk)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        own.append(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        _ptr(d_o), _ptr(dS_final), B, T, H, Dk, Dv, N, chunk, _dtype_code(q.dtype), _dtype_code(g["dq"].dtype),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]), _ptr(g.get("dS0")),
        _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, *own)
    return g


def gdn_chunk_bwd(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None, **kw):
    """Gradient of gdn_chunk_fwd: log_alpha and the returned dlog_alpha are [B, T, H]."""
    return kda_chunk_bwd(q, k, v, log_alpha, beta, d_o, S0, cu_seqlens, dS_final, _fn="gdn_chunk_bwd", **kw)


def kda_chunk_bwd_fused_workspace_bytes(B, T, H, Dk, Dv, num_seqs, has_cu_seqlens, chunk=CHUNK, has_out_gate=False,
                                        scalar_gate=False) -> int:
    fn = "gdn_chunk_bwd_fused_workspace_bytes" if scalar_gate else "kda_chunk_bwd_fused_workspace_bytes"
    return int(getattr(load_library(), fn)(B, T, H, Dk, Dv, num_seqs, int(has_cu_seqlens), chunk, int(has_out_gate)))


def kda_chunk_bwd_fused(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None, *,
                        qk_l2norm=False, beta_logits=False, decay_logits=None, out_gate=None,
                        grad_dtype=torch.float32, grads=None, want_dS0=True, workspace=None, chunk=CHUNK,
                        stream=None, _fn="kda_chunk_bwd_fused"):
    """Gradient of kda_chunk_fwd_fused with respect to its raw inputs (the maps and the gate
    as in kda_chunk_fwd_fused; d_o is the gradient of the gated output).  Returns a dict dq,
    dk, dv, dlog_alpha, dbeta, dgate (grad_dtype; dgate None without a gate) and dS0."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if d_o.dtype != q.dtype or (out_gate is not None and out_gate.dtype != q.dtype):
        raise TypeError("d_o and out_gate must have the inputs' dtype")
    g = dict(grads or {})
    dev = q.device
    own = []
    shapes = [("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("dlog_alpha", log_alpha.shape), ("dbeta", beta.shape)]
    if out_gate is not None:
        shapes.append(("dgate", out_gate.shape))
    for name, shape in shapes:
        if g.get(name) is None:
            g[name] = torch.empty(shape, dtype=grad_dtype, device=dev)
            own.append(g[name])
    if out_gate is None:
        g["dgate"] = None
    if g.get("dS0") is None and want_dS0:
        g["dS0"] = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
        own.append(g["dS0"])
    _check_dev(q, k, v, log_alpha, beta, d_o, S0, cu_seqlens, dS_final, workspace, out_gate,
               *[t for t in g.values() if t is not None])
    sg = _fn.startswith("gdn")
    ws_need = kda_chunk_bwd_fused_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, chunk,
                                                  out_gate is not None, sg)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 256), dtype=torch.uint8, device=dev)
        own.append(workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    fz = _fusion(qk_l2norm, beta_logits, decay_logits, out_gate)
    st = getattr(load_library(), _fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
        _ptr(d_o), _ptr(dS_final), B, T, H, Dk, Dv, N, chunk, _dtype_code(q.dtype), _dtype_code(g["dq"].dtype),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]), _ptr(g.get("dS0")),
        _ptr(g["dgate"]), _ptr(workspace), ws_bytes, ctypes.byref(fz), _stream_ptr(stream))
    if st != KDA_OK:
        raise KDAError(st, _fn)
    _keep_for(stream, *own)
    return g


def gdn_chunk_bwd_fused(q, k, v, log_alpha, beta, d_o, S0=None, cu_seqlens=None, dS_final=None, **kw):
    """Gradient of gdn_chunk_fwd_fused: log_alpha (decay logits) and dlog_alpha are [B, T, H]."""
    return kda_chunk_bwd_fused(q, k, v, log_alpha, beta, d_o, S0, cu_seqlens, dS_final, _fn="gdn_chunk_bwd_fused",
                               **kw)
