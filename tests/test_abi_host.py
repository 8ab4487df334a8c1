"""CPU-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/kda.h declares, and rejects bad arguments before any HIP call.
Pointer arguments here are fake addresses that the library must never touch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

from gated_delta_rule_62_amd import kda  # noqa: E402

FAKE = ctypes.c_void_p(1 << 40)          # 16-byte aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p((1 << 40) + 4)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so is not built")
    return kda.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:kda|gdn)_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(kda.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libkda.so"


def test_status_strings(lib):
    names = [kda.status_string(i) for i in range(6)]
    assert names == ["KDA_OK", "KDA_ERR_INVALID_ARGUMENT", "KDA_ERR_UNSUPPORTED",
                     "KDA_ERR_WORKSPACE_TOO_SMALL", "KDA_ERR_HIP", "KDA_ERR_SCRATCH_LIMIT"]


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The no-allocation prefill checks its fixed scratch limit (and the arguments) before any
    HIP call: a packed batch whose order table alone exceeds the limit is rejected."""
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=ctypes.c_void_p(3 << 40), B=1, T=0,
                 H=2, Dk=128, Dv=128, N=20_000_000, chunk=0, in_dt=kda.KDA_BF16, out_dt=kda.KDA_BF16,
                 o=ctypes.c_void_p(2 << 40), Sf=None)
        a.update(kw)
        return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"],
                                         a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["in_dt"],
                                         a["out_dt"], a["o"], a["Sf"], None)
    assert kda.kda_chunk_fwd_workspace_bytes(1, 0, 2, 128, 128, 20_000_000, True) > kda.NOALLOC_SCRATCH_BYTES
    assert call() == kda.KDA_ERR_SCRATCH_LIMIT
    # every equal-length plan fits: the segment summaries of the long-context shape are 48 MiB
    assert kda.kda_chunk_fwd_workspace_bytes(1, 1 << 20, 32, 128, 128, 1, False) <= kda.NOALLOC_SCRATCH_BYTES
    # argument errors are still reported first
    assert call(N=1, cu=None, T=64, Dk=96, Dv=96) == kda.KDA_ERR_UNSUPPORTED
    assert call(N=1, cu=None, T=64, q=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(N=0, cu=None, B=0, T=0) == kda.KDA_OK


def test_workspace_query_plans(lib):
    q = kda.kda_chunk_fwd_workspace_bytes
    st = 256   # every plan starts with the call's 256-byte status block
    # long context, 32 heads -> 3 matrices per unit and segment gap.  1024 chunks of 64 tokens
    # are cut into 8 segments (one workgroup per compute unit in each pass); 2048 chunks of 32
    # into 9, since segment 0's output pass runs beside the summaries of segments 1..7.
    assert q(1, 65536, 32, 128, 128, 1, False) == st + 3 * 32 * 8 * 128 * 128 * 4
    # the 64-token plan needs 7 segment gaps; its query also covers the 32-token evaluation of the
    # scalar-gate and fused calls, so it returns the larger of the two
    assert q(1, 65536, 32, 128, 128, 1, False, chunk=64) == max(st + 3 * 32 * 7 * 128 * 128 * 4,
                                                                st + 3 * 32 * 8 * 128 * 128 * 4)
    # training shape, 64 units: 5 segments of 32-token chunks (summaries of 1..3 beside 0)
    assert q(4, 4096, 16, 128, 128, 4, False) == st + 3 * 64 * 4 * 128 * 128 * 4
    # enough units to fill the chip: single pass, only the status block
    assert q(64, 4096, 32, 128, 128, 64, False) == st
    # packed sequences: the status block and an int32 order table (rounded to 256 bytes)
    assert q(1, 1000, 32, 128, 128, 64, True) == st + 256
    assert q(1, 1000, 32, 128, 128, 8, True) == st + 256          # 256 pairs fill the chip
    # more than 4096 sequences: the bucketed order's 2 x 1024 counters after the order table
    assert q(1, 100000, 2, 128, 128, 4096, True) == st + 4096 * 4
    assert q(1, 100000, 2, 128, 128, 5000, True) == st + 20224 + 8192
    assert q(1, 200, 32, 128, 128, 1, True) == st + 256           # 7 chunks: too short to cut
    # a packed chunk-64 call needs only the order table; the query also covers the 32-token
    # (segmented) evaluation of a scalar-gate or fused call with the same arguments
    assert q(1, 65536, 32, 128, 128, 1, True, chunk=64) == max(st + 256, q(1, 65536, 32, 128, 128, 1, True, chunk=32))
    # fewer than 256 (sequence, head) pairs, 32-token chunks: a segment table (4 + 5N + 2 int32,
    # rounded to 256 bytes) and 3 matrices per head for each of 256 / H segment slots
    mat = 128 * 128 * 4
    assert q(1, 65536, 32, 128, 128, 1, True) == st + 256 + 3 * 32 * 8 * mat
    assert q(1, 1000, 32, 128, 128, 7, True) == st + 256 + 3 * 32 * 8 * mat
    assert q(1, 24740, 8, 128, 128, 5, True) == st + 256 + 3 * 8 * 32 * mat
    assert q(1, 5000, 3, 64, 64, 60, True) == st + 1280 + 3 * 3 * 85 * 64 * 64 * 4   # 306 int32
    assert q(1, 65536, 32, 128, 128, 1, True) <= kda.NOALLOC_SCRATCH_BYTES
    # unsupported sizes report 0
    assert q(1, 64, 2, 96, 96, 1, False) == 0
    assert q(1, 64, 2, 128, 128, 1, False, chunk=16) == 0


def call_fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, Dk=128, Dv=128,
             N=1, chunk=64, in_dt=kda.KDA_BF16, out_dt=kda.KDA_BF16, o=ctypes.c_void_p(2 << 40),
             Sf=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"], a["T"],
                             a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["in_dt"], a["out_dt"], a["o"],
                             a["Sf"], a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_argument_errors(lib):
    assert call_fwd(lib, Dk=96, Dv=96) == kda.KDA_ERR_UNSUPPORTED
    assert call_fwd(lib, Dk=128, Dv=64) == kda.KDA_ERR_UNSUPPORTED
    assert call_fwd(lib, chunk=16) == kda.KDA_ERR_UNSUPPORTED
    assert call_fwd(lib, in_dt=7) == kda.KDA_ERR_UNSUPPORTED
    assert call_fwd(lib, q=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_fwd(lib, k=FAKE_MIS) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_fwd(lib, B=2, N=2, cu=ctypes.c_void_p(3 << 40)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_fwd(lib, N=3) == kda.KDA_ERR_INVALID_ARGUMENT            # N != B without cu_seqlens
    assert call_fwd(lib, o=FAKE) == kda.KDA_ERR_INVALID_ARGUMENT         # o aliases q
    assert call_fwd(lib, T=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    # segmented plan needs a workspace
    assert call_fwd(lib, T=65536, H=32) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    # every plan holds the call's status word: a workspace is always required
    assert call_fwd(lib) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert call_fwd(lib, ws=None, ws_bytes=256) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_fwd(lib, ws=FAKE_MIS, ws_bytes=256) == kda.KDA_ERR_INVALID_ARGUMENT
    # the workspace must not overlap an input or an output
    assert call_fwd(lib, ws=FAKE, ws_bytes=256) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_fwd(lib, ws=ctypes.c_void_p(2 << 40), ws_bytes=256) == kda.KDA_ERR_INVALID_ARGUMENT
    # N == 0 sequences: nothing to do, no HIP call
    assert call_fwd(lib, B=0, N=0, T=0) == kda.KDA_OK


def test_decode_argument_errors(lib):
    def step(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, Si=ctypes.c_void_p(4 << 40), So=ctypes.c_void_p(4 << 40),
                 N=2, H=2, Dk=128, Dv=128, i=kda.KDA_BF16, o_dt=kda.KDA_F32, o=ctypes.c_void_p(5 << 40))
        a.update(kw)
        return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["b"], a["Si"], a["So"], a["N"], a["H"],
                                      a["Dk"], a["Dv"], a["i"], a["o_dt"], a["o"], None)
    assert step(N=0) == kda.KDA_OK
    assert step(Dk=64, Dv=128) == kda.KDA_ERR_UNSUPPORTED
    assert step(Si=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert step(So=ctypes.c_void_p((4 << 40) + 256)) == kda.KDA_ERR_INVALID_ARGUMENT   # partial overlap
    assert step(o=ctypes.c_void_p((4 << 40) + 512)) == kda.KDA_ERR_INVALID_ARGUMENT    # o inside the state
    assert step(q=FAKE_MIS) == kda.KDA_ERR_INVALID_ARGUMENT


def test_recurrent_fwd_argument_errors(lib):
    def rec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=ctypes.c_void_p(4 << 40), cu=None, B=2, T=8, H=2,
                 Dk=128, Dv=128, N=2, in_dt=kda.KDA_BF16, out_dt=kda.KDA_F32, o=ctypes.c_void_p(5 << 40),
                 Sf=ctypes.c_void_p(4 << 40))
        a.update(kw)
        return lib.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"], a["T"],
                                     a["H"], a["Dk"], a["Dv"], a["N"], a["in_dt"], a["out_dt"], a["o"], a["Sf"],
                                     None)
    assert rec(B=0, N=0, T=0) == kda.KDA_OK                                   # nothing to do, no HIP call
    assert rec(Dk=96, Dv=96) == kda.KDA_ERR_UNSUPPORTED
    assert rec(out_dt=5) == kda.KDA_ERR_UNSUPPORTED
    assert rec(q=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert rec(v=FAKE_MIS) == kda.KDA_ERR_INVALID_ARGUMENT
    assert rec(N=3) == kda.KDA_ERR_INVALID_ARGUMENT                           # N != B without cu_seqlens
    assert rec(cu=ctypes.c_void_p(3 << 40)) == kda.KDA_ERR_INVALID_ARGUMENT   # cu_seqlens needs B == 1
    assert rec(Sf=ctypes.c_void_p((4 << 40) + 256)) == kda.KDA_ERR_INVALID_ARGUMENT   # partial overlap with S0
    assert rec(o=FAKE) == kda.KDA_ERR_INVALID_ARGUMENT                        # o aliases the inputs
    assert rec(o=ctypes.c_void_p((4 << 40) + 1024)) == kda.KDA_ERR_INVALID_ARGUMENT   # o inside the state


def test_fused_argument_errors(lib):
    def fwd(fusion, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, Dk=128, Dv=128,
                 N=1, chunk=0, in_dt=kda.KDA_BF16, out_dt=kda.KDA_BF16, o=ctypes.c_void_p(2 << 40),
                 Sf=None, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.kda_chunk_fwd_fused(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"],
                                       a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["in_dt"],
                                       a["out_dt"], a["o"], a["Sf"], a["ws"], a["ws_bytes"],
                                       ctypes.byref(fusion), None)

    def fz(flags=0, bias=0.0, scale=1.0, gate=None):
        f = kda.Fusion()
        f.flags, f.decay_bias, f.decay_scale, f.out_gate = flags, bias, scale, gate
        return f
    assert fwd(fz(flags=8)) == kda.KDA_ERR_INVALID_ARGUMENT                        # unknown flag
    assert fwd(fz(flags=kda.KDA_FUSE_DECAY_LOGSIGMOID, scale=0.0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert fwd(fz(flags=kda.KDA_FUSE_DECAY_LOGSIGMOID, scale=-2.0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert fwd(fz(gate=(3 << 40) + 4)) == kda.KDA_ERR_INVALID_ARGUMENT             # misaligned gate
    assert fwd(fz(gate=(2 << 40) + 64)) == kda.KDA_ERR_INVALID_ARGUMENT            # gate overlaps o
    # a 64-token request is accepted (evaluated with 32-token chunks): here it stops at the missing workspace
    assert fwd(fz(flags=kda.KDA_FUSE_QK_L2NORM), chunk=64) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    q = kda.kda_chunk_fwd_workspace_bytes
    for shape in ((1, 65536, 32, 128, 128, 1, False), (4, 4096, 16, 128, 128, 4, False), (1, 1000, 2, 64, 64, 3, True)):
        assert q(*shape, 64) >= q(*shape, 32)   # enough for either evaluation
    assert fwd(fz(flags=kda.KDA_FUSE_QK_L2NORM), B=0, N=0, T=0) == kda.KDA_OK       # nothing to do

    def step(fusion):
        return lib.kda_recurrent_step_fused(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(4 << 40),
                                            ctypes.c_void_p(4 << 40), 2, 2, 128, 128, kda.KDA_BF16, kda.KDA_F32,
                                            ctypes.c_void_p(5 << 40), ctypes.byref(fusion), None)
    assert step(fz(flags=16)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert step(fz(gate=(4 << 40) + 1024)) == kda.KDA_ERR_INVALID_ARGUMENT          # gate inside the state


def test_backward_workspace_query(lib):
    q = kda.kda_chunk_bwd_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    rec = 3 * 32 * 32 + 2 * 128 + 32 + 32 * 128               # floats per (chunk, head) record
    nc, H, D = 4 * 128, 16, 128                                # 4 sequences of 4096 tokens
    want = up(4 * nc * H * rec) + up(4 * (nc + 4) * H * D * D) + up(4 * nc * H * D * D) + 2 * up(4 * nc * H * 32 * D)
    assert q(4, 4096, 16, 128, 128, 4, False) == want
    # packed: a chunk-start table and room for ceil(T / 32) + N chunks
    nc = 1000 // 32 + 1 + 3
    want = up(4 * 4) + up(4 * nc * 2 * (3 * 32 * 32 + 2 * 64 + 32 + 32 * 64)) + \
        up(4 * (nc + 3) * 2 * 64 * 64) + up(4 * nc * 2 * 64 * 64) + 2 * up(4 * nc * 2 * 32 * 64)
    assert q(1, 1000, 2, 64, 64, 3, True) == want
    assert q(1, 64, 2, 96, 96, 1, False) == 0
    assert q(1, 64, 2, 128, 128, 1, False, chunk=64) == q(1, 64, 2, 128, 128, 1, False)
    assert q(1, 64, 2, 128, 128, 1, False, chunk=16) == 0


def test_backward_windowed_workspace(lib, monkeypatch):
    """Past the workspace limit (2 GiB) an equal-length backward runs in windows of W chunks per
    sequence: per (sequence, head) W chunks of data, W + 1 states, one checkpoint per later
    window and the carried state gradient."""
    q = kda.kda_chunk_bwd_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    rec = 3 * 32 * 32 + 2 * 128 + 32 + 32 * 128
    per_chunk = 4 * (rec + 2 * 128 * 128 + 2 * 32 * 128)
    st = 4 * 128 * 128

    def windowed(units, W, n_win):
        return (up(4 * units * W * rec) + up(st * units * (W + 1)) + up(st * units * W) +
                2 * up(4 * units * W * 32 * 128) + up(st * units * (n_win - 1)) + up(st * units))
    # training shape: 1.59 GB, under the limit: one pass, unchanged
    assert q(4, 4096, 16, 128, 128, 4, False) == up(4 * 512 * 16 * rec) + up(st * 516 * 16) + \
        up(st * 512 * 16) + 2 * up(4 * 512 * 16 * 32 * 128)
    # long context (2048 chunks, 32 heads): 6 windows of 342 chunks, 2.13 GB instead of 12.7 GB
    lc = q(1, 65536, 32, 128, 128, 1, False)
    assert lc == windowed(32, 342, 6) and lc <= 2 << 30
    assert 2048 * 32 * per_chunk > 12.6e9
    # a smaller limit (the environment override) gives smaller windows: 23 windows of 90 chunks
    monkeypatch.setenv("KDA_BWD_WORKSPACE_LIMIT", str(600 << 20))
    assert q(1, 65536, 32, 128, 128, 1, False) == windowed(32, 90, 23) <= 600 << 20
    assert q(2, 1000, 2, 128, 128, 2, False) == up(4 * 64 * 2 * rec) + up(st * 66 * 2) + \
        up(st * 64 * 2) + 2 * up(4 * 64 * 2 * 32 * 128)   # 2 x 32 chunks: one pass
    # no window fits 4 MiB: the least, 8 windows of 4 chunks (5.46 MB)
    monkeypatch.setenv("KDA_BWD_WORKSPACE_LIMIT", str(4 << 20))
    assert q(2, 1000, 2, 128, 128, 2, False) == windowed(4, 4, 8)
    # packed batches keep one pass
    assert q(1, 1000, 2, 64, 64, 3, True) > 0


def test_backward_argument_errors(lib):
    outs = {n: ctypes.c_void_p((10 + i) << 40) for i, n in enumerate(("dq", "dk", "dv", "dg", "db", "dS0"))}

    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, do=ctypes.c_void_p(2 << 40),
                 dSf=None, B=2, T=64, H=2, Dk=128, Dv=128, N=2, chunk=0, in_dt=kda.KDA_BF16,
                 g_dt=kda.KDA_F32, ws=ctypes.c_void_p(8 << 40), ws_bytes=1 << 40)
        a.update(outs)
        a.update(kw)
        return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["do"], a["dSf"],
                                 a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["in_dt"],
                                 a["g_dt"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dS0"], a["ws"],
                                 a["ws_bytes"], None)
    assert bwd(B=0, N=0, T=0) == kda.KDA_OK                                    # nothing to do, no HIP call
    assert bwd(Dk=96, Dv=96) == kda.KDA_ERR_UNSUPPORTED
    assert bwd(chunk=16) == kda.KDA_ERR_UNSUPPORTED
    assert bwd(chunk=64, B=0, N=0, T=0) == kda.KDA_OK   # the forward's 64-token chunks: evaluated at 32
    assert bwd(g_dt=3) == kda.KDA_ERR_UNSUPPORTED
    assert bwd(do=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert bwd(dk=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert bwd(dv=FAKE_MIS) == kda.KDA_ERR_INVALID_ARGUMENT
    assert bwd(N=3) == kda.KDA_ERR_INVALID_ARGUMENT                            # N != B without cu_seqlens
    assert bwd(cu=ctypes.c_void_p(3 << 40)) == kda.KDA_ERR_INVALID_ARGUMENT    # cu_seqlens needs B == 1
    assert bwd(dq=FAKE) == kda.KDA_ERR_INVALID_ARGUMENT                        # output aliases an input
    assert bwd(dk=ctypes.c_void_p((10 << 40) + 64)) == kda.KDA_ERR_INVALID_ARGUMENT   # outputs overlap
    assert bwd(dS0=ctypes.c_void_p((8 << 40) + 4096)) == kda.KDA_ERR_INVALID_ARGUMENT  # inside the workspace
    assert bwd(dSf=ctypes.c_void_p(15 << 40), dS0=ctypes.c_void_p((15 << 40) + 1024)) == \
        kda.KDA_ERR_INVALID_ARGUMENT                                           # dS0 overlaps dS_final
    assert bwd(ws_bytes=1024) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(ws=None, ws_bytes=0) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
