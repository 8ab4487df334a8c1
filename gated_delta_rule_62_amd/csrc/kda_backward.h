// kda_backward.h -- host-side plan and launcher of the chunkwise backward
// (kda_backward.hip), shared with kda_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Gradient of the chunkwise prefill (kda_backward.hip).  Chunk length 32.
struct BackwardArgs {
    const void *q, *k, *v, *g, *beta, *dO;   // inputs and the output gradient, in dtype
    const float *S0, *dS_final;              // [N, H, D, D] or nullptr (zeros)
    const int32_t* cu;                       // packed sequence offsets or nullptr
    void *dq, *dk, *dv, *dg, *dbeta;         // gradients, out dtype
    float* dS0;                              // [N, H, D, D] or nullptr
    // workspace views (set by launch_backward)
    float *prep = nullptr, *states = nullptr, *dstates = nullptr;
    float *rbuf = nullptr, *debuf = nullptr;  // per (chunk, head): R = V - K S and dE, C x Dv
    int32_t* seq_chunk0 = nullptr;
    // Workspace slots are head-major, so the chunks of one (sequence, head) are adjacent:
    // per-chunk data (records, dS_next, R, dE) at h * ncs + chunk, states at h * nss + slot.
    int ncs = 0, nss = 0;
    // Windowed plan (W > 0, equal-length batches): the kernels cover chunks [w0, w0 + W) of
    // every sequence, window wi; per-chunk slots n * W + (i - w0), state slots n * (W + 1) +
    // (i - w0).  ckpt holds the entry state of every window after the first, dcarry the state
    // gradient passed from a window to the one before it ([N * H, D, D] each).
    int W = 0, w0 = 0, wi = 0;
    float *ckpt = nullptr, *dcarry = nullptr;
    int B, T, H, D, N;
    bool in_bf16, out_bf16;
    bool scalar_gate = false;                // log_alpha and dlog_alpha are [B, T, H]
    bool split_fp32 = false;                 // fp32 inputs, split-bf16 products (a bf16-input bound)
};

struct BackwardPlan {
    size_t nc_max = 0;   // upper bound on the number of chunks
    int W = 0;           // chunks per sequence per window (0: one pass over every chunk)
    int n_win = 1;       // windows
    size_t off_seq = 0, off_prep = 0, off_states = 0, off_dstates = 0, off_r = 0, off_de = 0;
    size_t off_ckpt = 0, off_dcarry = 0;
    size_t workspace_bytes = 0;
};

// Workspace bound of the backward: a plan whose per-chunk data for every chunk would exceed it
// processes equal-length sequences in windows of chunks, last window first (the
// KDA_BWD_WORKSPACE_LIMIT environment variable, in bytes, overrides it).
constexpr size_t kBwdWorkspaceLimit = size_t(2) << 30;

BackwardPlan plan_backward(int B, int T, int H, int D, int N, bool varlen);
hipError_t launch_backward(BackwardArgs a, const BackwardPlan& plan, void* workspace, hipStream_t stream);

}  // namespace kda
