// kda_launch.h -- host-side launch plans and launchers shared by kda_api.hip and
// the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kDefaultChunk = 32;     // chunk length C (tokens) when the caller passes 0
constexpr int kComputeUnits = 256;    // MI355X
constexpr int kMinChunksPerSegment = 4;
constexpr size_t kStatusBytes = 256;  // status word at the start of every prefill workspace
constexpr int kWaitLimit = 1 << 16;   // polls before a kernel's ordering wait gives up
// Equal-length batches of at most this many tokens per sequence take the token-by-token
// kernel (on MI355X it beats a one-chunk pass up to about 7 tokens: the state traffic is the
// same and the chunk's fixed intra-chunk work is skipped).
constexpr int kRecurrentMaxT = 4;
// Packed batches of at most this many sequences are ordered longest first exactly (one kernel,
// O(N) per sequence); larger ones by length buckets of 32 tokens (four small kernels, O(1) per
// sequence).
constexpr int kOrderExactMax = 4096;
constexpr int kOrderBuckets = 1024;

inline bool chunk_supported(int c) { return c == 0 || c == 32 || c == 64; }

// How a prefill call is split into kernels.
//  G == 1: one pass, one workgroup per (sequence, head).
//  G  > 1 (equal-length batches only): every sequence is cut into G segments of
//         cps chunks.  Pass 1 runs segments 0..G-2 from a zero state and also
//         carries the segment's transition matrix; a small combine kernel chains
//         the segment entry states; pass 2 reruns every segment from its true
//         entry state and writes o and S_final.
//         With split0, segment 0 needs no summary: its output pass runs in the same
//         launch as pass 1 (which then covers segments 1..G-2) and leaves its exit state
//         as segment 1's entry, so pass 2 covers segments 1..G-1.  Both passes then fill
//         the chip with one segment more than the plain schedule.
//  seg_items > 0 (packed batches of fewer than kComputeUnits (sequence, head) pairs, 32-token
//         chunks): the split schedule per sequence.  A first kernel reads cu_seqlens and writes
//         a segment table (the segment length and, per sequence, its segments and the prefix
//         sums that map workgroups to them); pass 1, the combine and pass 2 are launched with
//         seg_items * H workgroups each (the table's upper bound), the surplus ones exiting.
// Every plan's workspace starts with the call's status word (kStatusBytes reserved): the
// first kernel of the call clears it, and a workgroup whose bounded ordering wait gave up
// sets it to 1 (and writes NaN to what it stores from then on).
// Fused prologue / epilogue of the _fused entry points (flags as in kda_fusion).
struct Fusion {
    int flags = 0;                     // 1: L2-normalise q, k; 2: beta logits; 4: log_alpha logits
    float decay_bias = 0.f, decay_scale = 1.f;
    const void* out_gate = nullptr;    // output-gate logits shaped like o (in dtype)
};

struct PrefillPlan {
    int chunk = kDefaultChunk;
    int G = 1;
    int chunks = 0;        // chunks per sequence (equal-length case)
    int cps = 0;           // chunks per segment
    bool split0 = false;   // segment 0's output pass runs beside pass 1 (G >= 3)
    int seg_items = 0;     // packed batches cut into segments: pass-1 workgroups per head (0: one pass)
    size_t off_status = 0, off_phi = 0, off_sloc = 0, off_se = 0, off_order = 0, off_buckets = 0;
    size_t workspace_bytes = 0;
};

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const float* S0;
    const int32_t* cu;
    void* o;
    float* S_final;
    void* workspace;
    int B, T, H, D, N;
    bool in_bf16, out_bf16;
    bool scalar_gate = false;   // log_alpha is [B, T, H] (one decay per token and head)
    // fused prologue / epilogue: 1 = L2-normalise q and k, 2 = beta holds logits,
    // 4 = log_alpha holds logits a (decay logsigmoid(a + decay_bias) / decay_scale)
    int fuse_flags = 0;
    float decay_bias = 0.f, decay_scale = 1.f;
    const void* out_gate = nullptr;   // [B, T, H, D] output-gate logits (in dtype) or nullptr
    int wait_limit = kWaitLimit;      // polls before an ordering wait gives up
};

PrefillPlan plan_prefill(int B, int T, int H, int D, int N, bool varlen, int chunk);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream);
// Clears the status word of a prefill workspace (for calls that run no prefill kernel).
hipError_t clear_prefill_status(void* workspace, const PrefillPlan& plan, hipStream_t stream);

// Entry states of the segments of W chunks (32 tokens each) of an equal-length batch, without
// outputs: the summaries of segments 0..G-2 from a zero state (S_loc and the transition Phi) and
// the combine chaining them from S0 (nullptr: zero).  entry receives [G-1][N*H][D][D] fp32, the
// entry state of segment s at slot s - 1.  The workspace holds a status word and the summaries.
size_t segment_states_workspace_bytes(int N, int H, int D, int G);
hipError_t launch_segment_states(const PrefillArgs& a, int W, int G, float* entry, hipStream_t stream);

hipError_t launch_decode(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const void* g, const void* b, const float* S_in,
                         float* S_out, void* o, int units, hipStream_t stream, bool scalar_gate,
                         const Fusion* fusion = nullptr);

// The elementwise steps of the fused layer's gradient (kda_fused_bwd.hip): rows = tokens x
// heads of D (= Dk = Dv) values.  Raw inputs in dtype; the mapped inputs, the rule's fp32
// gradients and the ungated output in the workspace; the raw inputs' gradients out.
struct FusedBwdArgs {
    const void *q, *k, *v, *log_alpha, *beta, *d_o, *gate;    // raw inputs (gate may be null)
    float *qh, *kh, *vf, *la, *bt, *doc, *rq, *rk;            // pre: mapped inputs, 1/|q|, 1/|k|
    const float *dqh, *dkh, *dvf, *dla, *dbt, *oc;            // the rule's gradients, ungated o
    void *dq, *dk, *dv, *dla_out, *dbeta_out, *dgate;         // gradients of the raw inputs
    size_t rows = 0;
    int D = 128;
    int flags = 0;
    float decay_bias = 0.f, decay_scale = 1.f;
    bool in_bf16 = false, out_bf16 = false, scalar_gate = false;
};
hipError_t launch_fused_bwd_pre(const FusedBwdArgs& a, hipStream_t stream);
hipError_t launch_fused_bwd_post(const FusedBwdArgs& a, hipStream_t stream);

hipError_t launch_recurrent_fwd(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                                const void* v, const void* g, const void* b, const float* S0,
                                const int32_t* cu, int T, int H, int units, void* o, float* S_final,
                                hipStream_t stream, bool scalar_gate, const Fusion* fusion = nullptr);

}  // namespace kda
