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
// Equal-length batches of at most this many tokens per sequence take the token-by-token
// kernel (on MI355X it beats a one-chunk pass up to about 7 tokens: the state traffic is the
// same and the chunk's fixed intra-chunk work is skipped).
constexpr int kRecurrentMaxT = 4;

inline bool chunk_supported(int c) { return c == 0 || c == 32 || c == 64; }

// How a prefill call is split into kernels.
//  G == 1: one pass, one workgroup per (sequence, head).
//  G  > 1 (equal-length batches only): every sequence is cut into G segments of
//         cps chunks.  Pass 1 runs segments 0..G-2 from a zero state and also
//         carries the segment's transition matrix; a small combine kernel chains
//         the segment entry states; pass 2 reruns every segment from its true
//         entry state and writes o and S_final.
//         With split0, segment 0 needs no summary: its output pass runs on a second
//         stream beside pass 1 (which then covers segments 1..G-2) and leaves its exit
//         state as segment 1's entry, so pass 2 covers segments 1..G-1.  Both passes then
//         fill the chip with one segment more than the plain schedule.
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
    size_t off_phi = 0, off_sloc = 0, off_se = 0, off_order = 0;
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
};

PrefillPlan plan_prefill(int B, int T, int H, int D, int N, bool varlen, int chunk);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream);

hipError_t launch_decode(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const void* g, const void* b, const float* S_in,
                         float* S_out, void* o, int units, hipStream_t stream, bool scalar_gate,
                         const Fusion* fusion = nullptr);

hipError_t launch_recurrent_fwd(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                                const void* v, const void* g, const void* b, const float* S0,
                                const int32_t* cu, int T, int H, int units, void* o, float* S_final,
                                hipStream_t stream, bool scalar_gate);

}  // namespace kda
