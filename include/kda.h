/*
 * kda.h -- C ABI of libkda.so: the KDA (fine-grained gated delta rule) layer on
 * AMD Instinct MI355X (gfx950), chunkwise prefill and single-token decode.
 *
 * The operation.  Per sequence and head, over tokens t in order, with state
 * S in R^{Dk x Dv}, keys/queries in R^{Dk}, values in R^{Dv}, a scalar write
 * strength beta_t and a per-key-channel decay alpha_t = exp(log_alpha_t):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * This is the fine-grained gated delta rule of "Decoding Hybrid Attention
 * Architectures" (intl.cloud.baidu.com article 9569726), section 3.4 (and
 * "Technical Analysis and Engineering Practices for Novel Hybrid Linear Attention
 * Architectures", article 9578008, section 2 item 4), written with the state
 * oriented d_k x d_v: decay acts on key channels, the write is k v^T, the read is
 * S^T q, and token t's output reads the state after its own write.  There is no
 * 1/sqrt(Dk) scaling of q; callers pre-scale q if they want one.
 *
 * Prefill evaluates the same result with the chunkwise algorithm of section 4 of
 * article 9569726 (section 3 of article 9578008); decode applies the rule to one
 * token (the constant-size recurrent state of section 1 of article 9569726).
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller, contiguous,
 *    row-major (last index fastest) and 16-byte aligned.
 *  - Nothing allocates: scratch memory is a caller-provided workspace.
 *  - All work is enqueued on `stream` (NULL = the default stream), and only there:
 *    the library creates no stream or event of its own, and no call synchronises.
 *    Errors detectable from the arguments are returned before any HIP call; a
 *    failed launch returns KDA_ERR_HIP.  Faults inside kernels show up at the
 *    caller's next synchronisation.
 *  - Preconditions that live in device memory are documented, not checked:
 *    cu_seqlens starts at 0, never decreases and ends at T; inputs are finite;
 *    log_alpha <= 0; beta in [0, 1].  Within one chunk, the summed log-decay of
 *    any channel must stay above -160 (the decay factors of a chunk are formed
 *    around its midpoint in fp32).
 *  - Outputs are bitwise deterministic for identical inputs: no result is summed
 *    with atomics (the one atomic counter, in the order of packed batches of more
 *    than 4096 sequences, decides only which workgroup runs which sequence).
 *  - Library functions are thread-safe and keep no mutable global state except
 *    kda_chunk_fwd_noalloc's fixed scratch array (one per GPU) and its device
 *    address, looked up once per GPU under a lock; calls that share a workspace
 *    (or, for kda_chunk_fwd_noalloc, a GPU) must be ordered (one stream, or events).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as hipStream_t. */
typedef struct ihipStream_t* kda_stream_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,     /* null pointer, bad size, misalignment, aliasing */
    KDA_ERR_UNSUPPORTED = 2,          /* head size, chunk size or dtype not built */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < kda_chunk_fwd_workspace_bytes() */
    KDA_ERR_HIP = 4,                  /* a HIP launch or API call failed */
    KDA_ERR_SCRATCH_LIMIT = 5         /* kda_chunk_fwd_noalloc: these sizes need more scratch
                                         than the library's fixed array holds */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Human-readable name of a status code (static storage). */
const char* kda_status_string(kda_status s);

/*
 * Workspace bytes kda_chunk_fwd needs for these sizes (same arguments, same
 * meaning).  has_cu_seqlens is 0 or 1.  Returns 0 for unsupported sizes, and at
 * least 256 otherwise.
 *
 * Layout.  The first 4 bytes of every prefill workspace are the call's status
 * word, an int32 on the device: the call's first kernel sets it to 0, and a
 * workgroup whose bounded ordering wait inside the kernels gave up (a wait that
 * polls an on-chip counter up to a fixed limit instead of forever) sets it to 1
 * and writes NaN to every output row and state it stores from then on.  Read it
 * after the call's work has completed: 0 means every wait completed.  The rest of
 * the workspace is private scratch (segment summaries, the packed-sequence order).
 * Packed batches with 32-token chunks and fewer than 256 (sequence, head) pairs
 * reserve segment summaries for 256 / H segments per head: the call cuts its
 * sequences into segments on the device, from cu_seqlens, so that one long
 * sequence still spreads over the chip.  For chunk 64 the size also covers the
 * 32-token evaluation that the scalar-gate and fused entry points use for such a
 * request, so one query serves every entry point that takes these arguments.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                     int has_cu_seqlens, int chunk);

/*
 * kda_chunk_fwd -- prefill: o and the final state of every sequence.
 *
 *   q, k, log_alpha : [B, T, H, Dk]   in_dtype
 *   v               : [B, T, H, Dv]   in_dtype
 *   beta            : [B, T, H]       in_dtype
 *   S0              : [N, H, Dk, Dv]  fp32 initial states, or NULL for zeros
 *   cu_seqlens      : int32 [N+1] device offsets of N packed sequences (B must be
 *                     1, sequence n owns tokens [cu[n], cu[n+1]), zero lengths
 *                     allowed), or NULL: then N = B sequences of T tokens each
 *   num_seqs        : N
 *   chunk           : chunk length in tokens: 32 or 64, or 0 for the default (32)
 *   o               : [B, T, H, Dv]   out_dtype (bf16 is round-to-nearest-even)
 *   S_final         : [N, H, Dk, Dv]  fp32, or NULL to skip
 *   workspace       : device scratch of workspace_bytes >= the query above, not
 *                     overlapping any other argument; its first word receives the
 *                     call's status (see the query)
 *
 * Supported: Dk == Dv in {64, 128}; in_dtype, out_dtype in {KDA_F32, KDA_BF16}.
 * A sequence of length 0 gets S_final = S0 (or zeros).  T == 0 or N == 0 only
 * writes S_final.  Inputs must not overlap outputs.  The result does not depend
 * on the chunk size beyond rounding.  Equal-length batches (cu_seqlens NULL) with
 * T <= 4 are evaluated token by token, as kda_recurrent_fwd does.
 * Streams: every kernel runs on `stream`, ordered after what is already enqueued
 * on it and before what is enqueued on it after the call.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                         kda_dtype in_dtype, kda_dtype out_dtype,
                         void* o, float* S_final,
                         void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and harnesses
 * that forbid hipMalloc.  The arguments are kda_chunk_fwd's without the workspace;
 * the call's scratch (status word, packed-sequence order, segment summaries) comes
 * from a fixed array of KDA_NOALLOC_SCRATCH_BYTES in the library's own device memory,
 * one per GPU, held until the process ends.  The call allocates nothing.
 *
 * Returns KDA_ERR_SCRATCH_LIMIT, before any HIP call, when
 * kda_chunk_fwd_workspace_bytes() for these sizes exceeds KDA_NOALLOC_SCRATCH_BYTES
 * (no equal-length plan and no packed plan of fewer than 256 (sequence, head)
 * pairs at Dk = Dv <= 128 does: their segment summaries stay under 48 MiB; packed
 * batches of more than about 16 million sequences do).  Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents (each call
 * clears what must start at zero itself): calls that overlap in time on one GPU --
 * on different streams, or from host threads whose streams are not ordered -- race
 * and give wrong results.  Calls ordered on one stream are safe.  The status word of
 * kda_chunk_fwd is kept in the array and is not readable here; a broken ordering
 * still shows as NaN outputs.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                                 const void* beta, const float* S0, const int32_t* cu_seqlens,
                                 int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                 kda_dtype in_dtype, kda_dtype out_dtype,
                                 void* o, float* S_final, kda_stream_t stream);

/*
 * kda_recurrent_step -- decode: one token for each of N independent sequences.
 *
 *   q, k, log_alpha : [N, H, Dk]  in_dtype      v : [N, H, Dv] in_dtype
 *   beta            : [N, H]      in_dtype
 *   S_in            : [N, H, Dk, Dv] fp32 state before the token
 *   S_out           : [N, H, Dk, Dv] fp32 state after the token; S_out == S_in
 *                     (in place) is allowed, any other overlap is rejected
 *   o               : [N, H, Dv]  out_dtype
 *
 * Supported: Dk == Dv in {64, 128}.  N == 0 is a no-op.
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, const float* S_in, float* S_out,
                              int N, int H, int Dk, int Dv,
                              kda_dtype in_dtype, kda_dtype out_dtype,
                              void* o, kda_stream_t stream);

/*
 * kda_recurrent_fwd -- the same result as kda_chunk_fwd, computed token by token per
 * sequence with the state held on chip: every (sequence, head) state is read once
 * and written once.  It is the multi-token continuation of decode (the constant-size
 * recurrent state of section 1 of article 9569726): a few new tokens per sequence on
 * top of a carried state, as in speculative verification or chunked continuation,
 * where the chunkwise form would be mostly padding.  Its cost grows with the longest
 * sequence, so long prompts belong to kda_chunk_fwd.
 *
 * Arguments and layouts are those of kda_chunk_fwd (there is no chunk and no
 * workspace).  S_final == S0 (in place) is allowed; any other overlap is rejected.
 * A single token's decay is taken no smaller than 2^-60 (log_alpha >= -41.59).
 */
kda_status kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S0, const int32_t* cu_seqlens,
                             int B, int T, int H, int Dk, int Dv, int num_seqs,
                             kda_dtype in_dtype, kda_dtype out_dtype,
                             void* o, float* S_final, kda_stream_t stream);

/*
 * Fused prologue and epilogue: the elementwise steps on either side of the layer
 * run inside its kernels instead of as separate passes over HBM.
 *
 *   KDA_FUSE_QK_L2NORM        q and k are L2-normalised per (token, head) over Dk:
 *                             x / sqrt(sum x^2 + 1e-12) (the pages take the keys as
 *                             normalised, "Decoding Hybrid Attention Architectures"
 *                             section 3.2)
 *   KDA_FUSE_BETA_SIGMOID     beta holds logits: beta = 1 / (1 + exp(-beta))
 *   KDA_FUSE_DECAY_LOGSIGMOID log_alpha holds logits a: log_alpha = logsigmoid(a +
 *                             decay_bias) / decay_scale (decay_scale > 0), so every
 *                             decay lies in (0, 1)
 *   out_gate                  NULL, or gate logits shaped like o in the input dtype:
 *                             o <- o * sigmoid(gate), per value channel
 *
 * The _fused functions take the arguments of their plain counterparts plus a
 * kda_fusion (NULL or all-zero = the plain function); kda_chunk_fwd_fused takes chunk 0,
 * 32 or 64 (64 is evaluated with 32-token chunks, which change the result only by rounding)
 * and uses kda_chunk_fwd_workspace_bytes() with the same chunk argument.
 */
typedef enum {
    KDA_FUSE_QK_L2NORM = 1,
    KDA_FUSE_BETA_SIGMOID = 2,
    KDA_FUSE_DECAY_LOGSIGMOID = 4
} kda_fuse_flag;

typedef struct {
    int flags;               /* bitwise OR of kda_fuse_flag */
    float decay_bias;        /* used with KDA_FUSE_DECAY_LOGSIGMOID */
    float decay_scale;       /* used with KDA_FUSE_DECAY_LOGSIGMOID, > 0 */
    const void* out_gate;    /* device pointer or NULL, 16-byte aligned */
} kda_fusion;

kda_status kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S0, const int32_t* cu_seqlens,
                               int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                               kda_dtype in_dtype, kda_dtype out_dtype,
                               void* o, float* S_final,
                               void* workspace, size_t workspace_bytes,
                               const kda_fusion* fusion, kda_stream_t stream);

kda_status kda_recurrent_step_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S_in, float* S_out,
                                    int N, int H, int Dk, int Dv,
                                    kda_dtype in_dtype, kda_dtype out_dtype,
                                    void* o, const kda_fusion* fusion, kda_stream_t stream);

/*
 * Scalar-gated variant (Gated DeltaNet): the same rule with one decay per token and
 * head, S_t = (I - beta_t k_t k_t^T) alpha_t S_{t-1} + beta_t k_t v_t^T, alpha_t a
 * scalar in (0, 1] ("Decoding Hybrid Attention Architectures", section 3.3 and the
 * variant table of section 3; "Technical Analysis ...", section 2).  It is KDA with
 * every key channel given the same decay, so each function below returns what its
 * kda_ counterpart returns for log_alpha broadcast over the key channels.
 *
 *   log_alpha : [B, T, H] (gdn_chunk_fwd, gdn_recurrent_fwd) or [N, H]
 *               (gdn_recurrent_step), in_dtype; every other argument as in the
 *               kda_ function of the same suffix.
 *
 * gdn_chunk_fwd takes chunk 0, 32 or 64 (64 is evaluated with 32-token chunks) and uses
 * kda_chunk_fwd_workspace_bytes() with the same chunk argument.
 * With a scalar decay the chunk's decay factors leave the contractions, so with
 * bf16 inputs the keys and queries are exact MFMA operands and the prefill does
 * about a third less matrix work and almost no per-element decay work.
 */
kda_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                         kda_dtype in_dtype, kda_dtype out_dtype,
                         void* o, float* S_final,
                         void* workspace, size_t workspace_bytes, kda_stream_t stream);

kda_status gdn_recurrent_step(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, const float* S_in, float* S_out,
                              int N, int H, int Dk, int Dv,
                              kda_dtype in_dtype, kda_dtype out_dtype,
                              void* o, kda_stream_t stream);

/*
 * Scalar gate with the fused prologue / epilogue: gdn_chunk_fwd and gdn_recurrent_step
 * plus a kda_fusion, with the maps of kda_chunk_fwd_fused applied to the scalar-gate
 * inputs (KDA_FUSE_DECAY_LOGSIGMOID maps the one log_alpha logit per token and head).
 * gdn_chunk_fwd_fused takes chunk 0, 32 or 64 (64 is evaluated with 32-token chunks) and
 * uses kda_chunk_fwd_workspace_bytes() with the same chunk argument.
 */
kda_status gdn_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S0, const int32_t* cu_seqlens,
                               int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                               kda_dtype in_dtype, kda_dtype out_dtype,
                               void* o, float* S_final,
                               void* workspace, size_t workspace_bytes,
                               const kda_fusion* fusion, kda_stream_t stream);

kda_status gdn_recurrent_step_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S_in, float* S_out,
                                    int N, int H, int Dk, int Dv,
                                    kda_dtype in_dtype, kda_dtype out_dtype,
                                    void* o, const kda_fusion* fusion, kda_stream_t stream);

kda_status gdn_recurrent_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S0, const int32_t* cu_seqlens,
                             int B, int T, int H, int Dk, int Dv, int num_seqs,
                             kda_dtype in_dtype, kda_dtype out_dtype,
                             void* o, float* S_final, kda_stream_t stream);

/*
 * kda_recurrent_fwd and gdn_recurrent_fwd with the fused prologue / epilogue (the maps of
 * kda_chunk_fwd_fused, per token).  kda_chunk_fwd_fused and gdn_chunk_fwd_fused take this
 * path for equal-length batches of at most 4 tokens per sequence.
 */
kda_status kda_recurrent_fwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                   const void* beta, const float* S0, const int32_t* cu_seqlens,
                                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                                   kda_dtype in_dtype, kda_dtype out_dtype,
                                   void* o, float* S_final, const kda_fusion* fusion, kda_stream_t stream);

kda_status gdn_recurrent_fwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                   const void* beta, const float* S0, const int32_t* cu_seqlens,
                                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                                   kda_dtype in_dtype, kda_dtype out_dtype,
                                   void* o, float* S_final, const kda_fusion* fusion, kda_stream_t stream);

/*
 * kda_chunk_bwd -- gradient of kda_chunk_fwd for training.
 *
 * The pages motivate the chunkwise form by training throughput ("Decoding Hybrid
 * Attention Architectures", section 4) and give no backward; this is the exact
 * gradient of the layer that kda_chunk_fwd computes (the recurrence of section 3.4),
 * evaluated through the same chunkwise form: a forward pass over the chunks that
 * keeps every chunk's entry state, a reverse pass that carries the state gradient
 * from the last chunk to the first, and one parallel step per (chunk, head).
 * Memory control (section 4's concern that training memory not grow with sequence
 * length): when that per-chunk data would exceed 2 GiB (the KDA_BWD_WORKSPACE_LIMIT
 * environment variable, in bytes, overrides the limit), equal-length batches run in
 * windows of chunks, last window first, with one checkpointed entry state per window
 * and the state gradient carried between windows.  fp32 inputs: the checkpoints come
 * from a sweep of the backward's forward state pass and the gradients are bitwise
 * those of the one-pass plan.  bf16 inputs: the checkpoints come from the prefill's
 * segment summaries chained by its combine (windows = segments), so they differ from
 * the one-pass plan in fp32 rounding order only.  Packed batches always take the
 * one-pass plan.
 *
 *   q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, in_dtype:
 *                     the arguments of the kda_chunk_fwd call being differentiated
 *   d_o             : [B, T, H, Dv] in_dtype, gradient of the loss with respect to o
 *   dS_final        : [N, H, Dk, Dv] fp32 gradient with respect to S_final, or NULL
 *                     for zero
 *   chunk           : 0, 32 or 64 (the chunk length of the forward call); the gradient
 *                     is evaluated with 32-token chunks in every case, since the
 *                     layer, and so its gradient, does not depend on the chunk length
 *                     beyond rounding
 *   dq, dk          : [B, T, H, Dk]   grad_dtype
 *   dv              : [B, T, H, Dv]   grad_dtype
 *   dlog_alpha      : [B, T, H, Dk]   grad_dtype
 *   dbeta           : [B, T, H]       grad_dtype
 *   dS0             : [N, H, Dk, Dv]  fp32 gradient with respect to S0, or NULL to skip
 *                     (written for every sequence, also when S0 is NULL)
 *   workspace       : device scratch of kda_chunk_bwd_workspace_bytes() bytes; per
 *                     chunk and head (of all chunks, or of one window) it holds the
 *                     chunk's record, entry state and state gradient in fp32, about
 *                     (2 Dk Dv + 3 C Dk + 3 C^2) * 4 bytes with C = 32
 *
 * Supported: Dk == Dv in {64, 128}; in_dtype, grad_dtype in {KDA_F32, KDA_BF16}
 * (bf16 gradients are the round-to-nearest-even bf16 of the fp32 result).  All
 * arithmetic is fp32.  Outputs must not overlap inputs, each other or the workspace.
 * With N == 0 nothing is written; with T == 0, dS0 = dS_final (or zeros).  Decays
 * follow kda_chunk_fwd's domain: the decay of half a chunk stays within fp32 range.
 */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                     int has_cu_seqlens, int chunk);

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         const void* d_o, const float* dS_final,
                         int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                         kda_dtype in_dtype, kda_dtype grad_dtype,
                         void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                         void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * gdn_chunk_bwd -- gradient of gdn_chunk_fwd (scalar gate): the same arguments as
 * kda_chunk_bwd except log_alpha [B, T, H] and dlog_alpha [B, T, H].  The scalar gate is
 * the per-channel rule with one log-decay broadcast over the key channels, so its
 * gradient is the per-channel dlog_alpha summed over the key channels.  Uses
 * kda_chunk_bwd_workspace_bytes().
 */
kda_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         const void* d_o, const float* dS_final,
                         int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                         kda_dtype in_dtype, kda_dtype grad_dtype,
                         void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                         void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_chunk_bwd_fused -- gradient of kda_chunk_fwd_fused: the fused layer's output
 * o = rule(maps(q, k, beta, log_alpha), v, S0) * sigmoid(gate) (the gate when
 * fusion->out_gate is set) and its final states, differentiated with respect to the raw
 * inputs.  The maps are those of kda_fusion (L2 norm of q and k, sigmoid of beta logits,
 * logsigmoid(a + decay_bias) / decay_scale of decay logits); the rule is the gated delta
 * rule of "Decoding Hybrid Attention Architectures" section 3.4.  The chain rule runs
 * through each map ("Decoding Hybrid Attention Architectures" section 3.2 takes the keys as
 * normalised; the maps themselves are this library's reading):
 *   x' = x / sqrt(sum x^2 + 1e-12):  dx = (dx' - x' (x' . dx')) / sqrt(sum x^2 + 1e-12)
 *   beta = sigmoid(b):               db = dbeta beta (1 - beta)
 *   log_alpha = logsigmoid(a + c)/s: da = dlog_alpha (1 - sigmoid(a + c)) / s
 *   o * sigmoid(g):                  d(o) = d_o sigmoid(g), dg = d_o o sigmoid(g)(1 - sigmoid(g))
 * Arguments as for kda_chunk_bwd, with d_o the gradient of the gated output, plus
 *   dgate      : [B, T, H, Dv] grad_dtype, the gradient of the gate logits (required when
 *                fusion->out_gate is set, else ignored)
 *   fusion     : the same kda_fusion as the forward call (NULL = the plain gradient)
 *   workspace  : kda_chunk_bwd_fused_workspace_bytes() bytes (has_out_gate 0 or 1): the
 *                rule's gradient workspace, then fp32 copies of the mapped inputs, of the
 *                rule's gradients and, with a gate, of the ungated output.
 * The rule's gradient runs on the mapped inputs in fp32: with fp32 matrix-core products for
 * fp32 raw inputs, and with split-bf16 products (hi + lo, fp32 accumulation) for bf16 raw
 * inputs, whose tolerance is the bf16 one; with a gate, one forward pass first recomputes the
 * ungated output.  dlog_alpha and dbeta hold the
 * gradients of the decay and beta logits under those flags.  Errors as for kda_chunk_bwd.
 */
size_t kda_chunk_bwd_fused_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                           int has_cu_seqlens, int chunk, int has_out_gate);

kda_status kda_chunk_bwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S0, const int32_t* cu_seqlens,
                               const void* d_o, const float* dS_final,
                               int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                               kda_dtype in_dtype, kda_dtype grad_dtype,
                               void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                               void* dgate, void* workspace, size_t workspace_bytes,
                               const kda_fusion* fusion, kda_stream_t stream);

/*
 * gdn_chunk_bwd_fused -- the same for the scalar gate (gdn_chunk_fwd_fused): log_alpha and
 * dlog_alpha [B, T, H], the decay map applied to the one logit per token and head.
 */
size_t gdn_chunk_bwd_fused_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                           int has_cu_seqlens, int chunk, int has_out_gate);

kda_status gdn_chunk_bwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S0, const int32_t* cu_seqlens,
                               const void* d_o, const float* dS_final,
                               int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                               kda_dtype in_dtype, kda_dtype grad_dtype,
                               void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                               void* dgate, void* workspace, size_t workspace_bytes,
                               const kda_fusion* fusion, kda_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
