/*
 * kda_oracle.h -- plain fp64 CPU oracle for the KDA gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP kernels.
 *
 * What it computes (per sequence and head, tokens in order), following
 * "Decoding Hybrid Attention Architectures" (intl.cloud.baidu.com article 9569726)
 * section 3.4 (fine-grained gated delta rule) and section 3.2 (the delta,
 * "difference", form of the update), written in one consistent orientation with
 * the state S of shape d_k x d_v:
 *
 *     S' = Diag(alpha_t) S_{t-1},          alpha_t = exp(log_alpha_t)   (per key channel)
 *     S_t = S' + beta_t k_t (v_t - S'^T k_t)^T                          (erase-then-write)
 *     o_t = S_t^T q_t                                                   (post-update state)
 *
 * which equals S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 *
 * Layouts (row-major, last index fastest):
 *   q, k, log_alpha : [B, T, H, Dk]      v, o : [B, T, H, Dv]      beta : [B, T, H]
 *   S0, S_final, S  : [N, H, Dk, Dv]
 * With cu_seqlens (int64, N+1 entries, host memory) B must be 1 and sequence n
 * owns tokens [cu_seqlens[n], cu_seqlens[n+1]); without it N = B and every
 * sequence has T tokens.
 *
 * Inputs are read exactly (bf16 and fp32 widen to fp64 without rounding); all
 * arithmetic is fp64.  Return value 0 on success, -1 on a bad argument.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Chunk-free token recurrence over whole sequences.
 * S0 may be NULL (zero initial state); its element type is s0_dtype.
 * o is written with element type o_dtype (ORACLE_F64 or ORACLE_F32).
 * S_final (fp64) may be NULL.
 * num_threads <= 0 uses the OpenMP default; parallelism is over (sequence, head). */
int oracle_kda_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, int in_dtype,
                   const void* S0, int s0_dtype,
                   const int64_t* cu_seqlens,
                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                   void* o, int o_dtype, double* S_final, int num_threads);

/* One decode token for N independent sequences: q, k, log_alpha [N, H, Dk],
 * v [N, H, Dv], beta [N, H]; S [N, H, Dk, Dv] fp64 is updated in place;
 * o [N, H, Dv] is written with element type o_dtype. */
int oracle_kda_step(const void* q, const void* k, const void* v, const void* log_alpha,
                    const void* beta, int in_dtype,
                    double* S, int N, int H, int Dk, int Dv,
                    void* o, int o_dtype, int num_threads);

/* Gradient of oracle_kda_fwd (exact reverse mode of the token recurrence, fp64).
 * d_o [B, T, H, Dv] (element type do_dtype) is the gradient of the loss with
 * respect to o; dS_final [N, H, Dk, Dv] (element type dsf_dtype) the gradient with
 * respect to S_final, or NULL for zero.  Outputs, all fp64 and fully written for
 * every token of every sequence: dq, dk, dlog_alpha [B, T, H, Dk], dv [B, T, H, Dv],
 * dbeta [B, T, H], and dS0 [N, H, Dk, Dv] (may be NULL).  Other arguments as in
 * oracle_kda_fwd.  Keeps every state of a (sequence, head) in memory. */
int oracle_kda_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, int in_dtype,
                   const void* S0, int s0_dtype,
                   const int64_t* cu_seqlens,
                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                   const void* d_o, int do_dtype, const void* dS_final, int dsf_dtype,
                   double* dq, double* dk, double* dv, double* dlog_alpha, double* dbeta,
                   double* dS0, int num_threads);

/* Threads the OpenMP runtime would use for num_threads <= 0. */
int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_ORACLE_H */
