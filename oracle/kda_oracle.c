/*
 * kda_oracle.c -- plain fp64 CPU oracle for the KDA gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h).  Slow on purpose: one token at a
 * time, one loop per term of the update, no blocking and no reordering beyond
 * what the recurrence states.
 *
 * Source of the recurrence: "Decoding Hybrid Attention Architectures"
 * (intl.cloud.baidu.com article 9569726), section 3.4, the fine-grained gated
 * delta rule S_t = (I - beta k k^T) Diag(a_t) S_{t-1} + beta (write), and section
 * 3.2 for the delta form of the update: the write along key k is scaled by the
 * error v - S^T k between the new value and what the state returns for k.  The
 * same rule appears as item 4
 * of section 2 of "Technical Analysis and Engineering Practices for Novel Hybrid
 * Linear Attention Architectures" (article 9578008).
 *
 * Readings taken where the pages are loose:
 *  - orientation: S is d_k x d_v, the decay acts on the key channels (rows),
 *    the write is k v^T and the read is S^T q;
 *  - decay happens before the erase/write, as the product order on the pages
 *    (I - beta k k^T) Diag(a_t) S_{t-1} says;
 *  - the output of token t reads the state after token t's own write;
 *  - no 1/sqrt(d_k) scaling of q.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_elem(const void* p, int dtype, size_t i) {
    if (dtype == ORACLE_F64) return ((const double*)p)[i];
    if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
    /* bf16: the upper half of an IEEE binary32 */
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void store_elem(void* p, int dtype, size_t i, double x) {
    if (dtype == ORACLE_F64) ((double*)p)[i] = x;
    else ((float*)p)[i] = (float)x;
}

static int dtype_ok(int d) { return d == ORACLE_F64 || d == ORACLE_F32 || d == ORACLE_BF16; }

/* S' = Diag(alpha_t) S_{t-1}: key channel c (row c) decays by exp(log_alpha[c]). */
static void decay_rows(double* S, int Dk, int Dv, const void* log_alpha, int in_dtype, size_t gi) {
    for (int c = 0; c < Dk; ++c) {
        double a = exp(load_elem(log_alpha, in_dtype, gi + c));
        for (int j = 0; j < Dv; ++j) S[(size_t)c * Dv + j] *= a;
    }
}

/* S_t = S' + beta k (v - S'^T k)^T: r = S'^T k is what the memory returns for key k;
 * the write moves that readout toward v by beta (erase along k, then write v). */
static void delta_write(double* S, int Dk, int Dv, const void* k, const void* v,
                        const void* beta, int in_dtype, size_t ki, size_t vi, size_t bi,
                        double* r, double* e) {
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, ki + c);
        for (int j = 0; j < Dv; ++j) r[j] += kc * S[(size_t)c * Dv + j];
    }
    double b = load_elem(beta, in_dtype, bi);
    for (int j = 0; j < Dv; ++j) e[j] = b * (load_elem(v, in_dtype, vi + j) - r[j]);
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, ki + c);
        for (int j = 0; j < Dv; ++j) S[(size_t)c * Dv + j] += kc * e[j];
    }
}

/* o_t = S_t^T q, written at o[oi .. oi+Dv). */
static void read_out(const double* S, int Dk, int Dv, const void* q, int in_dtype, size_t qi,
                     void* o, int o_dtype, size_t oi, double* r) {
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        double qc = load_elem(q, in_dtype, qi + c);
        for (int j = 0; j < Dv; ++j) r[j] += qc * S[(size_t)c * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) store_elem(o, o_dtype, oi + j, r[j]);
}

/*
 * One token on one (sequence, head) state S (Dk x Dv, fp64): decay, then the
 * delta write, then the read-out of the updated state.  xi indexes the token's
 * Dk-vectors (q, k, log_alpha), vi its Dv-vectors (v, o), bi its beta.
 */
static void kda_token(double* S, int Dk, int Dv,
                      const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* beta, int in_dtype, size_t xi, size_t vi, size_t bi,
                      void* o, int o_dtype, double* r, double* e) {
    decay_rows(S, Dk, Dv, log_alpha, in_dtype, xi);
    delta_write(S, Dk, Dv, k, v, beta, in_dtype, xi, vi, bi, r, e);
    read_out(S, Dk, Dv, q, in_dtype, xi, o, o_dtype, vi, r);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_kda_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, int in_dtype,
                   const void* S0, int s0_dtype,
                   const int64_t* cu_seqlens,
                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                   void* o, int o_dtype, double* S_final, int num_threads) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || num_seqs < 0) return -1;
    if (!dtype_ok(in_dtype) || (S0 && !dtype_ok(s0_dtype))) return -1;
    if (o_dtype != ORACLE_F64 && o_dtype != ORACLE_F32) return -1;
    if (cu_seqlens) {
        if (B != 1 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (num_seqs != B) {
        return -1;
    }
    if ((size_t)B * T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return -1;

    long units = (long)num_seqs * H;
#ifdef _OPENMP
    int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (long u = 0; u < units; ++u) {
        int n = (int)(u / H), h = (int)(u % H);
        /* global token range of sequence n (tokens are rows of the [B*T] axis) */
        int64_t t0 = cu_seqlens ? cu_seqlens[n] : (int64_t)n * T;
        int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : (int64_t)(n + 1) * T;
        double* S = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
        double* r = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)Dv);
        size_t sbase = ((size_t)n * H + h) * (size_t)Dk * Dv;
        for (size_t i = 0; i < (size_t)Dk * Dv; ++i)
            S[i] = S0 ? load_elem(S0, s0_dtype, sbase + i) : 0.0;
        for (int64_t t = t0; t < t1; ++t) {
            size_t row = (size_t)t * H + h;
            kda_token(S, Dk, Dv, q, k, v, log_alpha, beta, in_dtype,
                      row * Dk, row * Dv, row, o, o_dtype, r, e);
        }
        if (S_final) memcpy(S_final + sbase, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(r);
        free(e);
    }
    return 0;
}

int oracle_kda_step(const void* q, const void* k, const void* v, const void* log_alpha,
                    const void* beta, int in_dtype,
                    double* S, int N, int H, int Dk, int Dv,
                    void* o, int o_dtype, int num_threads) {
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    if (!dtype_ok(in_dtype) || (o_dtype != ORACLE_F64 && o_dtype != ORACLE_F32)) return -1;
    if (N > 0 && (!q || !k || !v || !log_alpha || !beta || !S || !o)) return -1;
    long units = (long)N * H;
#ifdef _OPENMP
    int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
#endif
    for (long u = 0; u < units; ++u) {
        double* r = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)Dv);
        kda_token(S + (size_t)u * Dk * Dv, Dk, Dv, q, k, v, log_alpha, beta, in_dtype,
                  (size_t)u * Dk, (size_t)u * Dv, (size_t)u, o, o_dtype, r, e);
        free(r);
        free(e);
    }
    return 0;
}

/*
 * Gradient of the token recurrence above (reverse mode, one token at a time from
 * the last to the first).  The forward state before every token is kept (the
 * recurrence is re-run first), then for token t, with dS the gradient with
 * respect to S_t:
 *
 *   S' = Diag(alpha) S_{t-1};  r = S'^T k;  e = beta (v - r);  S_t = S' + k e^T
 *   dS  += q do^T                       dq = S_t do
 *   dk   = dS e + S' dr                 de = dS^T k,   dr = -beta de
 *   dv   = beta de                      dbeta = de . (v - r)
 *   dS'  = dS + k dr^T                  dlog_alpha_c = sum_j dS'_cj S'_cj
 *   dS_{t-1} = Diag(alpha) dS'
 *
 * which is the chain rule applied to each line of kda_token in reverse order.
 */
static void kda_token_bwd(double* dS, const double* Sprev, double* Sp, double* r, double* e,
                          double* de, double* dr, int Dk, int Dv,
                          const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* beta, int in_dtype, const void* d_o, int do_dtype,
                          size_t xi, size_t vi, size_t bi,
                          double* dq, double* dk, double* dv, double* dla, double* dbeta) {
    /* recompute S' = Diag(alpha) S_{t-1}, r = S'^T k, e = beta (v - r) */
    for (int c = 0; c < Dk; ++c) {
        double a = exp(load_elem(log_alpha, in_dtype, xi + c));
        for (int j = 0; j < Dv; ++j) Sp[(size_t)c * Dv + j] = a * Sprev[(size_t)c * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, xi + c);
        for (int j = 0; j < Dv; ++j) r[j] += kc * Sp[(size_t)c * Dv + j];
    }
    double bt = load_elem(beta, in_dtype, bi);
    for (int j = 0; j < Dv; ++j) e[j] = bt * (load_elem(v, in_dtype, vi + j) - r[j]);

    /* o_t = S_t^T q with S_t = S' + k e^T */
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, xi + c);
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j)
            acc += (Sp[(size_t)c * Dv + j] + kc * e[j]) * load_elem(d_o, do_dtype, vi + j);
        dq[xi + c] = acc;
    }
    for (int c = 0; c < Dk; ++c) {
        double qc = load_elem(q, in_dtype, xi + c);
        for (int j = 0; j < Dv; ++j) dS[(size_t)c * Dv + j] += qc * load_elem(d_o, do_dtype, vi + j);
    }

    /* S_t = S' + k e^T */
    for (int j = 0; j < Dv; ++j) de[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, xi + c);
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
            acc += dS[(size_t)c * Dv + j] * e[j];
            de[j] += kc * dS[(size_t)c * Dv + j];
        }
        dk[xi + c] = acc;
    }

    /* e = beta (v - r) */
    double db = 0.0;
    for (int j = 0; j < Dv; ++j) {
        db += de[j] * (load_elem(v, in_dtype, vi + j) - r[j]);
        dv[vi + j] = bt * de[j];
        dr[j] = -bt * de[j];
    }
    dbeta[bi] = db;

    /* r = S'^T k: dS' = dS + k dr^T, dk += S' dr */
    for (int c = 0; c < Dk; ++c) {
        double kc = load_elem(k, in_dtype, xi + c);
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
            acc += Sp[(size_t)c * Dv + j] * dr[j];
            dS[(size_t)c * Dv + j] += kc * dr[j];
        }
        dk[xi + c] += acc;
    }

    /* S' = Diag(alpha) S_{t-1}: d log_alpha_c = alpha_c sum_j dS'_cj S_{t-1,cj} */
    for (int c = 0; c < Dk; ++c) {
        double a = exp(load_elem(log_alpha, in_dtype, xi + c));
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
            acc += dS[(size_t)c * Dv + j] * Sp[(size_t)c * Dv + j];
            dS[(size_t)c * Dv + j] *= a;
        }
        dla[xi + c] = acc;
    }
}

int oracle_kda_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, int in_dtype,
                   const void* S0, int s0_dtype,
                   const int64_t* cu_seqlens,
                   int B, int T, int H, int Dk, int Dv, int num_seqs,
                   const void* d_o, int do_dtype, const void* dS_final, int dsf_dtype,
                   double* dq, double* dk, double* dv, double* dlog_alpha, double* dbeta,
                   double* dS0, int num_threads) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || num_seqs < 0) return -1;
    if (!dtype_ok(in_dtype) || (S0 && !dtype_ok(s0_dtype))) return -1;
    if (!dtype_ok(do_dtype) || (dS_final && !dtype_ok(dsf_dtype))) return -1;
    if (cu_seqlens) {
        if (B != 1 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (num_seqs != B) {
        return -1;
    }
    if ((size_t)B * T > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk ||
                              !dv || !dlog_alpha || !dbeta))
        return -1;

    const size_t DD = (size_t)Dk * Dv;
    long units = (long)num_seqs * H;
#ifdef _OPENMP
    int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (long u = 0; u < units; ++u) {
        int n = (int)(u / H), h = (int)(u % H);
        int64_t t0 = cu_seqlens ? cu_seqlens[n] : (int64_t)n * T;
        int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : (int64_t)(n + 1) * T;
        size_t L = (size_t)(t1 - t0);
        size_t sbase = ((size_t)n * H + h) * DD;
        /* states[i] = the state before token t0 + i, i = 0..L-1 */
        double* states = (double*)malloc(sizeof(double) * DD * (L > 0 ? L : 1));
        double* S = (double*)malloc(sizeof(double) * DD);
        double* Sp = (double*)malloc(sizeof(double) * DD);
        double* dS = (double*)malloc(sizeof(double) * DD);
        double* r = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* de = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* dr = (double*)malloc(sizeof(double) * (size_t)Dv);
        for (size_t i = 0; i < DD; ++i) S[i] = S0 ? load_elem(S0, s0_dtype, sbase + i) : 0.0;
        for (int64_t t = t0; t < t1; ++t) {
            size_t row = (size_t)t * H + h;
            memcpy(states + (size_t)(t - t0) * DD, S, sizeof(double) * DD);
            decay_rows(S, Dk, Dv, log_alpha, in_dtype, row * Dk);
            delta_write(S, Dk, Dv, k, v, beta, in_dtype, row * Dk, row * Dv, row, r, e);
        }
        for (size_t i = 0; i < DD; ++i)
            dS[i] = dS_final ? load_elem(dS_final, dsf_dtype, sbase + i) : 0.0;
        for (int64_t t = t1 - 1; t >= t0; --t) {
            size_t row = (size_t)t * H + h;
            kda_token_bwd(dS, states + (size_t)(t - t0) * DD, Sp, r, e, de, dr, Dk, Dv,
                          q, k, v, log_alpha, beta, in_dtype, d_o, do_dtype,
                          row * Dk, row * Dv, row, dq, dk, dv, dlog_alpha, dbeta);
        }
        if (dS0) memcpy(dS0 + sbase, dS, sizeof(double) * DD);
        free(states);
        free(S);
        free(Sp);
        free(dS);
        free(r);
        free(e);
        free(de);
        free(dr);
    }
    return 0;
}
