// kda_decode.hip -- token-by-token KDA kernels for gfx950: the single-token decode step and
// the multi-token recurrent forward (a few new tokens per sequence on top of a carried state).
//
// One token of the fine-grained gated delta rule ("Decoding Hybrid Attention
// Architectures", intl.cloud.baidu.com article 9569726, section 3.4) for N x H
// independent (sequence, head) states.  The recurrent state is what makes decode
// cost independent of context length (same page, section 1), so the step is one
// streaming pass over the fp32 state: HBM-bound, ~0.9 flop per byte.
//
// Per (n, h), with S' = Diag(alpha) S:
//     r = S'^T k,  p = S'^T q,  e = beta (v - r)
//     S_out = S' + k e^T
//     o = S_out^T q = p + (k . q) e
// so the state is read once and written once, with both reductions over Dk taken
// from the same registers.
//
// Mapping: one 256-thread workgroup per (n, h).  Thread t owns 4 consecutive
// columns (cg = t % (D/4)) of ROWS consecutive rows (rg = t / (D/4)); a wave reads
// whole 512-byte state rows with 16-byte loads, so every load and store is fully
// coalesced.  Column partial sums over a thread's rows are combined across the
// row groups through LDS.  The state is touched once per step, so its loads and
// stores are non-temporal (`nt`): on MI355X that lifts the step from about 5.1 to
// 5.9 TB/s of state traffic.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kDecodeThreads = 256;

typedef float vf4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float4* p) {
    const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store_stream(float4* p, float4 x) {
    __builtin_nontemporal_store(vf4{x.x, x.y, x.z, x.w}, reinterpret_cast<vf4*>(p));
}

// Fused prologue / epilogue of a decode step (FUSE kernels).
struct DecodeFusion {
    int flags;                // 1: L2-normalise q and k; 2: beta holds logits; 4: log_alpha holds logits
    float decay_bias, decay_scale;
    const void* out_gate;     // [N, H, D] output-gate logits or nullptr
};

__device__ __forceinline__ float sigmoid_d(float x) { return __builtin_amdgcn_rcpf(1.f + fast_exp(-x)); }

// SG: log_alpha is one value per (sequence, head) (the scalar gate of Gated DeltaNet).
// FUSE: q, k unnormalised, beta and log_alpha as logits, optional output gate.  With
// nk = 1/|k|, nq = 1/|q|: r = nk S'^T k, p = nq S'^T q, e = beta (v - r),
// S_out = S' + k (nk e)^T, o = p + (k . q) nk nq e.
template <int D, typename IN, bool OUT_BF16, bool SG = false, bool FUSE = false>
__global__ __launch_bounds__(kDecodeThreads)
void decode_step_kernel(const typename IN::storage* __restrict__ q,
                        const typename IN::storage* __restrict__ k,
                        const typename IN::storage* __restrict__ v,
                        const typename IN::storage* __restrict__ log_alpha,
                        const typename IN::storage* __restrict__ beta,
                        const float* S_in, float* S_out, void* __restrict__ o, DecodeFusion fu) {
    constexpr int CG = D / 4;                 // column groups of 4
    constexpr int RG = kDecodeThreads / CG;   // row groups
    constexpr int ROWS = D / RG;              // rows per thread
    static_assert(ROWS * RG == D && CG * RG == kDecodeThreads, "decode tiling");

    __shared__ float s_alpha[D], s_k[D], s_q[D];
    __shared__ float4 s_r[RG][CG];
    __shared__ float4 s_p[RG][CG];
    __shared__ float s_kq[kDecodeThreads / 64];
    __shared__ float s_kk[kDecodeThreads / 64], s_qq[kDecodeThreads / 64];

    const int unit = blockIdx.x;              // n * H + h
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const size_t vec = static_cast<size_t>(unit) * D;
    const size_t sbase = static_cast<size_t>(unit) * D * D;

    // Issue the state loads first: they are the whole cost of the step.
    float4 s[ROWS];
    const float4* src = reinterpret_cast<const float4*>(S_in + sbase);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) s[i] = load_stream(&src[(rg * ROWS + i) * CG + cg]);

    float kq = 0.f, k2 = 0.f, q2 = 0.f;
    if (t < D) {
        float kk = IN::to_f32(k[vec + t]);
        float qq = IN::to_f32(q[vec + t]);
        float g = IN::to_f32(SG ? log_alpha[unit] : log_alpha[vec + t]);
        if constexpr (FUSE) {
            if (fu.flags & 4) {
                // logsigmoid(g + bias) / scale, stable for any g
                const float x = g + fu.decay_bias;
                g = (fminf(x, 0.f) - __builtin_amdgcn_logf(1.f + fast_exp(-fabsf(x))) * 0.6931471805599453f) /
                    fu.decay_scale;
            }
        }
        s_alpha[t] = fast_exp(g);
        s_k[t] = kk;
        s_q[t] = qq;
        kq = kk * qq;
        k2 = kk * kk;
        q2 = qq * qq;
    }
    // k . q (and |k|^2, |q|^2): wave reduction, then across waves through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kq += __shfl_xor(kq, off, 64);
        if constexpr (FUSE) {
            k2 += __shfl_xor(k2, off, 64);
            q2 += __shfl_xor(q2, off, 64);
        }
    }
    if ((t & 63) == 0) {
        s_kq[t >> 6] = kq;
        if constexpr (FUSE) {
            s_kk[t >> 6] = k2;
            s_qq[t >> 6] = q2;
        }
    }
    float b = IN::to_f32(beta[unit]);
    if constexpr (FUSE) {
        if (fu.flags & 2) b = sigmoid_d(b);
    }
    __syncthreads();

    float4 r = make_float4(0.f, 0.f, 0.f, 0.f), p = r;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int c = rg * ROWS + i;
        const float a = s_alpha[c], kc = s_k[c], qc = s_q[c];
        s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;          // S' = Diag(alpha) S
        r.x += kc * s[i].x; r.y += kc * s[i].y; r.z += kc * s[i].z; r.w += kc * s[i].w;
        p.x += qc * s[i].x; p.y += qc * s[i].y; p.z += qc * s[i].z; p.w += qc * s[i].w;
    }
    s_r[rg][cg] = r;
    s_p[rg][cg] = p;
    __syncthreads();

    r = make_float4(0.f, 0.f, 0.f, 0.f);
    p = r;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const float4 a = s_r[g][cg], c = s_p[g][cg];
        r.x += a.x; r.y += a.y; r.z += a.z; r.w += a.w;
        p.x += c.x; p.y += c.y; p.z += c.z; p.w += c.w;
    }
    float kqs = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeThreads / 64; ++w) kqs += s_kq[w];
    float nk = 1.f;   // 1/|k| and 1/|q| under the fused normalisation
    if constexpr (FUSE) {
        if (fu.flags & 1) {
            float kks = 1e-12f, qqs = 1e-12f;
#pragma unroll
            for (int w = 0; w < kDecodeThreads / 64; ++w) {
                kks += s_kk[w];
                qqs += s_qq[w];
            }
            nk = __builtin_amdgcn_rsqf(kks);
            const float nq = __builtin_amdgcn_rsqf(qqs);
            r.x *= nk; r.y *= nk; r.z *= nk; r.w *= nk;
            p.x *= nq; p.y *= nq; p.z *= nq; p.w *= nq;
            kqs *= nk * nq;
        }
    }

    const int j0 = cg * 4;
    float4 e;
    e.x = b * (IN::to_f32(v[vec + j0 + 0]) - r.x);
    e.y = b * (IN::to_f32(v[vec + j0 + 1]) - r.y);
    e.z = b * (IN::to_f32(v[vec + j0 + 2]) - r.z);
    e.w = b * (IN::to_f32(v[vec + j0 + 3]) - r.w);

    const float4 eu = make_float4(nk * e.x, nk * e.y, nk * e.z, nk * e.w);   // k_normalised e^T = k (nk e)^T
    float4* dst = reinterpret_cast<float4*>(S_out + sbase);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const float kc = s_k[rg * ROWS + i];
        float4 x = s[i];
        x.x += kc * eu.x; x.y += kc * eu.y; x.z += kc * eu.z; x.w += kc * eu.w;
        store_stream(&dst[(rg * ROWS + i) * CG + cg], x);
    }
    if (rg == 0) {
        float ov[4] = {p.x + kqs * e.x, p.y + kqs * e.y, p.z + kqs * e.z, p.w + kqs * e.w};
        if constexpr (FUSE) {
            if (fu.out_gate) {
                const typename IN::storage* gp = static_cast<const typename IN::storage*>(fu.out_gate);
#pragma unroll
                for (int c = 0; c < 4; ++c) ov[c] *= sigmoid_d(IN::to_f32(gp[vec + j0 + c]));
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) store_out<OUT_BF16>(o, vec + j0 + c, ov[c]);
    }
}

// ------------------------------------------------------------------ multi-token recurrent forward
// The same rule applied to every token of each sequence in order, with the state held in
// registers between tokens: per (sequence, head) the state is read once and written once,
// whatever the number of tokens.  This is the serving shape of a few new tokens per
// sequence on top of a long context (speculative verification, chunked continuation),
// where a chunk's intra-chunk work would be mostly padding.
//
// Mapping: one workgroup of 2D threads per (sequence, head); the two lanes of a pair own the
// upper and lower half of state column j, so the reductions r = S'^T k and p = S'^T q over
// the key channels are private to the pair (one DPP exchange) and a token needs a single
// workgroup barrier: thread c < D also stages row c's per-token factors in LDS for everyone.
//
// Lazy decay: a thread carries St = Diag(1/A) S with A the product of the decays since
// the last renormalisation (per key channel).  With A' = alpha A,
//     r = St^T (A' k),  p = St^T (A' q),  St <- St + (k / A') e^T,
// three fused multiply-adds per state element and token.  When some A' falls below 2^-32
// the whole workgroup folds A' back into St (St <- Diag(A') St, A <- 1).  A single token's
// decay is taken no smaller than 2^-60 (log_alpha >= -41.59; below that the decayed state is
// negligible against any write), so A' >= 2^-92 and every factor stays well inside fp32.
struct RecArgs {
    const void *q, *k, *v, *g, *beta;
    const float* S0;
    const int32_t* cu;
    void* o;
    float* S_final;
    int T, H;
    DecodeFusion fu;   // fused prologue / epilogue (FUSE kernels only)
};

// x plus the value of the other lane of its pair (DPP quad_perm [1, 0, 3, 2])
__device__ __forceinline__ float pair_sum(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes of a wave, valid in lane 63: butterflies inside quads, half-rows
// and rows, then the row broadcasts (DPP only, no LDS round trip).
__device__ __forceinline__ float wave_sum_lane63(float x) {
    x += dpp_f<0xB1>(x);          // quad_perm [1, 0, 3, 2]
    x += dpp_f<0x4E>(x);          // quad_perm [2, 3, 0, 1]
    x += dpp_f<0x141>(x);         // row_half_mirror
    x += dpp_f<0x140>(x);         // row_mirror
    x += dpp_f<0x142, 0xa>(x);    // row_bcast:15 into rows 1 and 3
    x += dpp_f<0x143, 0xc>(x);    // row_bcast:31 into rows 2 and 3
    return x;
}

// FUSE: the maps of the fused decode step per token (nk = 1/|k|, nq = 1/|q| as per-token
// scalars on the raw products, sigmoid beta, logsigmoid decay, the output gate at the store).
template <int D, typename IN, bool OUT_BF16, bool SG = false, bool FUSE = false>
__global__ __launch_bounds__(2 * D)
void recurrent_fwd_kernel(RecArgs a) {
    using ST = typename IN::storage;
    constexpr int NT = 2 * D, NW = NT / 64, R = D / 2;   // R rows per lane
    constexpr float kRenorm = 2.3283064365386963e-10f;  // 2^-32
    constexpr float kMinLog2Decay = -60.f;

    __shared__ float4 s_f[2][3][D / 4];   // per row c (4 at a time): A' k, A' q, k / A'
    __shared__ float4 s_ren[2][D / 4];    // renormalisation factors A'
    __shared__ float s_kq[2][NW];
    __shared__ float s_kk[2][NW], s_qq[2][NW];   // fused prologue: partial |k|^2, |q|^2
    __shared__ int s_flag[2][NW];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int j = t >> 1, half = t & 1, r0 = half * R;
    const int unit = blockIdx.x, H = a.H;
    const int n = unit / H, h = unit % H;
    long t0, t1;
    if (a.cu) {
        t0 = a.cu[n];
        t1 = a.cu[n + 1];
    } else {
        t0 = static_cast<long>(n) * a.T;
        t1 = t0 + a.T;
    }
    const size_t sbase = static_cast<size_t>(unit) * D * D;

    float st[R];
    if (a.S0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            st[i] = __builtin_nontemporal_load(a.S0 + sbase + static_cast<size_t>(r0 + i) * D + j);
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) st[i] = 0.f;
    }

    const ST* qp = static_cast<const ST*>(a.q);
    const ST* kp = static_cast<const ST*>(a.k);
    const ST* vp = static_cast<const ST*>(a.v);
    const ST* gp = static_cast<const ST*>(a.g);
    const ST* bp = static_cast<const ST*>(a.beta);
    const ST* gtp = FUSE ? static_cast<const ST*>(a.fu.out_gate) : nullptr;
    // token inputs of this thread: channel c (threads t < D) of q, k, log_alpha; column j of v
    // (and of the output gate); beta
    struct Tok { ST q, k, g, v, b, gt; };
    const int c = t < D ? t : t - D;
    // (tokens past the end re-read the last one, so every load is unconditional and in bounds)
    auto load_tok = [&](long tk) {
        const long tc = tk < t1 ? tk : t1 - 1;
        const size_t base = (static_cast<size_t>(tc) * H + h) * D;
        Tok x;
        x.q = qp[base + c];
        x.k = kp[base + c];
        x.g = SG ? gp[static_cast<size_t>(tc) * H + h] : gp[base + c];
        x.v = vp[base + j];
        x.b = bp[static_cast<size_t>(tc) * H + h];
        if constexpr (FUSE) {
            if (gtp) x.gt = gtp[base + j];
        }
        return x;
    };
    float A = 1.f;   // running decay product of row c (threads t < D)
    float ap = 1.f;  // A' of the token staged last
    // Stage token x's factors of row c into buffer buf (threads t < D); returns A'.
    auto stage = [&](const Tok& x, int buf) {
        const float xq = IN::to_f32(x.q), xk = IN::to_f32(x.k);
        float lg = IN::to_f32(x.g) * 1.4426950408889634f;   // log2 of the token's decay
        if constexpr (FUSE) {
            if (a.fu.flags & 4) {   // log2 sigmoid(g + bias) / scale, stable for any g
                const float y = IN::to_f32(x.g) + a.fu.decay_bias;
                lg = (fminf(y, 0.f) * 1.4426950408889634f -
                      __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(y) * 1.4426950408889634f))) /
                     a.fu.decay_scale;
            }
        }
        const float ap = A * __builtin_amdgcn_exp2f(fmaxf(lg, kMinLog2Decay));
        float kq = 0.f, kk = 0.f, qq = 0.f;
        bool low = false;
        if (t < D) {
            reinterpret_cast<float*>(&s_f[buf][0][c >> 2])[c & 3] = ap * xk;
            reinterpret_cast<float*>(&s_f[buf][1][c >> 2])[c & 3] = ap * xq;
            reinterpret_cast<float*>(&s_f[buf][2][c >> 2])[c & 3] = xk * __builtin_amdgcn_rcpf(ap);
            reinterpret_cast<float*>(&s_ren[buf][c >> 2])[c & 3] = ap;
            kq = xk * xq;
            kk = xk * xk;
            qq = xq * xq;
            low = ap < kRenorm;
        }
        kq = wave_sum_lane63(kq);
        if constexpr (FUSE) {
            kk = wave_sum_lane63(kk);
            qq = wave_sum_lane63(qq);
        }
        const bool any_low = __builtin_amdgcn_ballot_w64(low) != 0;
        if (lane == 63) {
            s_kq[buf][w] = kq;
            s_flag[buf][w] = any_low;
            if constexpr (FUSE) {
                s_kk[buf][w] = kk;
                s_qq[buf][w] = qq;
            }
        }
        return ap;
    };

    if (t0 < t1) {
        // One token: stage the next token's factors (from nxt) into the other buffer, then
        // r, p, the output and the state update from buffer buf; cur (token tk's v and beta)
        // is then refilled with token tk + 4.  Four token slots are in flight, so a token's
        // inputs are requested three tokens before its factors are staged.
        auto token = [&](long tk, int buf, Tok& cur, const Tok& nxt) {
            __syncthreads();
            bool ren = false;
            float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                ren |= s_flag[buf][i] != 0;
                kq += s_kq[buf][i];
                if constexpr (FUSE) {
                    kk += s_kk[buf][i];
                    qq += s_qq[buf][i];
                }
            }
            A = ren ? 1.f : ap;
            const float xv = IN::to_f32(cur.v);
            float xb = IN::to_f32(cur.b);
            float nk = 1.f, nq = 1.f, gt = 0.f;
            if constexpr (FUSE) {
                if (a.fu.flags & 1) {
                    nk = __builtin_amdgcn_rsqf(kk + 1e-12f);
                    nq = __builtin_amdgcn_rsqf(qq + 1e-12f);
                }
                if (a.fu.flags & 2) xb = sigmoid_d(xb);
                if (gtp) gt = IN::to_f32(cur.gt);
            }
            if (tk + 1 < t1) ap = stage(nxt, buf ^ 1);
            cur = load_tok(tk + 4);
            float rr[4] = {0.f, 0.f, 0.f, 0.f}, pp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i4 = 0; i4 < R / 4; ++i4) {
                const float4 fk = s_f[buf][0][r0 / 4 + i4], fq = s_f[buf][1][r0 / 4 + i4];
                const int m = i4 & 3;
                rr[m] += fk.x * st[4 * i4] + fk.y * st[4 * i4 + 1] + fk.z * st[4 * i4 + 2] + fk.w * st[4 * i4 + 3];
                pp[m] += fq.x * st[4 * i4] + fq.y * st[4 * i4 + 1] + fq.z * st[4 * i4 + 2] + fq.w * st[4 * i4 + 3];
            }
            const float r = nk * pair_sum((rr[0] + rr[1]) + (rr[2] + rr[3]));
            const float p = nq * pair_sum((pp[0] + pp[1]) + (pp[2] + pp[3]));
            const float e = xb * (xv - r);
            if (half == 0) {
                float ov = p + (kq * (nk * nq)) * e;
                if constexpr (FUSE) {
                    if (gtp) ov *= sigmoid_d(gt);
                }
                store_out<OUT_BF16>(a.o, (static_cast<size_t>(tk) * H + h) * D + j, ov);
            }
            const float ek = nk * e;   // the update takes the normalised key: k (e / |k|)
#pragma unroll
            for (int i4 = 0; i4 < R / 4; ++i4) {
                const float4 fu = s_f[buf][2][r0 / 4 + i4];
                st[4 * i4] += fu.x * ek;
                st[4 * i4 + 1] += fu.y * ek;
                st[4 * i4 + 2] += fu.z * ek;
                st[4 * i4 + 3] += fu.w * ek;
            }
            if (ren) {
#pragma unroll
                for (int i4 = 0; i4 < R / 4; ++i4) {
                    const float4 f = s_ren[buf][r0 / 4 + i4];
                    st[4 * i4] *= f.x;
                    st[4 * i4 + 1] *= f.y;
                    st[4 * i4 + 2] *= f.z;
                    st[4 * i4 + 3] *= f.w;
                }
            }
        };
        Tok x0 = load_tok(t0), x1 = load_tok(t0 + 1), x2 = load_tok(t0 + 2), x3 = load_tok(t0 + 3);
        ap = stage(x0, 0);
        // four tokens per trip with fixed slot roles (no register rotation, which would make
        // each trip wait for the newest loads)
        for (long base = t0; base < t1; base += 4) {
            token(base, 0, x0, x1);
            if (base + 1 >= t1) break;
            token(base + 1, 1, x1, x2);
            if (base + 2 >= t1) break;
            token(base + 2, 0, x2, x3);
            if (base + 3 >= t1) break;
            token(base + 3, 1, x3, x0);
        }
        // fold the remaining decay product into the state (row c's A lives in thread c)
        __syncthreads();
        if (t < D) reinterpret_cast<float*>(&s_ren[0][c >> 2])[c & 3] = A;
        __syncthreads();
#pragma unroll
        for (int i4 = 0; i4 < R / 4; ++i4) {
            const float4 f = s_ren[0][r0 / 4 + i4];
            st[4 * i4] *= f.x;
            st[4 * i4 + 1] *= f.y;
            st[4 * i4 + 2] *= f.z;
            st[4 * i4 + 3] *= f.w;
        }
    }
    if (a.S_final) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            __builtin_nontemporal_store(st[i], a.S_final + sbase + static_cast<size_t>(r0 + i) * D + j);
    }
}

template <int D, typename IN, bool OUT_BF16, bool SG, bool FUSE = false>
static hipError_t launch_recurrent_t(const RecArgs& a, int units, hipStream_t stream) {
    hipLaunchKernelGGL((recurrent_fwd_kernel<D, IN, OUT_BF16, SG, FUSE>), dim3(units), dim3(2 * D), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_recurrent_fwd(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                                const void* v, const void* g, const void* b, const float* S0,
                                const int32_t* cu, int T, int H, int units, void* o, float* S_final,
                                hipStream_t stream, bool scalar_gate, const Fusion* fusion) {
    RecArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = b;
    a.S0 = S0; a.cu = cu; a.o = o; a.S_final = S_final; a.T = T; a.H = H;
    const bool fused = fusion && (fusion->flags || fusion->out_gate);
    a.fu = fused ? DecodeFusion{fusion->flags, fusion->decay_bias, fusion->decay_scale, fusion->out_gate}
                 : DecodeFusion{0, 0.f, 1.f, nullptr};
#define KDA_REC_CASE(DD, INT, OB)                                                          \
    if (D == DD && in_bf16 == std::is_same<INT, BF16>::value && out_bf16 == OB) {            \
        if (fused) return scalar_gate ? launch_recurrent_t<DD, INT, OB, true, true>(a, units, stream) \
                                      : launch_recurrent_t<DD, INT, OB, false, true>(a, units, stream); \
        return scalar_gate ? launch_recurrent_t<DD, INT, OB, true>(a, units, stream)               \
                           : launch_recurrent_t<DD, INT, OB, false>(a, units, stream);             \
    }
    KDA_REC_CASE(128, BF16, true)
    KDA_REC_CASE(128, BF16, false)
    KDA_REC_CASE(128, F32, true)
    KDA_REC_CASE(128, F32, false)
    KDA_REC_CASE(64, BF16, true)
    KDA_REC_CASE(64, BF16, false)
    KDA_REC_CASE(64, F32, true)
    KDA_REC_CASE(64, F32, false)
#undef KDA_REC_CASE
    return hipErrorInvalidValue;
}

template <int D, typename IN, bool OUT_BF16, bool SG, bool FUSE = false>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* g,
                                  const void* b, const float* S_in, float* S_out, void* o,
                                  int units, hipStream_t stream, DecodeFusion fu = DecodeFusion{0, 0.f, 1.f, nullptr}) {
    using T = typename IN::storage;
    hipLaunchKernelGGL((decode_step_kernel<D, IN, OUT_BF16, SG, FUSE>), dim3(units), dim3(kDecodeThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<const T*>(g), static_cast<const T*>(b), S_in, S_out, o, fu);
    return hipGetLastError();
}

// Host-side dispatch over the built variants; arguments already validated.
hipError_t launch_decode(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const void* g, const void* b, const float* S_in,
                         float* S_out, void* o, int units, hipStream_t stream, bool scalar_gate,
                         const Fusion* fusion) {
    const bool fused = fusion && (fusion->flags || fusion->out_gate);
    const DecodeFusion fu = fused ? DecodeFusion{fusion->flags, fusion->decay_bias, fusion->decay_scale,
                                                 fusion->out_gate}
                                  : DecodeFusion{0, 0.f, 1.f, nullptr};
#define KDA_DECODE_CASE(DD, INT, OB)                                                        \
    if (D == DD && in_bf16 == std::is_same<INT, BF16>::value && out_bf16 == OB) {             \
        if (fused) return scalar_gate ? launch_decode_t<DD, INT, OB, true, true>(q, k, v, g, b, S_in, S_out, o, units, stream, fu) \
                         : launch_decode_t<DD, INT, OB, false, true>(q, k, v, g, b, S_in, S_out, o, units, stream, fu); \
        return scalar_gate ? launch_decode_t<DD, INT, OB, true>(q, k, v, g, b, S_in, S_out, o, units, stream) \
                           : launch_decode_t<DD, INT, OB, false>(q, k, v, g, b, S_in, S_out, o, units, stream); \
    }
    KDA_DECODE_CASE(128, BF16, true)
    KDA_DECODE_CASE(128, BF16, false)
    KDA_DECODE_CASE(128, F32, true)
    KDA_DECODE_CASE(128, F32, false)
    KDA_DECODE_CASE(64, BF16, true)
    KDA_DECODE_CASE(64, BF16, false)
    KDA_DECODE_CASE(64, F32, true)
    KDA_DECODE_CASE(64, F32, false)
#undef KDA_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
