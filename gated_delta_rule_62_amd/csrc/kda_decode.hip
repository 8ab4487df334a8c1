// kda_decode.hip -- single-token KDA decode step (gfx950).
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

template <int D, typename IN, bool OUT_BF16>
__global__ __launch_bounds__(kDecodeThreads)
void decode_step_kernel(const typename IN::storage* __restrict__ q,
                        const typename IN::storage* __restrict__ k,
                        const typename IN::storage* __restrict__ v,
                        const typename IN::storage* __restrict__ log_alpha,
                        const typename IN::storage* __restrict__ beta,
                        const float* S_in, float* S_out, void* __restrict__ o) {
    constexpr int CG = D / 4;                 // column groups of 4
    constexpr int RG = kDecodeThreads / CG;   // row groups
    constexpr int ROWS = D / RG;              // rows per thread
    static_assert(ROWS * RG == D && CG * RG == kDecodeThreads, "decode tiling");

    __shared__ float s_alpha[D], s_k[D], s_q[D];
    __shared__ float4 s_r[RG][CG];
    __shared__ float4 s_p[RG][CG];
    __shared__ float s_kq[kDecodeThreads / 64];

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

    float kq = 0.f;
    if (t < D) {
        float kk = IN::to_f32(k[vec + t]);
        float qq = IN::to_f32(q[vec + t]);
        s_alpha[t] = fast_exp(IN::to_f32(log_alpha[vec + t]));
        s_k[t] = kk;
        s_q[t] = qq;
        kq = kk * qq;
    }
    // k . q: wave reduction, then across waves through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off, 64);
    if ((t & 63) == 0) s_kq[t >> 6] = kq;
    const float b = IN::to_f32(beta[unit]);
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

    const int j0 = cg * 4;
    float4 e;
    e.x = b * (IN::to_f32(v[vec + j0 + 0]) - r.x);
    e.y = b * (IN::to_f32(v[vec + j0 + 1]) - r.y);
    e.z = b * (IN::to_f32(v[vec + j0 + 2]) - r.z);
    e.w = b * (IN::to_f32(v[vec + j0 + 3]) - r.w);

    float4* dst = reinterpret_cast<float4*>(S_out + sbase);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const float kc = s_k[rg * ROWS + i];
        float4 x = s[i];
        x.x += kc * e.x; x.y += kc * e.y; x.z += kc * e.z; x.w += kc * e.w;
        store_stream(&dst[(rg * ROWS + i) * CG + cg], x);
    }
    if (rg == 0) {
        store_out<OUT_BF16>(o, vec + j0 + 0, p.x + kqs * e.x);
        store_out<OUT_BF16>(o, vec + j0 + 1, p.y + kqs * e.y);
        store_out<OUT_BF16>(o, vec + j0 + 2, p.z + kqs * e.z);
        store_out<OUT_BF16>(o, vec + j0 + 3, p.w + kqs * e.w);
    }
}

template <int D, typename IN, bool OUT_BF16>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* g,
                                  const void* b, const float* S_in, float* S_out, void* o,
                                  int units, hipStream_t stream) {
    using T = typename IN::storage;
    hipLaunchKernelGGL((decode_step_kernel<D, IN, OUT_BF16>), dim3(units), dim3(kDecodeThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<const T*>(g), static_cast<const T*>(b), S_in, S_out, o);
    return hipGetLastError();
}

// Host-side dispatch over the built variants; arguments already validated.
hipError_t launch_decode(int D, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const void* g, const void* b, const float* S_in,
                         float* S_out, void* o, int units, hipStream_t stream) {
#define KDA_DECODE_CASE(DD, INT, OB)                                                        \
    if (D == DD && in_bf16 == std::is_same<INT, BF16>::value && out_bf16 == OB)               \
        return launch_decode_t<DD, INT, OB>(q, k, v, g, b, S_in, S_out, o, units, stream);
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
