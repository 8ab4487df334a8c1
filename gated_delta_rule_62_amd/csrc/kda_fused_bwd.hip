// kda_fused_bwd.hip -- the elementwise steps of the fused layer's gradient (gfx950).
//
// The fused layer applies maps to its raw inputs before the gated delta rule and a gate to its
// output: q, k L2-normalised per (token, head) (x / sqrt(sum x^2 + 1e-12), the normalised
// keys of "Decoding Hybrid Attention Architectures", intl.cloud.baidu.com article 9569726,
// section 3.2), beta = sigmoid of a logit, log_alpha = logsigmoid(a + bias) / scale of a logit,
// o <- o sigmoid(gate).  Its gradient is the chain rule through those maps around the gradient
// of the rule itself (kda_backward.hip), which runs on the mapped inputs in fp32:
//   fused_pre_kernel   raw inputs -> mapped q, k, beta, log_alpha, v (fp32), the upstream
//                      gradient of the ungated output d_o sigmoid(gate), and 1/|q|, 1/|k|
//   fused_post_kernel  the rule's gradients -> gradients of the raw inputs:
//                      dx = (dx' - x' (x' . dx')) / |x| for x' = x / |x|,
//                      db = dbeta s (1 - s) with s = sigmoid(b),
//                      da = dlog_alpha (1 - sigmoid(a + bias)) / scale,
//                      dgate = d_o o s (1 - s) with s = sigmoid(gate) and o the ungated output.
// Eight consecutive values of a (token, head) row of Dk = Dv = D values per lane (16-byte
// accesses), D / 8 lanes per row; the dot products over the row are reductions over those lanes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kWavesPerBlock = 4;

// Eight consecutive values of a row in the input's type (16 bytes of bf16 or 32 of fp32), and
// their fp32 widening.
template <class IN>
struct Vec8 {
    static constexpr bool B16 = std::is_same<IN, BF16>::value;
    float x[8];
    __device__ __forceinline__ void load(const void* p, size_t i) {
        if constexpr (B16) {
            const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = __uint_as_float(u[j] << 16);
                x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
            const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
    }
};

// One value of a per-row input ([tokens, H]) in fp32.
template <class IN>
__device__ __forceinline__ float ld_in(const void* p, size_t i, IN) {
    return IN::to_f32(static_cast<const typename IN::storage*>(p)[i]);
}

__device__ __forceinline__ void load8(float (&x)[8], const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<float4*>(p) = float4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<float4*>(p + 4) = float4{x[4], x[5], x[6], x[7]};
}

// Eight outputs: fp32, or the round-to-nearest-even bf16 of each (16 bytes).
template <bool OUT_BF16>
__device__ __forceinline__ void store_out8(void* base, size_t i, const float (&x)[8]) {
    if constexpr (OUT_BF16) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const __bf16 lo = static_cast<__bf16>(x[2 * j]), hi = static_cast<__bf16>(x[2 * j + 1]);
            w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        *reinterpret_cast<uint4*>(static_cast<__bf16*>(base) + i) = uint4{w[0], w[1], w[2], w[3]};
    } else {
        store8(static_cast<float*>(base) + i, x);
    }
}

// Sum over the LPR lanes of one row (an aligned group of LPR lanes of the wave).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// sigmoid(x) without overflow for any x
__device__ __forceinline__ float sigm(float x) {
    const float e = fast_exp(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// log(sigmoid(x)) = min(x, 0) - log1p(e^-|x|)
__device__ __forceinline__ float logsigm(float x) { return fminf(x, 0.f) - log1pf(fast_exp(-fabsf(x))); }

// Rows of D values, 8 consecutive values per lane: LPR = D / 8 lanes per row, 64 / LPR rows per
// wave.  The launch covers every row; the lanes of a row past the last exit together.
template <int D>
struct RowMap {
    static constexpr int LPR = D / 8, RPW = 64 / LPR, RPB = RPW * kWavesPerBlock;
    size_t row;
    int c, first;
    __device__ __forceinline__ RowMap() {
        const int t = threadIdx.x;
        row = static_cast<size_t>(blockIdx.x) * RPB + t / LPR;
        c = 8 * (t % LPR);
        first = t % LPR == 0;
    }
};

template <int D, class IN, bool SG>
__global__ __launch_bounds__(64 * kWavesPerBlock) void fused_pre_kernel(FusedBwdArgs a) {
    using RM = RowMap<D>;
    const RM m;
    if (m.row >= a.rows) return;
    const size_t i = m.row * D + m.c;
    Vec8<IN> q, k, v, d;
    q.load(a.q, i);
    k.load(a.k, i);
    v.load(a.v, i);
    d.load(a.d_o, i);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sq += q.x[j] * q.x[j];
        sk += k.x[j] * k.x[j];
    }
    const bool l2 = a.flags & 1;
    const float rq = l2 ? 1.f / sqrtf(row_sum<RM::LPR>(sq) + 1e-12f) : 1.f;
    const float rk = l2 ? 1.f / sqrtf(row_sum<RM::LPR>(sk) + 1e-12f) : 1.f;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = q.x[j] * rq;
    store8(a.qh + i, o);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = k.x[j] * rk;
    store8(a.kh + i, o);
    store8(a.vf + i, v.x);
    if (a.gate) {
        Vec8<IN> g;
        g.load(a.gate, i);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = d.x[j] * sigm(g.x[j]);
        store8(a.doc + i, o);
    } else {
        store8(a.doc + i, d.x);
    }
    if constexpr (!SG) {
        Vec8<IN> g;
        g.load(a.log_alpha, i);
        if (a.flags & 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = logsigm(g.x[j] + a.decay_bias) / a.decay_scale;
            store8(a.la + i, o);
        } else {
            store8(a.la + i, g.x);
        }
    }
    if (m.first) {
        a.rq[m.row] = rq;
        a.rk[m.row] = rk;
        const float b = ld_in(a.beta, m.row, IN{});
        a.bt[m.row] = (a.flags & 2) ? sigm(b) : b;
        if constexpr (SG) {
            const float x = ld_in(a.log_alpha, m.row, IN{});
            a.la[m.row] = (a.flags & 4) ? logsigm(x + a.decay_bias) / a.decay_scale : x;
        }
    }
}

template <int D, class IN, bool OB, bool SG>
__global__ __launch_bounds__(64 * kWavesPerBlock) void fused_post_kernel(FusedBwdArgs a) {
    using RM = RowMap<D>;
    const RM m;
    if (m.row >= a.rows) return;
    const size_t i = m.row * D + m.c;
    const bool l2 = a.flags & 1;
    float dq[8], dk[8], qh[8], kh[8], o[8];
    load8(dq, a.dqh + i);
    load8(dk, a.dkh + i);
    load8(qh, a.qh + i);
    load8(kh, a.kh + i);
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pq += qh[j] * dq[j];
        pk += kh[j] * dk[j];
    }
    if (l2) {
        pq = row_sum<RM::LPR>(pq);
        pk = row_sum<RM::LPR>(pk);
    }
    const float rq = a.rq[m.row], rk = a.rk[m.row];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = l2 ? (dq[j] - qh[j] * pq) * rq : dq[j];
    store_out8<OB>(a.dq, i, o);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = l2 ? (dk[j] - kh[j] * pk) * rk : dk[j];
    store_out8<OB>(a.dk, i, o);
    load8(o, a.dvf + i);
    store_out8<OB>(a.dv, i, o);
    if constexpr (!SG) {
        load8(o, a.dla + i);
        if (a.flags & 4) {
            Vec8<IN> x;
            x.load(a.log_alpha, i);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = o[j] * sigm(-(x.x[j] + a.decay_bias)) / a.decay_scale;
        }
        store_out8<OB>(a.dla_out, i, o);
    }
    if (a.gate) {
        Vec8<IN> g, d;
        g.load(a.gate, i);
        d.load(a.d_o, i);
        float oc[8];
        load8(oc, a.oc + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float s = sigm(g.x[j]);
            o[j] = d.x[j] * oc[j] * s * (1.f - s);
        }
        store_out8<OB>(a.dgate, i, o);
    }
    if (m.first) {
        const float g = a.dbt[m.row];
        const float s = sigm(ld_in(a.beta, m.row, IN{}));
        store_out<OB>(a.dbeta_out, m.row, (a.flags & 2) ? g * s * (1.f - s) : g);
        if constexpr (SG) {
            const float h = a.dla[m.row];
            store_out<OB>(a.dla_out, m.row,
                          (a.flags & 4) ? h * sigm(-(ld_in(a.log_alpha, m.row, IN{}) + a.decay_bias)) / a.decay_scale : h);
        }
    }
}

template <int D, class IN, bool SG>
hipError_t pre_typed(const FusedBwdArgs& a, hipStream_t st) {
    constexpr int RPB = RowMap<D>::RPB;
    const unsigned grid = static_cast<unsigned>((a.rows + RPB - 1) / RPB);
    fused_pre_kernel<D, IN, SG><<<grid, 64 * kWavesPerBlock, 0, st>>>(a);
    return hipGetLastError();
}

template <int D, class IN, bool OB, bool SG>
hipError_t post_typed(const FusedBwdArgs& a, hipStream_t st) {
    constexpr int RPB = RowMap<D>::RPB;
    const unsigned grid = static_cast<unsigned>((a.rows + RPB - 1) / RPB);
    fused_post_kernel<D, IN, OB, SG><<<grid, 64 * kWavesPerBlock, 0, st>>>(a);
    return hipGetLastError();
}

template <class IN, bool SG>
hipError_t pre_d(const FusedBwdArgs& a, hipStream_t st) {
    return a.D == 64 ? pre_typed<64, IN, SG>(a, st) : pre_typed<128, IN, SG>(a, st);
}

template <class IN, bool OB, bool SG>
hipError_t post_d(const FusedBwdArgs& a, hipStream_t st) {
    return a.D == 64 ? post_typed<64, IN, OB, SG>(a, st) : post_typed<128, IN, OB, SG>(a, st);
}

}  // namespace

hipError_t launch_fused_bwd_pre(const FusedBwdArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (a.in_bf16) return a.scalar_gate ? pre_d<BF16, true>(a, st) : pre_d<BF16, false>(a, st);
    return a.scalar_gate ? pre_d<F32, true>(a, st) : pre_d<F32, false>(a, st);
}

hipError_t launch_fused_bwd_post(const FusedBwdArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (a.in_bf16) {
        if (a.out_bf16) return a.scalar_gate ? post_d<BF16, true, true>(a, st) : post_d<BF16, true, false>(a, st);
        return a.scalar_gate ? post_d<BF16, false, true>(a, st) : post_d<BF16, false, false>(a, st);
    }
    if (a.out_bf16) return a.scalar_gate ? post_d<F32, true, true>(a, st) : post_d<F32, true, false>(a, st);
    return a.scalar_gate ? post_d<F32, false, true>(a, st) : post_d<F32, false, false>(a, st);
}

}  // namespace kda
