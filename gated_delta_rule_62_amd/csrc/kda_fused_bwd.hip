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
// One wave per (token, head) row of Dk = Dv = D values, D / 64 per lane; the dot products over
// the row are wave reductions.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// sigmoid(x) without overflow for any x
__device__ __forceinline__ float sigm(float x) {
    const float e = fast_exp(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// log(sigmoid(x)) = min(x, 0) - log1p(e^-|x|)
__device__ __forceinline__ float logsigm(float x) { return fminf(x, 0.f) - log1pf(fast_exp(-fabsf(x))); }

template <int D, class IN, bool SG>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fused_pre_kernel(FusedBwdArgs a) {
    constexpr int E = D / 64;
    const size_t row = static_cast<size_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int l = threadIdx.x & 63;
    using S = typename IN::storage;
    const S* q = static_cast<const S*>(a.q);
    const S* k = static_cast<const S*>(a.k);
    const S* v = static_cast<const S*>(a.v);
    const S* dO = static_cast<const S*>(a.d_o);
    const S* gate = static_cast<const S*>(a.gate);
    const S* la = static_cast<const S*>(a.log_alpha);
    const S* bt = static_cast<const S*>(a.beta);
    const size_t base = row * D;
    float qv[E], kv[E], sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = IN::to_f32(q[base + l + 64 * e]);
        kv[e] = IN::to_f32(k[base + l + 64 * e]);
        sq += qv[e] * qv[e];
        sk += kv[e] * kv[e];
    }
    const bool l2 = a.flags & 1;
    const float rq = l2 ? 1.f / sqrtf(wave_sum(sq) + 1e-12f) : 1.f;
    const float rk = l2 ? 1.f / sqrtf(wave_sum(sk) + 1e-12f) : 1.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t i = base + l + 64 * e;
        a.qh[i] = qv[e] * rq;
        a.kh[i] = kv[e] * rk;
        a.vf[i] = IN::to_f32(v[i]);
        const float d = IN::to_f32(dO[i]);
        a.doc[i] = gate ? d * sigm(IN::to_f32(gate[i])) : d;
        if constexpr (!SG) {
            const float x = IN::to_f32(la[i]);
            a.la[i] = (a.flags & 4) ? logsigm(x + a.decay_bias) / a.decay_scale : x;
        }
    }
    if (l == 0) {
        a.rq[row] = rq;
        a.rk[row] = rk;
        const float b = IN::to_f32(bt[row]);
        a.bt[row] = (a.flags & 2) ? sigm(b) : b;
        if constexpr (SG) {
            const float x = IN::to_f32(la[row]);
            a.la[row] = (a.flags & 4) ? logsigm(x + a.decay_bias) / a.decay_scale : x;
        }
    }
}

template <int D, class IN, bool OB, bool SG>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fused_post_kernel(FusedBwdArgs a) {
    constexpr int E = D / 64;
    const size_t row = static_cast<size_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int l = threadIdx.x & 63;
    using S = typename IN::storage;
    const S* dO = static_cast<const S*>(a.d_o);
    const S* gate = static_cast<const S*>(a.gate);
    const S* la = static_cast<const S*>(a.log_alpha);
    const S* bt = static_cast<const S*>(a.beta);
    const size_t base = row * D;
    const bool l2 = a.flags & 1;
    float dq[E], dk[E], pq = 0.f, pk = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t i = base + l + 64 * e;
        dq[e] = a.dqh[i];
        dk[e] = a.dkh[i];
        pq += a.qh[i] * dq[e];
        pk += a.kh[i] * dk[e];
    }
    if (l2) {
        pq = wave_sum(pq);
        pk = wave_sum(pk);
    }
    const float rq = a.rq[row], rk = a.rk[row];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t i = base + l + 64 * e;
        const float gq = l2 ? (dq[e] - a.qh[i] * pq) * rq : dq[e];
        const float gk = l2 ? (dk[e] - a.kh[i] * pk) * rk : dk[e];
        store_out<OB>(a.dq, i, gq);
        store_out<OB>(a.dk, i, gk);
        store_out<OB>(a.dv, i, a.dvf[i]);
        if constexpr (!SG) {
            const float g = a.dla[i];
            store_out<OB>(a.dla_out, i,
                          (a.flags & 4) ? g * sigm(-(IN::to_f32(la[i]) + a.decay_bias)) / a.decay_scale : g);
        }
        if (gate) {
            const float s = sigm(IN::to_f32(gate[i]));
            store_out<OB>(a.dgate, i, IN::to_f32(dO[i]) * a.oc[i] * s * (1.f - s));
        }
    }
    if (l == 0) {
        const float g = a.dbt[row];
        const float s = sigm(IN::to_f32(bt[row]));
        store_out<OB>(a.dbeta_out, row, (a.flags & 2) ? g * s * (1.f - s) : g);
        if constexpr (SG) {
            const float h = a.dla[row];
            store_out<OB>(a.dla_out, row,
                          (a.flags & 4) ? h * sigm(-(IN::to_f32(la[row]) + a.decay_bias)) / a.decay_scale : h);
        }
    }
}

template <int D, class IN, bool SG>
hipError_t pre_typed(const FusedBwdArgs& a, hipStream_t st) {
    const unsigned grid = static_cast<unsigned>((a.rows + kRowsPerBlock - 1) / kRowsPerBlock);
    fused_pre_kernel<D, IN, SG><<<grid, 64 * kRowsPerBlock, 0, st>>>(a);
    return hipGetLastError();
}

template <int D, class IN, bool OB, bool SG>
hipError_t post_typed(const FusedBwdArgs& a, hipStream_t st) {
    const unsigned grid = static_cast<unsigned>((a.rows + kRowsPerBlock - 1) / kRowsPerBlock);
    fused_post_kernel<D, IN, OB, SG><<<grid, 64 * kRowsPerBlock, 0, st>>>(a);
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
