// kda_backward.hip -- gradient of the chunkwise KDA prefill on gfx950.
//
// The forward is the chunkwise form of "Decoding Hybrid Attention Architectures"
// (intl.cloud.baidu.com article 9569726), section 4, for the fine-grained gated
// delta rule of its section 3.4; the pages motivate the chunk form by training
// throughput (section 4) but give no backward, so this is the chain rule through that
// form.  Per chunk of C tokens (ragged tails are padded with zero q, k, v, beta and
// zero log-decay, which changes nothing), entry state S, chunk-local cumulative
// log-decay b and m = b at the chunk's midpoint row:
//
//   Q' = Q e^{b-m}, K' = K e^{b-m}, K'' = K e^{m-b}, e_m = e^m, e_n = e^{b_last-m}
//   L = StrictTril(K' K''^T), M = (I + Diag(beta) L)^-1, P = Tril(Q' K''^T)
//   S_m = Diag(e_m) S,  R = V - K' S_m,  E = M Diag(beta) R
//   O = Q' S_m + P E,   S_next = Diag(e_n)(S_m + K''^T E)
//
// and with dS_n = Diag(e_n) dS_next (dS_next: gradient with respect to the exit state)
//
//   dE = P^T dO + K'' dS_n,  dY = M^T dE,  dV = Diag(beta) dY
//   dS = Diag(e_m)(dS_n + Q'^T dO - K'^T dV)                       (entry-state gradient)
//   dbeta = rowsum(dY R) + rowsum(dA L),  dA = -StrictTril(dY E^T),  dL = Diag(beta) dA
//   dP = Tril(dO E^T)
//   dQ' = dO S_m^T + dP K'',  dK' = -dV S_m^T + dL K'',  dK'' = dP^T Q' + dL^T K' + E dS_n^T
//   dq = e^{b-m} dQ',  dk = e^{b-m} dK' + e^{m-b} dK''
//   db = Q' dQ' + K' dK' - K'' dK'' (+ rowsum(dS_next S_next) on the last row)
//   dlog_alpha = reverse cumulative sum of db over the chunk's rows.
//
// Kernels (operands from LDS; products on the fp32 matrix cores for fp32 inputs, and as
// split-bf16 products on the bf16 matrix cores for bf16 inputs, whose tolerance is wider;
// the state passes also keep R = V - K' S_m and dE of every chunk, which the gradient step
// reads instead of recomputing):
//   seq_scan_kernel   packed batches: first chunk index of every sequence
//   prep_kernel       per (chunk, head): Q', K', K'', M, P, L, e_m, e_n, beta, b - m -> record
//   state_fwd_kernel  per (sequence, head, 16 value columns): every chunk's entry state
//                     and the final state, chunks in order
//   state_rev_kernel  same split: every chunk's dS_next, chunks in reverse order; dS0
//   grad_kernel       per (chunk, head): dq, dk, dv, dlog_alpha, dbeta
// The scalar-gated variant (one log-decay per token and head, broadcast over the key
// channels) runs the same kernels; its dlog_alpha is the per-channel one summed over the
// key channels.
// The state passes are independent per value column because every operator of the
// recurrence multiplies the state from the left.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"
#include "kda_backward.h"

namespace kda {
namespace {

constexpr int BC = 32;    // chunk length
constexpr int BT = 256;   // threads per workgroup (4 waves)
constexpr int TW = 16;    // value columns per state-pass workgroup
constexpr int GW = 32;    // value columns per step of the gradient kernel

using f4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;

// Offsets (in floats) inside the per-(chunk, head) record written by prep_kernel.
template <int D>
struct Rec {
    static constexpr int QP = 0, KP = BC * D, KPP = 2 * BC * D, M = 3 * BC * D, P = M + BC * BC,
                         L = P + BC * BC, EM = L + BC * BC, EN = EM + D, BETA = EN + D, X = BETA + BC,
                         SIZE = X + BC * D;
    static_assert(SIZE % 4 == 0, "records must stay 16-byte aligned");
};

template <class IN>
__device__ __forceinline__ float ld_in(const void* p, size_t i) {
    return IN::to_f32(static_cast<const typename IN::storage*>(p)[i]);
}

// ---------------------------------------------------------------- chunk addressing
// Sequence n owns chunks [chunk0(n), chunk0(n+1)) and state slots chunk0(n) + n + i,
// i = 0..chunks(n) (the last one holds the final state).
__device__ __forceinline__ int chunk0(const BackwardArgs& a, int n) {
    return a.cu ? a.seq_chunk0[n] : n * ((a.T + BC - 1) / BC);
}

// Workspace slot of per-chunk data (record, dS_next, R, dE) and of a state, head-major.
__device__ __forceinline__ size_t cslot(const BackwardArgs& a, int j, int h) { return (size_t)h * a.ncs + j; }
__device__ __forceinline__ size_t sslot(const BackwardArgs& a, size_t j, int h) { return (size_t)h * a.nss + j; }

__device__ __forceinline__ int seq_first_token(const BackwardArgs& a, int n) {
    return a.cu ? a.cu[n] : n * a.T;
}

__device__ __forceinline__ int seq_len(const BackwardArgs& a, int n) {
    return a.cu ? max(a.cu[n + 1] - a.cu[n], 0) : a.T;
}

__device__ __forceinline__ int seq_chunks(const BackwardArgs& a, int n) { return (seq_len(a, n) + BC - 1) / BC; }

// State slot of the entry state of chunk i of sequence n (i = the chunk count: the final state),
// in the compact layout (WIN false) or in the current window's.
template <bool WIN>
__device__ __forceinline__ size_t state_slot(const BackwardArgs& a, int n, int i) {
    return WIN ? (size_t)n * (a.W + 1) + (i - a.w0) : (size_t)chunk0(a, n) + n + i;
}

struct ChunkPos {
    int n, i, t0, len;   // sequence, chunk within it, first token row of [B*T], valid rows
};

// Chunk of per-chunk slot j (the compact layout, or the current window's).
__device__ bool chunk_pos(const BackwardArgs& a, int j, ChunkPos& p) {
    int n;
    if (a.W) {
        n = j / a.W;
        const int i = a.w0 + j % a.W;
        if (n >= a.N || i >= seq_chunks(a, n)) return false;
        p.n = n;
        p.i = i;
        p.t0 = seq_first_token(a, n) + i * BC;
        p.len = min(BC, seq_len(a, n) - i * BC);
        return true;
    }
    if (!a.cu) {
        const int cps = (a.T + BC - 1) / BC;
        if (cps == 0) return false;
        n = j / cps;
        if (n >= a.B) return false;
    } else {
        const int32_t* sc = a.seq_chunk0;
        if (j >= sc[a.N]) return false;
        int lo = 0, hi = a.N - 1;   // last n with sc[n] <= j; then sc[n + 1] > j
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sc[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    }
    p.n = n;
    p.i = j - chunk0(a, n);
    p.t0 = seq_first_token(a, n) + p.i * BC;
    p.len = min(BC, seq_len(a, n) - p.i * BC);
    return true;
}

// ---------------------------------------------------------------- matrix-core helpers
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 32-bit constant in a scalar register: the bf16 pairs (-1, 0) and (0, -1) below must not
// become inline constants, which name a 32-bit float.
__device__ __forceinline__ uint32_t sreg_const(uint32_t v) {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
    return r;
}

// Two fp32 values -> packed bf16 hi = bf16(x) and lo = bf16(x - hi); x - hi is exact and
// v_dot2_f32_bf16 forms it in one instruction as hi . (-e_i) + x_i.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const bf16x2 hb = __builtin_bit_cast(bf16x2, h);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, sreg_const(0x0000bf80u)), x0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, sreg_const(0xbf800000u)), x1, false);
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// Eight fp32 values -> hi and lo bf16x8 operands.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split_pair(x[2 * p], x[2 * p + 1], h[p], l[p]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// acc (16 x 16) += A (16 x K) B (K x 16), A(i, k) = A[i*ai + k*ak], B(k, j) = B[k*bk + j*bj],
// K a multiple of 32.  Lane l holds C(4 (l / 16) + v, l % 16) in acc[v]; the operands of all
// steps are requested before the products so the reads overlap.
//  * SPLIT = false: fp32 matrix cores (v_mfma_f32_16x16x4_f32); lane l supplies A(l % 16,
//    k0 + l / 16) and B(k0 + l / 16, l % 16) for each 4-deep step.
//  * SPLIT = true: bf16 matrix cores.  Every fp32 operand is split into hi + lo bf16 and each
//    32-deep step issues hi.hi + hi.lo + lo.hi (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//    about 16 mantissa bits of each operand (relative error near 2^-16 per product) at 3/16 of
//    the fp32 matrix-core time.  Lane l supplies A(l % 16, k0 + 8 (l / 16) + j) and
//    B(k0 + 8 (l / 16) + j, l % 16), j = 0..7.
template <int K, bool SPLIT>
__device__ __forceinline__ void mma(f4& acc, const float* A, int ai, int ak, const float* B, int bk, int bj) {
    static_assert(K % 32 == 0, "");
    const int lane = threadIdx.x & 63, i = lane & 15, kq = lane >> 4;
    float a[K / 4], b[K / 4];
    if constexpr (SPLIT) {
        const float* pa = A + i * ai + 8 * kq * ak;
        const float* pb = B + 8 * kq * bk + i * bj;
#pragma unroll
        for (int s = 0; s < K / 32; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                a[8 * s + j] = pa[(32 * s + j) * ak];
                b[8 * s + j] = pb[(32 * s + j) * bk];
            }
#pragma unroll
        for (int s = 0; s < K / 32; ++s) {
            bf16x8 ah, al, bh, bl;
            split8(a + 8 * s, ah, al);
            split8(b + 8 * s, bh, bl);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        }
    } else {
        const float* pa = A + i * ai + kq * ak;
        const float* pb = B + kq * bk + i * bj;
#pragma unroll
        for (int s = 0; s < K / 4; ++s) {
            a[s] = pa[4 * s * ak];
            b[s] = pb[4 * s * bk];
        }
#pragma unroll
        for (int s = 0; s < K / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
}

__device__ __forceinline__ int acc_row(int v) { return 4 * ((threadIdx.x & 63) >> 4) + v; }
__device__ __forceinline__ int acc_col() { return threadIdx.x & 15; }

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations, not
// for global loads in flight (a prefetch may stay outstanding across it).  Every
// exchange between waves in these kernels goes through LDS.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Native 4 x fp32 and 2 x u32 vectors: they stay in registers (HIP's v4f is a struct
// whose copies can end up as memory copies through private memory).
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// A ROWS x COLS fp32 block of a dense global array (row stride gs) staged through
// registers: load() issues every global load of the block and nothing waits on them
// until store() writes the block to LDS (row stride ls), so a block can be fetched
// while the previous one is being used.
template <int ROWS, int COLS, int NT = BT>
struct Stage {
    static constexpr int C4 = COLS / 4, N4 = ROWS * C4, IT = (N4 + NT - 1) / NT;
    static_assert(COLS % 4 == 0, "");
    v4f x[IT];
    __device__ __forceinline__ static bool live(int e) { return N4 % NT == 0 || e < N4; }
    __device__ __forceinline__ void load(const float* g, size_t gs) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = threadIdx.x + it * NT;
            if (live(e)) x[it] = *reinterpret_cast<const v4f*>(g + (size_t)(e / C4) * gs + 4 * (e % C4));
        }
    }
    __device__ __forceinline__ void store(float* s, int ls) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = threadIdx.x + it * NT;
            if (live(e)) *reinterpret_cast<v4f*>(s + (e / C4) * ls + 4 * (e % C4)) = x[it];
        }
    }
};

template <int ROWS, int COLS>
__device__ __forceinline__ void s2g(float* g, size_t gs, const float* s, int ls) {
    static_assert(COLS % 4 == 0, "");
    for (int e = threadIdx.x; e < ROWS * COLS / 4; e += BT) {
        const int r = e / (COLS / 4), c = 4 * (e % (COLS / 4));
        *reinterpret_cast<v4f*>(g + r * gs + c) = *reinterpret_cast<const v4f*>(s + r * ls + c);
    }
}

// One chunk's rows [t0, t0 + len) of a [tokens, H, W] input, COLS columns from col0,
// staged like Stage in the input's own type (converted to fp32 on the way to LDS);
// rows past len are zero.
template <class IN, int COLS, int NT = BT>
struct StageRows {
    static constexpr bool B16 = std::is_same<IN, BF16>::value;
    static constexpr int C4 = COLS / 4, N4 = BC * C4, IT = (N4 + NT - 1) / NT;
    static_assert(COLS % 4 == 0, "");
    using raw_t = typename std::conditional<B16, v2u, v4f>::type;
    raw_t x[IT];
    int len_ = 0;
    __device__ __forceinline__ static bool live(int e) { return N4 % NT == 0 || e < N4; }
    // Rows past len read row len - 1 (always in bounds for len >= 1) and are zeroed by
    // store(), so no load sits behind a branch.
    __device__ __forceinline__ void load(const void* p, int t0, int len, int H, int h, int W, int col0) {
        len_ = len;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = threadIdx.x + it * NT, r = min(e / C4, len - 1), c = 4 * (e % C4);
            if (live(e)) {
                const size_t idx = ((size_t)(t0 + r) * H + h) * W + col0 + c;
                x[it] = *reinterpret_cast<const raw_t*>(static_cast<const typename IN::storage*>(p) + idx);
            }
        }
    }
    __device__ __forceinline__ static v4f widen(const raw_t& v) {
        if constexpr (B16) {
            return v4f{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
        } else {
            return v;
        }
    }
    __device__ __forceinline__ void store(float* s, int ls) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = threadIdx.x + it * NT;
            const bool ok = e / C4 < len_;
            v4f v = widen(x[it]);
            v.x = ok ? v.x : 0.f;
            v.y = ok ? v.y : 0.f;
            v.z = ok ? v.z : 0.f;
            v.w = ok ? v.w : 0.f;
            if (live(e)) *reinterpret_cast<v4f*>(s + (e / C4) * ls + 4 * (e % C4)) = v;
        }
    }
};

// The D x TW column tile of a [D, D] state starting at g (or zeros when g is null) into LDS.
template <int D>
__device__ __forceinline__ void init_tile(float* s, int ls, const float* g) {
    for (int e = threadIdx.x; e < D * TW / 4; e += BT) {
        const int r = e / (TW / 4), c = 4 * (e % (TW / 4));
        v4f x{0.f, 0.f, 0.f, 0.f};
        if (g) x = *reinterpret_cast<const v4f*>(g + (size_t)r * D + c);
        *reinterpret_cast<v4f*>(s + r * ls + c) = x;
    }
}

// Maps a linear workgroup index to (unit, column tile) so that the tiles of one unit
// land on one XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
__device__ __forceinline__ void unit_tile(int b, int nwg, int ntile, int& unit, int& tile) {
    int idx = b;
    if (nwg % 8 == 0) idx = (b % 8) * (nwg / 8) + b / 8;
    unit = idx / ntile;
    tile = idx % ntile;
}

// ---------------------------------------------------------------- kernels
__global__ __launch_bounds__(BT) void seq_scan_kernel(const int32_t* cu, int N, int32_t* sc) {
    __shared__ int32_t buf[BT];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += BT) {
        const int n = base + threadIdx.x;
        const int c = n < N ? (max(cu[n + 1] - cu[n], 0) + BC - 1) / BC : 0;
        buf[threadIdx.x] = c;
        __syncthreads();
        for (int off = 1; off < BT; off <<= 1) {
            const int x = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += x;
            __syncthreads();
        }
        const int incl = buf[threadIdx.x];
        if (n < N) sc[n] = carry + incl - c;
        __syncthreads();
        if (threadIdx.x == BT - 1) carry += incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) sc[N] = carry;
}

template <int D, class IN, bool SG>
__global__ __launch_bounds__(BT) void prep_kernel(BackwardArgs a) {
    constexpr bool SPLIT = std::is_same<IN, BF16>::value;   // split-bf16 products for bf16 inputs
    constexpr int LD = D + 4, LC = BC + 4;
    __shared__ __attribute__((aligned(16))) float sQ[BC * LD], sK[BC * LD], sKpp[BC * LD], sG[BC * LD];
    __shared__ __attribute__((aligned(16))) float sL[BC * LC], sP[BC * LC];
    __shared__ float sB[BC], sEm[D], sEn[D];
    const int j = blockIdx.x / a.H, h = blockIdx.x % a.H;
    ChunkPos p;
    if (!chunk_pos(a, j, p)) return;
    const int tid = threadIdx.x, w = tid >> 6;

    {
        StageRows<IN, D> rq, rk, rg;
        rq.load(a.q, p.t0, p.len, a.H, h, D, 0);
        rk.load(a.k, p.t0, p.len, a.H, h, D, 0);
        if constexpr (!SG) rg.load(a.g, p.t0, p.len, a.H, h, D, 0);
        const float bt = tid < p.len ? ld_in<IN>(a.beta, (size_t)(p.t0 + tid) * a.H + h) : 0.f;
        // scalar gate: one log-decay per (token, head), the same for every key channel
        const float gs = SG && tid < p.len ? ld_in<IN>(a.g, (size_t)(p.t0 + tid) * a.H + h) : 0.f;
        rq.store(sQ, LD);
        rk.store(sK, LD);
        if constexpr (!SG) rg.store(sG, LD);
        if (tid < BC) {
            sB[tid] = bt;
            if (SG) sEm[tid] = gs;
        }
    }
    __syncthreads();
    if constexpr (SG) {
        for (int e = tid; e < BC * D; e += BT) sG[(e / D) * LD + e % D] = sEm[e / D];
        __syncthreads();
    }

    if (tid < D) {
        float b = 0.f;
        for (int r = 0; r < BC; ++r) {
            b += sG[r * LD + tid];
            sG[r * LD + tid] = b;
        }
        const float m = sG[(BC / 2 - 1) * LD + tid];
        for (int r = 0; r < BC; ++r) {
            const float x = sG[r * LD + tid] - m;
            sG[r * LD + tid] = x;
            const float up = fast_exp(x), dn = fast_exp(-x);
            const float kv = sK[r * LD + tid];
            sQ[r * LD + tid] *= up;
            sK[r * LD + tid] = kv * up;
            sKpp[r * LD + tid] = kv * dn;
        }
        sEm[tid] = fast_exp(m);
        sEn[tid] = fast_exp(b - m);
    }
    __syncthreads();

    // L and P: the three lower 16x16 tiles of each (the upper-right tile is zero)
    for (int t = w; t < 6; t += 4) {
        const bool isP = t >= 3;
        const int tt = t % 3, ti = tt == 0 ? 0 : 1, tj = tt == 2 ? 1 : 0;
        f4 acc = zero4();
        mma<D, SPLIT>(acc, (isP ? sQ : sK) + 16 * ti * LD, LD, 1, sKpp + 16 * tj * LD, 1, LD);
        float* out = isP ? sP : sL;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * ti + acc_row(v), c = 16 * tj + acc_col();
            out[r * LC + c] = (isP ? r >= c : r > c) ? acc[v] : 0.f;
        }
    }
    {
        const int r = tid / 16, c = 16 + tid % 16;
        sL[r * LC + c] = 0.f;
        sP[r * LC + c] = 0.f;
    }
    __syncthreads();

    float* rec = a.prep + cslot(a, j, h) * Rec<D>::SIZE;
    if (tid < BC) {
        // M = (I + Diag(beta) L)^-1 by forward substitution; lane tid owns column tid.  Row r's
        // sum over i < r runs in four independent partial sums (the dependent chain is a quarter
        // as long).
        float col[BC];
#pragma unroll
        for (int r = 0; r < BC; ++r) {
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < r; ++i) part[i & 3] += sL[r * LC + i] * col[i];
            col[r] = (r == tid ? 1.f : 0.f) - sB[r] * ((part[0] + part[1]) + (part[2] + part[3]));
        }
#pragma unroll
        for (int r = 0; r < BC; ++r) rec[Rec<D>::M + r * BC + tid] = col[r];
    }
    s2g<BC, D>(rec + Rec<D>::QP, D, sQ, LD);
    s2g<BC, D>(rec + Rec<D>::KP, D, sK, LD);
    s2g<BC, D>(rec + Rec<D>::KPP, D, sKpp, LD);
    s2g<BC, BC>(rec + Rec<D>::P, BC, sP, LC);
    s2g<BC, BC>(rec + Rec<D>::L, BC, sL, LC);
    s2g<BC, D>(rec + Rec<D>::X, D, sG, LD);
    if (tid < D) {
        rec[Rec<D>::EM + tid] = sEm[tid];
        rec[Rec<D>::EN + tid] = sEn[tid];
    }
    if (tid < BC) rec[Rec<D>::BETA + tid] = sB[tid];
}

// WM: 0 every chunk (compact layout), 1 the current window, 2 the current window's checkpoint only.
template <int D, class IN, int WM>
__global__ __launch_bounds__(BT) void state_fwd_kernel(BackwardArgs a) {
    constexpr bool WIN = WM != 0, CKPT = WM == 2;
    constexpr bool SPLIT = std::is_same<IN, BF16>::value;   // split-bf16 products for bf16 inputs
    constexpr int LD = D + 4, LC = BC + 4, LT = TW + 4, NTILE = D / TW;
    __shared__ __attribute__((aligned(16))) float sKp[BC * LD], sKpp[BC * LD], sM[BC * LC];
    __shared__ __attribute__((aligned(16))) float sS[D * LT], sR[2 * BC * LT], sE[BC * LT], sV[BC * LT];
    __shared__ float sB[BC], sEm[D], sEn[D];
    int u, jt;
    unit_tile(blockIdx.x, gridDim.x, NTILE, u, jt);
    const int n = u / a.H, h = u % a.H, tid = threadIdx.x, w = tid >> 6;
    const int L = seq_len(a, n), nch = (L + BC - 1) / BC, tok0 = seq_first_token(a, n);
    const size_t DD = (size_t)D * D;
    // chunks [i0, i1) of the sequence: all of them, or the window's
    const int i0 = WIN ? a.w0 : 0, i1 = WIN ? min(nch, a.w0 + a.W) : nch;
    if (WIN && a.w0 > 0 && nch <= a.w0) return;   // the sequence ended before this window
    // per-chunk and state slots of chunk i: c0 + i and s0 + i
    const int c0 = WIN ? n * a.W - a.w0 : chunk0(a, n);
    const size_t s0 = WIN ? (size_t)n * (a.W + 1) - a.w0 : (size_t)c0 + n;
    const float* init = WIN && a.w0 > 0 ? a.ckpt + ((size_t)(a.wi - 1) * a.N * a.H + u) * DD : a.S0 ? a.S0 + (size_t)u * DD : nullptr;
    init_tile<D>(sS, LT, init ? init + jt * TW : nullptr);
    // the next chunk's operands are fetched into registers while this chunk computes
    Stage<BC, D> rKp, rKpp;
    Stage<BC, BC> rM;
    StageRows<IN, TW> rV;
    float rEm = 0.f, rEn = 0.f, rB = 0.f;
    auto fetch = [&](int i) __attribute__((always_inline)) {
        const float* rec = a.prep + cslot(a, c0 + i, h) * Rec<D>::SIZE;
        rKp.load(rec + Rec<D>::KP, D);
        rKpp.load(rec + Rec<D>::KPP, D);
        rM.load(rec + Rec<D>::M, BC);
        rEm = rec[Rec<D>::EM + (tid & (D - 1))];
        rEn = rec[Rec<D>::EN + (tid & (D - 1))];
        rB = rec[Rec<D>::BETA + (tid & (BC - 1))];
        rV.load(a.v, tok0 + i * BC, min(BC, L - i * BC), a.H, h, D, jt * TW);
    };
    // R of the previous chunk, kept in registers until the next chunk's global stores
    constexpr int RQ = BC * TW / BT;
    static_assert(BC * TW % BT == 0 && D * TW % (4 * BT) == 0, "");
    float rkeep[RQ];
    auto store_r = [&](int ic) __attribute__((always_inline)) {
        float* rout = a.rbuf + cslot(a, c0 + ic, h) * BC * D + jt * TW;
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int e = tid + q * BT;
            rout[(size_t)(e / TW) * D + e % TW] = rkeep[q];
        }
    };
    if (i1 > i0) fetch(i0);
    for (int i = i0; i < i1; ++i) {
        lds_barrier();
        rKp.store(sKp, LD);
        rKpp.store(sKpp, LD);
        rM.store(sM, LC);
        rV.store(sV, LT);
        sEm[tid & (D - 1)] = rEm;   // every thread: copies of one value, no divergent wait
        sEn[tid & (D - 1)] = rEn;
        sB[tid & (BC - 1)] = rB;
        // this chunk's global stores (the entry state, the previous chunk's R) go out before the
        // next chunk's loads, so waiting for those loads never waits on a store
        if constexpr (!CKPT) {
            float* slot = a.states + sslot(a, s0 + i, h) * DD + jt * TW;
#pragma unroll
            for (int q = 0; q < D * TW / (4 * BT); ++q) {
                const int e = tid + q * BT, r = e / (TW / 4), c = 4 * (e % (TW / 4));
                *reinterpret_cast<v4f*>(slot + (size_t)r * D + c) = *reinterpret_cast<const v4f*>(sS + r * LT + c);
            }
            if (i > i0) store_r(i - 1);
        }
        if (i + 1 < i1) fetch(i + 1);
        lds_barrier();
        // scale the entry state to S_m
#pragma unroll
        for (int q = 0; q < D * TW / (4 * BT); ++q) {
            const int e = tid + q * BT, r = e / (TW / 4), c = 4 * (e % (TW / 4));
            const v4f x = *reinterpret_cast<const v4f*>(sS + r * LT + c);
            const float m = sEm[r];
            *reinterpret_cast<v4f*>(sS + r * LT + c) = v4f{x.x * m, x.y * m, x.z * m, x.w * m};
        }
        lds_barrier();
        {   // K' S_m, the key-channel sum split in two halves over the waves
            const int rt = w & 1, kh = w >> 1;
            f4 acc = zero4();
            mma<D / 2, SPLIT>(acc, sKp + 16 * rt * LD + kh * (D / 2), LD, 1, sS + kh * (D / 2) * LT, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) sR[kh * BC * LT + (16 * rt + acc_row(v)) * LT + acc_col()] = acc[v];
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < RQ; ++q) {   // R = V - K' S_m (kept for the gradient step), Y = Diag(beta) R
            const int e = tid + q * BT, r = e / TW, c = e % TW;
            const float rr = sV[r * LT + c] - sR[r * LT + c] - sR[BC * LT + r * LT + c];
            rkeep[q] = rr;
            sR[r * LT + c] = sB[r] * rr;
        }
        lds_barrier();
        if (w < 2) {   // E = M Y
            f4 acc = zero4();
            mma<BC, SPLIT>(acc, sM + 16 * w * LC, LC, 1, sR, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) sE[(16 * w + acc_row(v)) * LT + acc_col()] = acc[v];
        }
        lds_barrier();
        for (int rt = w; rt < D / 16; rt += 4) {   // S_next = Diag(e_n)(S_m + K''^T E)
            f4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = sS[(16 * rt + acc_row(v)) * LT + acc_col()];
            mma<BC, SPLIT>(acc, sKpp + 16 * rt, 1, LD, sE, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * rt + acc_row(v);
                sS[r * LT + acc_col()] = acc[v] * sEn[r];
            }
        }
    }
    if (!CKPT && i1 > i0) store_r(i1 - 1);
    __syncthreads();
    // the exit state: the final state or the window's last slot, or in the checkpoint sweep the
    // next window's entry state (only for a sequence that goes on)
    float* slot = a.states + sslot(a, s0 + i1, h) * DD + jt * TW;
    if (CKPT) {
        if (i1 >= nch) return;
        slot = a.ckpt + ((size_t)a.wi * a.N * a.H + u) * DD + jt * TW;
    }
    for (int e = tid; e < D * TW / 4; e += BT) {
        const int r = e / (TW / 4), c = 4 * (e % (TW / 4));
        *reinterpret_cast<v4f*>(slot + (size_t)r * D + c) = *reinterpret_cast<const v4f*>(sS + r * LT + c);
    }
}

template <int D, class IN, bool WIN>
__global__ __launch_bounds__(BT) void state_rev_kernel(BackwardArgs a) {
    constexpr bool SPLIT = std::is_same<IN, BF16>::value;   // split-bf16 products for bf16 inputs
    constexpr int LD = D + 4, LC = BC + 4, LT = TW + 4, NTILE = D / TW;
    __shared__ __attribute__((aligned(16))) float sQp[BC * LD], sKp[BC * LD], sKpp[BC * LD];
    __shared__ __attribute__((aligned(16))) float sM[BC * LC], sP[BC * LC];
    __shared__ __attribute__((aligned(16))) float sS[D * LT], sO[BC * LT], sR[BC * LT], sV[BC * LT];
    __shared__ float sB[BC], sEm[D], sEn[D];
    int u, jt;
    unit_tile(blockIdx.x, gridDim.x, NTILE, u, jt);
    const int n = u / a.H, h = u % a.H, tid = threadIdx.x, w = tid >> 6;
    const int L = seq_len(a, n), nch = (L + BC - 1) / BC, tok0 = seq_first_token(a, n);
    const size_t DD = (size_t)D * D;
    const int i0 = WIN ? a.w0 : 0, i1 = WIN ? min(nch, a.w0 + a.W) : nch;
    if (WIN && a.w0 > 0 && nch <= a.w0) return;   // the sequence ended before this window
    const int c0 = WIN ? n * a.W - a.w0 : chunk0(a, n);   // per-chunk slot of chunk i: c0 + i
    // dS_final where the sequence ends in this window, else the gradient the later window left
    const float* init = WIN && nch > a.w0 + a.W ? a.dcarry + (size_t)u * DD : a.dS_final ? a.dS_final + (size_t)u * DD : nullptr;
    init_tile<D>(sS, LT, init ? init + jt * TW : nullptr);
    // the previous chunk's operands are fetched into registers while this chunk computes
    Stage<BC, D> rQp, rKp, rKpp;
    Stage<BC, BC> rM, rP;
    StageRows<IN, TW> rO;
    float rEm = 0.f, rEn = 0.f, rB = 0.f;
    auto fetch = [&](int i) __attribute__((always_inline)) {
        const float* rec = a.prep + cslot(a, c0 + i, h) * Rec<D>::SIZE;
        rQp.load(rec + Rec<D>::QP, D);
        rKp.load(rec + Rec<D>::KP, D);
        rKpp.load(rec + Rec<D>::KPP, D);
        rM.load(rec + Rec<D>::M, BC);
        rP.load(rec + Rec<D>::P, BC);
        rEm = rec[Rec<D>::EM + (tid & (D - 1))];
        rEn = rec[Rec<D>::EN + (tid & (D - 1))];
        rB = rec[Rec<D>::BETA + (tid & (BC - 1))];
        rO.load(a.dO, tok0 + i * BC, min(BC, L - i * BC), a.H, h, D, jt * TW);
    };
    // dE of the chunk after this one, kept in registers until this chunk's global stores
    constexpr int RQ = BC * TW / BT;
    static_assert(BC * TW % BT == 0 && D * TW % (4 * BT) == 0, "");
    float dkeep[RQ];
    auto store_de = [&](int ic) __attribute__((always_inline)) {
        float* deout = a.debuf + cslot(a, c0 + ic, h) * BC * D + jt * TW;
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int e = tid + q * BT;
            deout[(size_t)(e / TW) * D + e % TW] = dkeep[q];
        }
    };
    if (i1 > i0) fetch(i1 - 1);
    for (int i = i1 - 1; i >= i0; --i) {
        const int j = c0 + i;
        lds_barrier();
        rQp.store(sQp, LD);
        rKp.store(sKp, LD);
        rKpp.store(sKpp, LD);
        rM.store(sM, LC);
        rP.store(sP, LC);
        rO.store(sO, LT);
        sEm[tid & (D - 1)] = rEm;   // every thread: copies of one value, no divergent wait
        sEn[tid & (D - 1)] = rEn;
        sB[tid & (BC - 1)] = rB;
        // this chunk's global stores (its dS_next, the next chunk's dE) go out before the
        // previous chunk's loads, so waiting for those loads never waits on a store
        {
            float* slot = a.dstates + cslot(a, j, h) * DD + jt * TW;
#pragma unroll
            for (int q = 0; q < D * TW / (4 * BT); ++q) {
                const int e = tid + q * BT, r = e / (TW / 4), c = 4 * (e % (TW / 4));
                *reinterpret_cast<v4f*>(slot + (size_t)r * D + c) = *reinterpret_cast<const v4f*>(sS + r * LT + c);
            }
            if (i < i1 - 1) store_de(i + 1);
        }
        if (i > i0) fetch(i - 1);
        lds_barrier();
        // scale dS_next to dS_n
#pragma unroll
        for (int q = 0; q < D * TW / (4 * BT); ++q) {
            const int e = tid + q * BT, r = e / (TW / 4), c = 4 * (e % (TW / 4));
            const v4f x = *reinterpret_cast<const v4f*>(sS + r * LT + c);
            const float m = sEn[r];
            *reinterpret_cast<v4f*>(sS + r * LT + c) = v4f{x.x * m, x.y * m, x.z * m, x.w * m};
        }
        lds_barrier();
        {   // dE = P^T dO + K'' dS_n, the key-channel sum split in two halves over the waves
            // (the second half's partial goes to sV, which holds -dV only later)
            const int rt = w & 1, kh = w >> 1;
            f4 acc = zero4();
            mma<D / 2, SPLIT>(acc, sKpp + 16 * rt * LD + kh * (D / 2), LD, 1, sS + kh * (D / 2) * LT, LT, 1);
            if (kh == 0) mma<BC, SPLIT>(acc, sP + 16 * rt, 1, LC, sO, LT, 1);
            float* part = kh == 0 ? sR : sV;
#pragma unroll
            for (int v = 0; v < 4; ++v) part[(16 * rt + acc_row(v)) * LT + acc_col()] = acc[v];
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < RQ; ++q) {   // dE (kept for the gradient step)
            const int e = tid + q * BT, r = e / TW, c = e % TW;
            const float x = sR[r * LT + c] + sV[r * LT + c];
            sR[r * LT + c] = x;
            dkeep[q] = x;
        }
        lds_barrier();
        if (w < 2) {   // -dV = -Diag(beta) M^T dE
            f4 acc = zero4();
            mma<BC, SPLIT>(acc, sM + 16 * w, 1, LC, sR, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * w + acc_row(v);
                sV[r * LT + acc_col()] = -sB[r] * acc[v];
            }
        }
        lds_barrier();
        for (int rt = w; rt < D / 16; rt += 4) {   // dS = Diag(e_m)(dS_n + Q'^T dO - K'^T dV)
            f4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = sS[(16 * rt + acc_row(v)) * LT + acc_col()];
            mma<BC, SPLIT>(acc, sQp + 16 * rt, 1, LD, sO, LT, 1);
            mma<BC, SPLIT>(acc, sKp + 16 * rt, 1, LD, sV, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * rt + acc_row(v);
                sS[r * LT + acc_col()] = acc[v] * sEm[r];
            }
        }
    }
    if (i1 > i0) store_de(i0);
    __syncthreads();
    // dS0 after the first window; before it, the gradient for the window before this one
    float* out = WIN && a.w0 > 0 ? a.dcarry : a.dS0;
    if (out) {
        for (int e = tid; e < D * TW / 4; e += BT) {
            const int r = e / (TW / 4), c = 4 * (e % (TW / 4));
            *reinterpret_cast<v4f*>(out + (size_t)u * DD + (size_t)r * D + jt * TW + c) =
                *reinterpret_cast<const v4f*>(sS + r * LT + c);
        }
    }
}

// Each wave owns one 16-column tile of D in GRAD_RTW of the chunk's two 16-row tiles (so 8 D /
// GRAD_RTW threads), and waves 0-3 also the four 16 x 16 tiles of the C x GW and C x C products.
constexpr int GRAD_RTW = 2;
template <int D>
constexpr int grad_threads() { return 8 * D / GRAD_RTW; }

template <int D, class IN, bool OB, bool SG>
__global__ __launch_bounds__(grad_threads<D>()) void grad_kernel(BackwardArgs a) {
    constexpr bool SPLIT = std::is_same<IN, BF16>::value;   // split-bf16 products for bf16 inputs
    constexpr int LD = D + 4, LC = BC + 4, LT = GW + 4, NCT = D / GW;
    constexpr int RTW = GRAD_RTW, GT = grad_threads<D>(), NW = GT / 64;   // threads and waves
    static_assert(NW >= 4 && NW == (D / 16) * (2 / RTW), "");
    static_assert(LT == LC, "the C x C products reuse C x GW buffers");
    static_assert(BC * LD <= D * LT, "the decay and db planes reuse the state tiles");
    __shared__ __attribute__((aligned(16))) float sQp[BC * LD], sKp[BC * LD], sKpp[BC * LD];
    __shared__ __attribute__((aligned(16))) float sM[BC * LC], sL[BC * LC];
    __shared__ __attribute__((aligned(16))) float sSm[D * LT], sdSn[D * LT];
    __shared__ __attribute__((aligned(16))) float sV[BC * LT], sY[BC * LT], sO[BC * LT], sE[BC * LT];
    __shared__ __attribute__((aligned(16))) float sdE[BC * LT], sdY[BC * LT], smdV[BC * LT];
    __shared__ float sB[BC], sEm[D], sEn[D], sDbn[D];
    const int j = blockIdx.x / a.H, h = blockIdx.x % a.H;
    ChunkPos p;
    if (!chunk_pos(a, j, p)) return;
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t DD = (size_t)D * D;
    const float* rec = a.prep + cslot(a, j, h) * Rec<D>::SIZE;
    const size_t slot = a.W ? state_slot<true>(a, p.n, p.i) : state_slot<false>(a, p.n, p.i);
    const float* S = a.states + sslot(a, slot, h) * DD;
    const float* dS = a.dstates + cslot(a, j, h) * DD;
    const float* Rg = a.rbuf + cslot(a, j, h) * BC * D;    // R = V - K' S_m of the state pass
    const float* dEg = a.debuf + cslot(a, j, h) * BC * D;  // dE of the reverse pass

    // one column tile of S, dS_next, R, dE and dO, fetched a tile ahead
    Stage<D, GW, GT> rS, rdS;
    Stage<BC, GW, GT> rR, rdE;
    StageRows<IN, GW, GT> rO;
    auto fetch = [&](int ct) __attribute__((always_inline)) {
        rS.load(S + ct * GW, D);
        rdS.load(dS + ct * GW, D);
        rR.load(Rg + ct * GW, D);
        rdE.load(dEg + ct * GW, D);
        rO.load(a.dO, p.t0, p.len, a.H, h, D, ct * GW);
    };
    Stage<BC, D, GT> rX;   // decay exponents b - m, used after the column loop
    {
        Stage<BC, D, GT> r1, r2, r3;
        Stage<BC, BC, GT> r4, r6;
        r1.load(rec + Rec<D>::QP, D);
        r2.load(rec + Rec<D>::KP, D);
        r3.load(rec + Rec<D>::KPP, D);
        r4.load(rec + Rec<D>::M, BC);
        r6.load(rec + Rec<D>::L, BC);
        const float em = rec[Rec<D>::EM + (tid & (D - 1))], en = rec[Rec<D>::EN + (tid & (D - 1))];
        const float bt = rec[Rec<D>::BETA + (tid & (BC - 1))];
        fetch(0);
        rX.load(rec + Rec<D>::X, D);
        r1.store(sQp, LD);
        r2.store(sKp, LD);
        r3.store(sKpp, LD);
        r4.store(sM, LC);
        r6.store(sL, LC);
        if (tid < D) {
            sEm[tid] = em;
            sEn[tid] = en;
            sDbn[tid] = 0.f;
        }
        if (tid < BC) sB[tid] = bt;
    }

    // this wave's 16-column tile dt of D and its row tiles rt0 .. rt0 + RTW - 1
    const int dt = w * RTW / 2, rt0 = RTW == 2 ? 0 : (w & 1);
    f4 dQp[RTW], dKp[RTW], dKpp[RTW];
#pragma unroll
    for (int q = 0; q < RTW; ++q) dQp[q] = dKp[q] = dKpp[q] = zero4();
    f4 dPacc = zero4(), dYE = zero4();
    float dbeta = 0.f;
    const int trt = w & 1, tct = (w >> 1) & 1;   // the C x GW (and C x C) tile of waves 0-3

    for (int ct = 0; ct < NCT; ++ct) {
        lds_barrier();
        rdE.store(sdE, LT);
        rO.store(sO, LT);
#pragma unroll
        for (int it = 0; it < Stage<BC, GW, GT>::IT; ++it) {   // R, and Y = Diag(beta) R
            constexpr int C4 = GW / 4;
            const int e = tid + it * GT, r = e / C4, c = 4 * (e % C4);
            if (Stage<BC, GW, GT>::live(e)) {
                const v4f x = rR.x[it];
                const float b = sB[r];
                *reinterpret_cast<v4f*>(sV + r * LT + c) = x;
                *reinterpret_cast<v4f*>(sY + r * LT + c) = v4f{x.x * b, x.y * b, x.z * b, x.w * b};
            }
        }
        // S_m, dS_n tiles; rowsum(dS_n * S_m), the first part of the last row's db term
        // rowsum(dS_next * S_next) = rowsum(dS_n * (S_m + K''^T E)) (the second part is taken
        // from E dS_n^T after the column loop)
#pragma unroll
        for (int it = 0; it < Stage<D, GW, GT>::IT; ++it) {
            constexpr int C4 = GW / 4;
            const int e = tid + it * GT, r = e / C4, c = 4 * (e % C4);
            const v4f x = rS.x[it], y = rdS.x[it];
            const float em = sEm[r], en = sEn[r];
            *reinterpret_cast<v4f*>(sSm + r * LT + c) = v4f{x.x * em, x.y * em, x.z * em, x.w * em};
            *reinterpret_cast<v4f*>(sdSn + r * LT + c) = v4f{y.x * en, y.y * en, y.z * en, y.w * en};
            float t = (y.x * x.x + y.y * x.y + y.z * x.z + y.w * x.w) * (em * en);
            // the GW / 4 v4f groups of row r sit in consecutive lanes
#pragma unroll
            for (int off = C4 / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
            if (c == 0) sDbn[r] += t;
        }
        if (ct + 1 < NCT) fetch(ct + 1);
        lds_barrier();
        if (w < 4) {
            f4 e = zero4();     // E = M Y
            mma<BC, SPLIT>(e, sM + 16 * trt * LC, LC, 1, sY + 16 * tct, LT, 1);
            f4 y = zero4();     // dY = M^T dE
            mma<BC, SPLIT>(y, sM + 16 * trt, 1, LC, sdE + 16 * tct, LT, 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * trt + acc_row(v), c = 16 * tct + acc_col();
                sE[r * LT + c] = e[v];
                sdY[r * LT + c] = y[v];
                const float dv = sB[r] * y[v];
                smdV[r * LT + c] = -dv;
                if (r < p.len) store_out<OB>(a.dv, ((size_t)(p.t0 + r) * a.H + h) * D + ct * GW + c, dv);
            }
        }
        lds_barrier();
        if (tid < BC) {
            float s = 0.f;
            for (int c = 0; c < GW; ++c) s += sdY[tid * LT + c] * sV[tid * LT + c];
            dbeta += s;
        }
#pragma unroll
        for (int q = 0; q < RTW; ++q) {
            const int rt = rt0 + q;
            mma<GW, SPLIT>(dQp[q], sO + 16 * rt * LT, LT, 1, sSm + 16 * dt * LT, 1, LT);
            mma<GW, SPLIT>(dKp[q], smdV + 16 * rt * LT, LT, 1, sSm + 16 * dt * LT, 1, LT);
            mma<GW, SPLIT>(dKpp[q], sE + 16 * rt * LT, LT, 1, sdSn + 16 * dt * LT, 1, LT);
        }
        // dP (+)= dO E^T, dY E^T on this wave's C x C tile
        if (w < 4) {
            mma<GW, SPLIT>(dPacc, sO + 16 * trt * LT, LT, 1, sE + 16 * tct * LT, 1, LT);
            mma<GW, SPLIT>(dYE, sdY + 16 * trt * LT, LT, 1, sE + 16 * tct * LT, 1, LT);
        }
    }
    lds_barrier();
    {   // db's last-row term, second part: sum over rows t of K''(t, r) (E dS_n^T)(t, r), with
        // E dS_n^T in dKpp before the dP and dL terms join it; channel r belongs to one wave
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < RTW; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                t += sKpp[(16 * (rt0 + q) + acc_row(v)) * LD + 16 * dt + acc_col()] * dKpp[q][v];
        static_assert(RTW == 2, "one wave per channel tile holds all of the chunk's rows");
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        if ((tid & 63) < 16) sDbn[16 * dt + acc_col()] += t;
    }
    // dP = Tril(dO E^T) -> sdE;  dA = -StrictTril(dY E^T) -> sdY  (both C x C, row stride LC)
    if (w < 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * trt + acc_row(v), c = 16 * tct + acc_col();
            sdE[r * LC + c] = r >= c ? dPacc[v] : 0.f;
            sdY[r * LC + c] = r > c ? -dYE[v] : 0.f;
        }
    }
    __syncthreads();
    if (tid < BC) {   // dbeta += rowsum(dA L); dL = Diag(beta) dA (in place)
        float s = 0.f;
        for (int c = 0; c < BC; ++c) {
            const float x = sdY[tid * LC + c];
            s += x * sL[tid * LC + c];
            sdY[tid * LC + c] = sB[tid] * x;
        }
        dbeta += s;
        if (tid < p.len) store_out<OB>(a.dbeta, (size_t)(p.t0 + tid) * a.H + h, dbeta);
    }
    // the decay exponents b - m of this chunk, into the S_m plane as [C][LD]
    float* sX = sSm;
    rX.store(sX, LD);
    __syncthreads();
    float* sDb = sdSn;   // db as [C][LD]
#pragma unroll
    for (int q = 0; q < RTW; ++q) {
        const int rt = rt0 + q;
        mma<BC, SPLIT>(dQp[q], sdE + 16 * rt * LC, LC, 1, sKpp + 16 * dt, LD, 1);   // + dP K''
        mma<BC, SPLIT>(dKp[q], sdY + 16 * rt * LC, LC, 1, sKpp + 16 * dt, LD, 1);   // + dL K''
        mma<BC, SPLIT>(dKpp[q], sdE + 16 * rt, 1, LC, sQp + 16 * dt, LD, 1);        // + dP^T Q'
        mma<BC, SPLIT>(dKpp[q], sdY + 16 * rt, 1, LC, sKp + 16 * dt, LD, 1);        // + dL^T K'
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rt + acc_row(v), c = 16 * dt + acc_col();
            const float x = sX[r * LD + c], up = fast_exp(x), dn = fast_exp(-x);
            const float gq = dQp[q][v], gk = dKp[q][v], gkk = dKpp[q][v];
            sDb[r * LD + c] = sQp[r * LD + c] * gq + sKp[r * LD + c] * gk - sKpp[r * LD + c] * gkk;
            if (r < p.len) {
                const size_t gi = ((size_t)(p.t0 + r) * a.H + h) * D + c;
                store_out<OB>(a.dq, gi, up * gq);
                store_out<OB>(a.dk, gi, up * gk + dn * gkk);
            }
        }
    }
    __syncthreads();
    if constexpr (SG) {
        // one log-decay per token: its gradient is the sum over key channels of the
        // per-channel one, i.e. the reverse cumulative sum of the row sums of db
        constexpr int TPR = GT / BC;   // threads per row
        const int r = tid / TPR, part = tid % TPR, lane = tid & 63;
        float t = 0.f;
        for (int c = part; c < D; c += TPR) t += sDb[r * LD + c];
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
        float* sRow = sY;   // [BC] row sums, then [BC] the channel sum of the last-row term
        if (part == 0) sRow[r] = t;
        if (w == 0) {
            float v = 0.f;
            for (int c = lane; c < D; c += 64) v += sDbn[c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) sRow[BC] = v;
        }
        __syncthreads();
        if (tid < p.len) {
            float acc = sRow[BC];
            for (int q = tid; q < BC; ++q) acc += sRow[q];
            store_out<OB>(a.dg, (size_t)(p.t0 + tid) * a.H + h, acc);
        }
    } else {   // dlog_alpha = reverse cumulative sum of db (last row: + rowsum(dS_next S_next)); the
        // rows are cut into GT / D parts, each part first sums its rows
        constexpr int NP = GT / D, RP = BC / NP;
        const int c = tid % D, part = tid / D;
        float* sPart = sY;
        float tot = 0.f;
        for (int r = part * RP; r < (part + 1) * RP; ++r) tot += sDb[r * LD + c];
        sPart[part * D + c] = tot;
        __syncthreads();
        float s = sDbn[c];
        for (int q = part + 1; q < NP; ++q) s += sPart[q * D + c];
        for (int r = (part + 1) * RP - 1; r >= part * RP; --r) {
            s += sDb[r * LD + c];
            if (r < p.len) store_out<OB>(a.dg, ((size_t)(p.t0 + r) * a.H + h) * D + c, s);
        }
    }
}

template <int D, class IN, bool OB, bool SG>
hipError_t launch_typed(BackwardArgs a, int nc_max, int n_win, hipStream_t st) {
    const int units = a.N * a.H;
    if (a.cu) {
        seq_scan_kernel<<<1, BT, 0, st>>>(a.cu, a.N, a.seq_chunk0);
    }
    if (!a.W) {
        if (nc_max > 0) prep_kernel<D, IN, SG><<<nc_max * a.H, BT, 0, st>>>(a);
        if (units > 0) {
            state_fwd_kernel<D, IN, 0><<<units * (D / TW), BT, 0, st>>>(a);
            state_rev_kernel<D, IN, false><<<units * (D / TW), BT, 0, st>>>(a);
        }
        if (nc_max > 0) grad_kernel<D, IN, OB, SG><<<nc_max * a.H, grad_threads<D>(), 0, st>>>(a);
        return hipGetLastError();
    }
    // Windows of W chunks per sequence.  A forward sweep over windows 0..n_win-2 keeps only the
    // entry state of every later window; then, from the last window to the first, each window
    // rebuilds its chunk records and entry states, runs the reverse pass from the state gradient
    // the later window left, and takes its chunks' gradients.
    const int grid = a.N * a.W * a.H;
    for (int wi = 0; wi + 1 < n_win; ++wi) {
        a.wi = wi;
        a.w0 = wi * a.W;
        prep_kernel<D, IN, SG><<<grid, BT, 0, st>>>(a);
        state_fwd_kernel<D, IN, 2><<<units * (D / TW), BT, 0, st>>>(a);
    }
    for (int wi = n_win - 1; wi >= 0; --wi) {
        a.wi = wi;
        a.w0 = wi * a.W;
        prep_kernel<D, IN, SG><<<grid, BT, 0, st>>>(a);
        state_fwd_kernel<D, IN, 1><<<units * (D / TW), BT, 0, st>>>(a);
        state_rev_kernel<D, IN, true><<<units * (D / TW), BT, 0, st>>>(a);
        grad_kernel<D, IN, OB, SG><<<grid, grad_threads<D>(), 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

BackwardPlan plan_backward(int B, int T, int H, int D, int N, bool varlen) {
    BackwardPlan pl;
    // sum over sequences of ceil(len / C) <= ceil(T / C) + N for a packed batch
    const size_t nc = varlen ? (size_t)((T + BC - 1) / BC) + (size_t)N : (size_t)B * ((T + BC - 1) / BC);
    const size_t rec = D == 64 ? Rec<64>::SIZE : Rec<128>::SIZE;
    auto up256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    pl.nc_max = nc;
    // per (chunk, head): record, entry state, state gradient, R, dE
    const size_t per_chunk = sizeof(float) * (rec + 2 * (size_t)D * D + 2 * (size_t)BC * D);
    const size_t state = sizeof(float) * (size_t)D * D;
    const size_t units = (size_t)N * H;
    size_t limit = kBwdWorkspaceLimit;
    if (const char* e = std::getenv("KDA_BWD_WORKSPACE_LIMIT")) limit = std::strtoull(e, nullptr, 10);
    const size_t full = nc * H * per_chunk + units * state;
    const int cmax = (T + BC - 1) / BC;
    if (!varlen && full > limit && cmax > 1 && units > 0) {
        // Windows of W chunks: the largest W whose data, W + 1 states per (sequence, head) and
        // one checkpoint per later window plus the carried gradient, fit the limit; when none
        // does, the W that needs the least.
        auto need = [&](int w) {
            const size_t nw = (size_t)((cmax + w - 1) / w);
            return units * ((size_t)w * per_chunk + state + nw * state);
        };
        int best = 1;
        size_t best_need = need(1);
        int chosen = 0;
        for (int k = 1; k <= cmax; ++k) {
            const int w = (cmax + k - 1) / k;
            if ((cmax + w - 1) / w != k) continue;   // the same W as a smaller k
            const size_t x = need(w);
            if (x <= limit) {
                chosen = w;
                break;
            }
            if (x < best_need) {
                best_need = x;
                best = w;
            } else if ((size_t)k * k > 4 * (size_t)cmax) {
                break;   // past the least
            }
        }
        pl.W = chosen ? chosen : best;
        pl.n_win = (cmax + pl.W - 1) / pl.W;
        size_t off = 0;
        pl.off_seq = 0;
        pl.off_prep = off;
        off += up256(sizeof(float) * units * pl.W * rec);
        pl.off_states = off;
        off += up256(state * units * (pl.W + 1));
        pl.off_dstates = off;
        off += up256(state * units * pl.W);
        pl.off_r = off;
        off += up256(sizeof(float) * units * pl.W * BC * D);
        pl.off_de = off;
        off += up256(sizeof(float) * units * pl.W * BC * D);
        pl.off_ckpt = off;
        off += up256(state * units * (pl.n_win - 1));
        pl.off_dcarry = off;
        off += up256(state * units);
        pl.workspace_bytes = off;
        return pl;
    }
    size_t off = 0;
    pl.off_seq = off;
    off += up256(varlen ? sizeof(int32_t) * (size_t)(N + 1) : 0);
    pl.off_prep = off;
    off += up256(sizeof(float) * nc * H * rec);
    pl.off_states = off;
    off += up256(sizeof(float) * (nc + (size_t)N) * H * D * D);
    pl.off_dstates = off;
    off += up256(sizeof(float) * nc * H * D * D);
    pl.off_r = off;
    off += up256(sizeof(float) * nc * H * BC * D);
    pl.off_de = off;
    off += up256(sizeof(float) * nc * H * BC * D);
    pl.workspace_bytes = off;
    return pl;
}

hipError_t launch_backward(BackwardArgs a, const BackwardPlan& pl, void* workspace, hipStream_t st) {
    char* ws = static_cast<char*>(workspace);
    a.seq_chunk0 = reinterpret_cast<int32_t*>(ws + pl.off_seq);
    a.prep = reinterpret_cast<float*>(ws + pl.off_prep);
    a.states = reinterpret_cast<float*>(ws + pl.off_states);
    a.dstates = reinterpret_cast<float*>(ws + pl.off_dstates);
    a.rbuf = reinterpret_cast<float*>(ws + pl.off_r);
    a.debuf = reinterpret_cast<float*>(ws + pl.off_de);
    const int nc = static_cast<int>(pl.nc_max);
    a.W = pl.W;
    if (pl.W) {
        a.ckpt = reinterpret_cast<float*>(ws + pl.off_ckpt);
        a.dcarry = reinterpret_cast<float*>(ws + pl.off_dcarry);
        a.ncs = a.N * pl.W;
        a.nss = a.N * (pl.W + 1);
    } else {
        a.ncs = nc;
        a.nss = nc + a.N;
    }
    const int nw = pl.n_win;
#define KDA_BWD_CASE(DD, IN, OB)                                                              \
    if (a.D == DD && a.in_bf16 == std::is_same<IN, BF16>::value && a.out_bf16 == OB)         \
        return a.scalar_gate ? launch_typed<DD, IN, OB, true>(a, nc, nw, st) : launch_typed<DD, IN, OB, false>(a, nc, nw, st);
    KDA_BWD_CASE(128, BF16, false)
    KDA_BWD_CASE(128, BF16, true)
    KDA_BWD_CASE(128, F32, false)
    KDA_BWD_CASE(128, F32, true)
    KDA_BWD_CASE(64, BF16, false)
    KDA_BWD_CASE(64, BF16, true)
    KDA_BWD_CASE(64, F32, false)
    KDA_BWD_CASE(64, F32, true)
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
