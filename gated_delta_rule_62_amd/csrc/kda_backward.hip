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
//   prep_kernel       per (chunk, head): M, P, L, e_m, e_n, beta, (b - m) log2 e -> record (Q', K', K''
//                     are rebuilt from q, k and b - m where they are read)
//   state_fwd         per (sequence, head, 32 value columns): every chunk's entry state
//                     and the final state, chunks in order
//   state_rev         same split: every chunk's dS_next, chunks in reverse order; dS0 (the two
//                     state passes are independent and run in one launch, state_pair_kernel)
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
constexpr int GW = 32;    // value columns per step of the gradient kernel

using f4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;

// fp32 inputs whose products may run split bf16 (hi + lo, about 16 mantissa bits per operand): the
// gradient of the fused layer on the fp32 mapped values of bf16 raw inputs, whose bound is that of
// bf16 inputs.  Loads and layouts are F32's.
struct F32S : F32 {};

// Offsets (in floats) inside the per-(chunk, head) record written by prep_kernel.
// The decayed keys and queries Q' = Q e^{b-m}, K' = K e^{b-m}, K'' = K e^{m-b} are not kept:
// every reader rebuilds them from q, k and X (b - m in log2 units) with the same fp32 operations,
// which reproduces them bit for bit and keeps the record at 29 KB (d = 128) instead of 77 KB.
template <int D>
struct Rec {
    static constexpr int M = 0, P = M + BC * BC, L = P + BC * BC, EM = L + BC * BC, EN = EM + D, BETA = EN + D,
                         X = BETA + BC, SIZE = X + BC * D;
    static_assert(SIZE % 4 == 0 && X % 4 == 0, "records must stay 16-byte aligned");
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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four fp32 values -> hi and lo bf16x4 operands.
__device__ __forceinline__ void split4(const float* x, bf16x4& hi, bf16x4& lo) {
    uint32_t h[2], l[2];
    split_pair(x[0], x[1], h[0], l[0]);
    split_pair(x[2], x[3], h[1], l[1]);
    hi = __builtin_bit_cast(bf16x4, u32x2{h[0], h[1]});
    lo = __builtin_bit_cast(bf16x4, u32x2{l[0], l[1]});
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

// Four consecutive values of one row of a [tokens, H, D] input in the input's own type (8 bytes of
// bf16 or 16 of fp32), and their fp32 widening.
template <class IN>
struct In4 {
    static constexpr bool B16 = std::is_same<IN, BF16>::value;
    using word = typename std::conditional<B16, v2u, v4f>::type;
    __device__ __forceinline__ static word load(const void* p, size_t idx) {
        return *reinterpret_cast<const word*>(static_cast<const typename IN::storage*>(p) + idx);
    }
    __device__ __forceinline__ static v4f widen(const word& v) {
        if constexpr (B16) {
            return v4f{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
        } else {
            return v;
        }
    }
};

// 2^x on the hardware exp2 unit.  The record keeps the decay exponents in log2 units,
// X2 = (b - m) log2(e) rounded once, so 2^{X2} is fast_exp(b - m) bit for bit.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The decayed operands of four elements of one row, from the input x (q or k) and the decay
// exponents X2: up = x 2^{X2} (Q' or K') and dn = x 2^{-X2} (K''), the same fp32 operations as
// prep_kernel; rows past the chunk's end (ok false) are zero.
__device__ __forceinline__ void decay4(v4f x, v4f X2, bool ok, v4f& up, v4f& dn) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xi = ok ? x[j] : 0.f;
        up[j] = xi * exp2_hw(X2[j]);
        dn[j] = xi * exp2_hw(-X2[j]);
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
    constexpr bool SPLIT = !std::is_same<IN, F32>::value;   // split-bf16 products for BF16 and F32S
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
            const float x2 = (sG[r * LD + tid] - m) * 1.4426950408889634f;   // (b - m) in log2 units
            sG[r * LD + tid] = x2;
            const float up = exp2_hw(x2), dn = exp2_hw(-x2);
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
    s2g<BC, BC>(rec + Rec<D>::P, BC, sP, LC);
    s2g<BC, BC>(rec + Rec<D>::L, BC, sL, LC);
    s2g<BC, D>(rec + Rec<D>::X, D, sG, LD);
    if (tid < D) {
        rec[Rec<D>::EM + tid] = sEm[tid];
        rec[Rec<D>::EN + tid] = sEn[tid];
    }
    if (tid < BC) rec[Rec<D>::BETA + tid] = sB[tid];
}

// ---------------------------------------------------------------- loader / compute state passes
// A state-pass workgroup owns an SW = 32 column slice of one (sequence, head)'s state and runs
// 12 waves.  Waves 0-7 compute: wave w holds columns 16 (w / 4) .. + 15 of the slice and rows
// [(w % 4) D/4, (w % 4 + 1) D/4) of the state in MFMA accumulators (NT = D / 64 stacked 16 x 16
// tiles; lane l holds rows 16 q + 4 (l / 16) + v, v = 0..3, of tile q at column l % 16).  Waves
// 8-11 load: each chunk's operands go from the record into registers two chunks ahead and into
// one of two LDS slots one chunk ahead, so the computing waves read only LDS and the memory
// latency is hidden behind two chunks of work.  Two workgroup barriers per chunk order both.
constexpr int SW = 32;               // value columns per workgroup
constexpr int SCW = 8, SLW = 4;      // computing and loading waves
constexpr int SLT = 64 * SLW;        // loading threads
constexpr int STH = 64 * (SCW + SLW);

// out (16 x 16) += A X, the sum over this wave's D / 4 state rows, with X the wave's state tiles
// as MFMA B operand (the k index taken in the order the accumulators hold the rows) and
// a[4 q + v] = A(l % 16, row 16 q + 4 (l / 16) + v of the wave).
//  * split bf16, two tiles: one 32-deep step, k slot 8 (l / 16) + j <-> tile j / 4, row 4 (l / 16) + j % 4;
//  * split bf16, one tile: one 16-deep step (v_mfma_f32_16x16x16_bf16);
//  * fp32: 4 NT steps of the 4-deep fp32 product, step (q, v) taking row 16 q + 4 (l / 16) + v.
template <int NT, bool SPLIT>
__device__ __forceinline__ void mma_xb(f4& out, const float (&a)[4 * NT], const f4 (&x)[NT]) {
    if constexpr (!SPLIT) {
#pragma unroll
        for (int q = 0; q < NT; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) out = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * q + v], x[q][v], out, 0, 0, 0);
    } else if constexpr (NT == 2) {
        const float b[8] = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
        bf16x8 ah, al, bh, bl;
        split8(a, ah, al);
        split8(b, bh, bl);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, out, 0, 0, 0);
    } else {
        static_assert(NT == 1, "");
        const float b[4] = {x[0][0], x[0][1], x[0][2], x[0][3]};
        bf16x4 ah, al, bh, bl;
        split4(a, ah, al);
        split4(b, bh, bl);
        out = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, out, 0, 0, 0);
    }
}

// out (16 x 16) += A B over a 32-deep sum, lane l supplying a[j] = A(l % 16, 8 (l / 16) + j) and
// b[j] = B(8 (l / 16) + j, l % 16); the fp32 form takes k = 8 (l / 16) + s in its step s.
template <bool SPLIT>
__device__ __forceinline__ void mma8(f4& out, const float (&a)[8], const float (&b)[8]) {
    if constexpr (SPLIT) {
        bf16x8 ah, al, bh, bl;
        split8(a, ah, al);
        split8(b, bh, bl);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, out, 0, 0, 0);
        out = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, out, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) out = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], out, 0, 0, 0);
    }
}

__device__ __forceinline__ void ld4(float* d, const float* p) {
    const v4f x = *reinterpret_cast<const v4f*>(p);
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
}

// Eight consecutive floats (16-byte aligned).
__device__ __forceinline__ void ld8(float (&d)[8], const float* p) {
    ld4(d, p);
    ld4(d + 4, p + 4);
}

// One 16-byte word of a C x SW block of bf16 or fp32 input per loading thread (8 bf16 or 4 fp32
// values; the bf16 block needs half the threads).
template <class IN>
struct Raw8 {
    static constexpr bool B16 = std::is_same<IN, BF16>::value;
    using word = typename std::conditional<B16, u32x4, v4f>::type;
    static constexpr int PER = B16 ? 8 : 4, WPR = SW / PER, WORDS = BC * WPR;   // values per word, words per row
    static_assert(WORDS <= SLT, "");
};

// Widen one such word to fp32.
template <class IN>
__device__ __forceinline__ void widen8(const typename Raw8<IN>::word& x, float* f) {
    if constexpr (Raw8<IN>::B16) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            f[2 * p] = __uint_as_float(x[p] << 16);
            f[2 * p + 1] = __uint_as_float(x[p] & 0xffff0000u);
        }
    } else {
        f[0] = x.x;
        f[1] = x.y;
        f[2] = x.z;
        f[3] = x.w;
    }
}

// Rows [t0, t0 + len) of a [tokens, H, D] input, this workgroup's SW columns from col0: one word
// per loading thread (rows past len read row len - 1, threads past the block its last word).
template <class IN>
__device__ __forceinline__ typename Raw8<IN>::word load_rows(const void* p, int lt, int t0, int len, int H, int h, int D,
                                                            int col0) {
    using R8 = Raw8<IN>;
    const int e = min(lt, R8::WORDS - 1), r = min(e / R8::WPR, len - 1), c = R8::PER * (e % R8::WPR);
    return *reinterpret_cast<const typename R8::word*>(static_cast<const typename IN::storage*>(p) +
                                                       ((size_t)(t0 + r) * H + h) * D + col0 + c);
}

// ... and its transpose into an LDS plane [column][token] (row stride ls), zero past len.
template <class IN>
__device__ __forceinline__ void put_rows_t(const typename Raw8<IN>::word& x, float* s, int ls, int lt, int len) {
    using R8 = Raw8<IN>;
    if (lt < R8::WORDS) {
        const int r = lt / R8::WPR, c = R8::PER * (lt % R8::WPR);
        float f[R8::PER];
        widen8<IN>(x, f);
#pragma unroll
        for (int p = 0; p < R8::PER; ++p) s[(c + p) * ls + r] = r < len ? f[p] : 0.f;
    }
}

// LDS slot of one chunk's operands for the forward state pass (floats).
template <int D>
struct FwdSlot {
    static constexpr int LK = D + 4, LM = BC + 4, LV = BC + 4;
    static constexpr int KP = 0, KPP = BC * LK, M = 2 * BC * LK, EM = M + BC * LM, EN = EM + D, BETA = EN + D,
                         VT = BETA + BC, SIZE = VT + SW * LV;   // VT: V^T, [column][token]
    static_assert(SIZE % 4 == 0, "");
};

// The loading waves' registers for one chunk: K rows and the decay exponents X of the same
// elements (K' and K'' are formed from them on the way to LDS), M, e_m / e_n / beta, and V.
template <int D, class IN>
struct FwdLoad {
    static constexpr int NK = BC * D / 4 / SLT;   // groups of 4 elements of K' (and K'') per thread
    static_assert(BC * D / 4 % SLT == 0 && BC * BC / 4 == SLT && 2 * D / 4 + BC / 4 <= SLT, "");
    typename In4<IN>::word k[NK];
    v4f x[NK], m, small;
    typename Raw8<IN>::word v;
};

// WM: 0 every chunk (compact layout), 1 the current window, 2 the current window's checkpoint only.
//
// Per chunk: (A) every computing wave scales its rows to S_m = Diag(e_m) S and forms its partial of
// Y = K' S_m over its rows; (B) R = V - Y, and one 16 x 16 tile each of E = M Diag(beta) R on the
// computing waves of row group 0 and 1; (C) every computing wave updates its rows,
// S <- Diag(e_n)(S_m + K''^T E).  The loading waves fill the next chunk's slot during (B).
template <int D>
struct alignas(16) FwdShared {
    float slot[2 * FwdSlot<D>::SIZE];
    float y[SCW * 16 * (BC + 4)], e[2 * 16 * (BC + 4)];
};

template <int D, class IN, int WM>
__device__ __forceinline__ void state_fwd_body(const BackwardArgs& a, FwdShared<D>& sh, int block, int nblocks) {
    constexpr bool WIN = WM != 0, CKPT = WM == 2;
    constexpr bool SPLIT = !std::is_same<IN, F32>::value;   // split-bf16 products for BF16 and F32S
    constexpr int NT = D / 64, NTILE = D / SW, LY = BC + 4;
    using SL = FwdSlot<D>;
    float* const sSlot = sh.slot;
    float* const sY = sh.y;
    float* const sE = sh.e;
    int u, jt;
    unit_tile(block, nblocks, NTILE, u, jt);
    const int n = u / a.H, h = u % a.H, tid = threadIdx.x, w = tid >> 6;
    const int L = seq_len(a, n), nch = (L + BC - 1) / BC, tok0 = seq_first_token(a, n);
    const size_t DD = (size_t)D * D;
    // chunks [i0, i1) of the sequence: all of them, or the window's
    const int i0 = WIN ? a.w0 : 0, i1 = WIN ? min(nch, a.w0 + a.W) : nch;
    if (WIN && a.w0 > 0 && nch <= a.w0) return;   // the sequence ended before this window
    // per-chunk and state slots of chunk i: c0 + i and s0 + i
    const int c0 = WIN ? n * a.W - a.w0 : chunk0(a, n);
    const size_t s0 = WIN ? (size_t)n * (a.W + 1) - a.w0 : (size_t)c0 + n;
    if (i1 <= i0) {   // nothing to do but pass the entry state through (an empty sequence)
        const float* init = WIN && a.w0 > 0 ? a.ckpt + ((size_t)(a.wi - 1) * a.N * a.H + u) * DD : a.S0 ? a.S0 + (size_t)u * DD : nullptr;
        if (CKPT) return;
        float* slot = a.states + sslot(a, s0 + i1, h) * DD + jt * SW;
        for (int e = tid; e < D * SW; e += STH)
            slot[(size_t)(e / SW) * D + e % SW] = init ? init[(size_t)(e / SW) * D + jt * SW + e % SW] : 0.f;
        return;
    }

    if (w >= SCW) {
        // ------------------------------------------------ loading waves
        const int lt = tid - 64 * SCW;
        using LDS_ = FwdLoad<D, IN>;
        auto load = [&](LDS_& x, int i) __attribute__((always_inline)) {
            i = min(i, i1 - 1);   // past the end: the last chunk again (never used)
            const float* rec = a.prep + cslot(a, c0 + i, h) * Rec<D>::SIZE;
            const int len = min(BC, L - i * BC);
#pragma unroll
            for (int k = 0; k < LDS_::NK; ++k) {
                const int e = lt + k * SLT, r = min(e / (D / 4), len - 1), c = 4 * (e % (D / 4));
                x.k[k] = In4<IN>::load(a.k, ((size_t)(tok0 + i * BC + r) * a.H + h) * D + c);
                x.x[k] = *reinterpret_cast<const v4f*>(rec + Rec<D>::X + 4 * e);
            }
            x.m = *reinterpret_cast<const v4f*>(rec + Rec<D>::M + 4 * lt);
            // e_m, e_n and beta are contiguous in the record: D + D + C floats
            x.small = *reinterpret_cast<const v4f*>(rec + Rec<D>::EM + 4 * min(lt, (2 * D + BC) / 4 - 1));
            // V rows of this workgroup's columns
            x.v = load_rows<IN>(a.v, lt, tok0 + i * BC, min(BC, L - i * BC), a.H, h, D, jt * SW);
        };
        auto put = [&](const LDS_& x, int i) __attribute__((always_inline)) {
            float* sl = sSlot + (i & 1) * SL::SIZE;
            const int len = min(BC, L - min(i, i1 - 1) * BC);
#pragma unroll
            for (int k = 0; k < LDS_::NK; ++k) {
                const int e = lt + k * SLT, r = e / (D / 4), c = 4 * (e % (D / 4));
                v4f kp, kpp;
                decay4(In4<IN>::widen(x.k[k]), x.x[k], r < len, kp, kpp);
                *reinterpret_cast<v4f*>(sl + SL::KP + r * SL::LK + c) = kp;
                *reinterpret_cast<v4f*>(sl + SL::KPP + r * SL::LK + c) = kpp;
            }
            *reinterpret_cast<v4f*>(sl + SL::M + (lt / (BC / 4)) * SL::LM + 4 * (lt % (BC / 4))) = x.m;
            if (lt < (2 * D + BC) / 4) *reinterpret_cast<v4f*>(sl + SL::EM + 4 * lt) = x.small;
            put_rows_t<IN>(x.v, sl + SL::VT, SL::LV, lt, len);
        };
        LDS_ xa, xb;
        // chunk i0 into its slot now; i0 + 1 and i0 + 2 into registers
        load(xa, i0);
        put(xa, i0);
        load(xb, i0 + 1);
        load(xa, i0 + 2);
        lds_barrier();
        // per chunk i: during (B) the slot of chunk i + 1 is written (from the registers loaded two
        // chunks before) and chunk i + 3 is requested into the same registers.  Chunks go in pairs
        // with no branch inside (an odd count ends with an idle step that the computing waves
        // match), so each wait covers exactly the older register set.
        for (int i = i0; i < i1; i += 2) {
            lds_barrier();                 // B1 of chunk i
            put(xb, i + 1);
            load(xb, i + 3);
            lds_barrier();                 // B2 of chunk i
            lds_barrier();                 // B1 of chunk i + 1
            put(xa, i + 2);
            load(xa, i + 4);
            lds_barrier();                 // B2 of chunk i + 1
        }
        return;
    }

    // ---------------------------------------------------- computing waves
    const int g = (tid & 63) >> 4, li = tid & 15, ct = w >> 2, rg = w & 3;
    const int r0 = rg * (D / 4) + 4 * g, col = jt * SW + 16 * ct + li;   // lane's first row, its column
    const float* init = WIN && a.w0 > 0 ? a.ckpt + ((size_t)(a.wi - 1) * a.N * a.H + u) * DD : a.S0 ? a.S0 + (size_t)u * DD : nullptr;
    f4 S[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[q][v] = init ? init[(size_t)(r0 + 16 * q + v) * D + col] : 0.f;
    float rkeep[8];   // R(8 g + j, col) of the last chunk (row group 0 stores it)
    auto store_r = [&](int ic) __attribute__((always_inline)) {
        if (rg == 0) {
            float* rout = a.rbuf + cslot(a, c0 + ic, h) * BC * D + col;
#pragma unroll
            for (int j = 0; j < 8; ++j) rout[(size_t)(8 * g + j) * D] = rkeep[j];
        }
    };
    lds_barrier();   // chunk i0's slot is ready
    for (int i = i0; i < i1; ++i) {
        const float* sl = sSlot + (i & 1) * SL::SIZE;
        if constexpr (!CKPT) {   // this chunk's entry state, the previous chunk's R
            float* slot = a.states + sslot(a, s0 + i, h) * DD + col;
#pragma unroll
            for (int q = 0; q < NT; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) slot[(size_t)(r0 + 16 * q + v) * D] = S[q][v];
            if (i > i0) store_r(i - 1);
        }
        // (A) S_m and this wave's partial of Y = K' S_m, stored transposed ([column][token])
        f4 Sm[NT];
        {
            float em[4 * NT];
#pragma unroll
            for (int q = 0; q < NT; ++q) ld4(em + 4 * q, sl + SL::EM + r0 + 16 * q);
#pragma unroll
            for (int q = 0; q < NT; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) Sm[q][v] = S[q][v] * em[4 * q + v];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float kp[4 * NT];
#pragma unroll
            for (int q = 0; q < NT; ++q) ld4(kp + 4 * q, sl + SL::KP + (16 * tt + li) * SL::LK + r0 + 16 * q);
            f4 y = zero4();
            mma_xb<NT, SPLIT>(y, kp, Sm);
            *reinterpret_cast<v4f*>(sY + (w * 16 + li) * LY + 16 * tt + 4 * g) = v4f{y[0], y[1], y[2], y[3]};
        }
        lds_barrier();   // B1
        // (B) R = V - Y (kept for the gradient step) and E = M Diag(beta) R; row groups 0 and 1
        // take token tile rg of their column half
        if (rg < 2) {
            float yb[8], br[8], vt[8], bt[8];
            ld8(br, sY + ((4 * ct) * 16 + li) * LY + 8 * g);
#pragma unroll
            for (int p = 1; p < 4; ++p) {
                ld8(yb, sY + ((4 * ct + p) * 16 + li) * LY + 8 * g);
#pragma unroll
                for (int j = 0; j < 8; ++j) br[j] += yb[j];
            }
            ld8(vt, sl + SL::VT + (16 * ct + li) * SL::LV + 8 * g);
            ld8(bt, sl + SL::BETA + 8 * g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                rkeep[j] = vt[j] - br[j];
                br[j] = bt[j] * rkeep[j];
            }
            float m[8];
            ld8(m, sl + SL::M + (16 * rg + li) * SL::LM + 8 * g);
            f4 e = zero4();
            mma8<SPLIT>(e, m, br);
            *reinterpret_cast<v4f*>(sE + (16 * ct + li) * LY + 16 * rg + 4 * g) = v4f{e[0], e[1], e[2], e[3]};
        }
        lds_barrier();   // B2
        // (C) S <- Diag(e_n)(S_m + K''^T E) on this wave's rows
        float eb[8];
        ld8(eb, sE + (16 * ct + li) * LY + 8 * g);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            float kpp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) kpp[j] = sl[SL::KPP + (8 * g + j) * SL::LK + rg * (D / 4) + 16 * q + li];
            f4 acc = Sm[q];
            mma8<SPLIT>(acc, kpp, eb);
            float en[4];
            ld4(en, sl + SL::EN + r0 + 16 * q);
#pragma unroll
            for (int v = 0; v < 4; ++v) S[q][v] = acc[v] * en[v];
        }
    }
    if ((i1 - i0) & 1) {   // the loading waves' idle step
        lds_barrier();
        lds_barrier();
    }
    if (!CKPT) store_r(i1 - 1);
    // the exit state: the final state or the window's last slot, or in the checkpoint sweep the
    // next window's entry state (only for a sequence that goes on)
    float* slot = a.states + sslot(a, s0 + i1, h) * DD + col;
    if (CKPT) {
        if (i1 >= nch) return;
        slot = a.ckpt + ((size_t)a.wi * a.N * a.H + u) * DD + col;
    }
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) slot[(size_t)(r0 + 16 * q + v) * D] = S[q][v];
}

template <int D, class IN, int WM>
__global__ __launch_bounds__(STH) void state_fwd_kernel(BackwardArgs a) {
    __shared__ FwdShared<D> sh;
    state_fwd_body<D, IN, WM>(a, sh, blockIdx.x, gridDim.x);
}

// LDS slot of one chunk's operands for the reverse state pass (floats).
template <int D>
struct RevSlot {
    static constexpr int LK = D + 4, LM = BC + 4, LV = BC + 4;
    static constexpr int QP = 0, KP = BC * LK, KPP = 2 * BC * LK, M = 3 * BC * LK, P = M + BC * LM, EM = P + BC * LM,
                         EN = EM + D, BETA = EN + D, OT = BETA + BC, SIZE = OT + SW * LV;   // OT: dO^T
    static_assert(SIZE % 4 == 0, "");
};

template <int D, class IN>
struct RevLoad {
    static constexpr int NK = BC * D / 4 / SLT;
    static_assert(BC * D / 4 % SLT == 0 && BC * BC / 4 == SLT && 2 * D / 4 + BC / 4 <= SLT, "");
    typename In4<IN>::word q[NK], k[NK];   // Q, K rows; Q', K', K'' are formed on the way to LDS
    v4f x[NK], m, p, small;                 // the decay exponents X of the same elements, M, P, ...
    typename Raw8<IN>::word o;
};

// Per chunk, in reverse: (A) every computing wave scales its rows of dS_next to dS_n = Diag(e_n)
// dS_next and forms its partial of dE = K'' dS_n (+ P^T dO from row groups 0 and 1, one token
// tile each); (B) dE, and one 16 x 16 tile each of -dV = -Diag(beta) M^T dE on row groups 0 and 1;
// (C) every computing wave takes its rows of dS = Diag(e_m)(dS_n + Q'^T dO - K'^T dV), the
// earlier chunk's dS_next.  The loading waves fill the earlier chunk's slot during (B).
template <int D>
struct alignas(16) RevShared {
    float slot[2 * RevSlot<D>::SIZE];
    float y[SCW * 16 * (BC + 4)], v[2 * 16 * (BC + 4)];
};

template <int D, class IN, bool WIN>
__device__ __forceinline__ void state_rev_body(const BackwardArgs& a, RevShared<D>& sh, int block, int nblocks) {
    constexpr bool SPLIT = !std::is_same<IN, F32>::value;   // split-bf16 products for BF16 and F32S
    constexpr int NT = D / 64, NTILE = D / SW, LY = BC + 4;
    using SL = RevSlot<D>;
    float* const sSlot = sh.slot;
    float* const sY = sh.y;
    float* const sV = sh.v;
    int u, jt;
    unit_tile(block, nblocks, NTILE, u, jt);
    const int n = u / a.H, h = u % a.H, tid = threadIdx.x, w = tid >> 6;
    const int L = seq_len(a, n), nch = (L + BC - 1) / BC, tok0 = seq_first_token(a, n);
    const size_t DD = (size_t)D * D;
    const int i0 = WIN ? a.w0 : 0, i1 = WIN ? min(nch, a.w0 + a.W) : nch;
    if (WIN && a.w0 > 0 && nch <= a.w0) return;   // the sequence ended before this window
    const int c0 = WIN ? n * a.W - a.w0 : chunk0(a, n);   // per-chunk slot of chunk i: c0 + i
    // dS_final where the sequence ends in this window, else the gradient the later window left
    const float* init = WIN && nch > a.w0 + a.W ? a.dcarry + (size_t)u * DD : a.dS_final ? a.dS_final + (size_t)u * DD : nullptr;
    // dS0 after the first window; before it, the gradient for the window before this one
    float* out = WIN && a.w0 > 0 ? a.dcarry : a.dS0;
    if (i1 <= i0) {   // an empty sequence: dS0 = dS_final
        if (out)
            for (int e = tid; e < D * SW; e += STH) {
                const size_t x = (size_t)u * DD + (size_t)(e / SW) * D + jt * SW + e % SW;
                out[x] = init ? init[x - (size_t)u * DD] : 0.f;
            }
        return;
    }

    if (w >= SCW) {
        // ------------------------------------------------ loading waves
        const int lt = tid - 64 * SCW;
        using LDS_ = RevLoad<D, IN>;
        auto load = [&](LDS_& x, int i) __attribute__((always_inline)) {
            i = max(i, i0);   // before the start: the first chunk again (never used)
            const float* rec = a.prep + cslot(a, c0 + i, h) * Rec<D>::SIZE;
            const int len = min(BC, L - i * BC);
#pragma unroll
            for (int k = 0; k < LDS_::NK; ++k) {
                const int e = lt + k * SLT, r = min(e / (D / 4), len - 1), c = 4 * (e % (D / 4));
                const size_t idx = ((size_t)(tok0 + i * BC + r) * a.H + h) * D + c;
                x.q[k] = In4<IN>::load(a.q, idx);
                x.k[k] = In4<IN>::load(a.k, idx);
                x.x[k] = *reinterpret_cast<const v4f*>(rec + Rec<D>::X + 4 * e);
            }
            x.m = *reinterpret_cast<const v4f*>(rec + Rec<D>::M + 4 * lt);
            x.p = *reinterpret_cast<const v4f*>(rec + Rec<D>::P + 4 * lt);
            x.small = *reinterpret_cast<const v4f*>(rec + Rec<D>::EM + 4 * min(lt, (2 * D + BC) / 4 - 1));
            x.o = load_rows<IN>(a.dO, lt, tok0 + i * BC, min(BC, L - i * BC), a.H, h, D, jt * SW);
        };
        auto put = [&](const LDS_& x, int i) __attribute__((always_inline)) {
            float* sl = sSlot + (i & 1) * SL::SIZE;
            const int len = min(BC, L - max(i, i0) * BC);
#pragma unroll
            for (int k = 0; k < LDS_::NK; ++k) {
                const int e = lt + k * SLT, r = e / (D / 4), c = 4 * (e % (D / 4));
                v4f qp, kp, kpp, unused;
                decay4(In4<IN>::widen(x.q[k]), x.x[k], r < len, qp, unused);
                decay4(In4<IN>::widen(x.k[k]), x.x[k], r < len, kp, kpp);
                *reinterpret_cast<v4f*>(sl + SL::QP + r * SL::LK + c) = qp;
                *reinterpret_cast<v4f*>(sl + SL::KP + r * SL::LK + c) = kp;
                *reinterpret_cast<v4f*>(sl + SL::KPP + r * SL::LK + c) = kpp;
            }
            const int mr = lt / (BC / 4), mc = 4 * (lt % (BC / 4));
            *reinterpret_cast<v4f*>(sl + SL::M + mr * SL::LM + mc) = x.m;
            *reinterpret_cast<v4f*>(sl + SL::P + mr * SL::LM + mc) = x.p;
            if (lt < (2 * D + BC) / 4) *reinterpret_cast<v4f*>(sl + SL::EM + 4 * lt) = x.small;
            put_rows_t<IN>(x.o, sl + SL::OT, SL::LV, lt, len);
        };
        LDS_ xa, xb;
        // chunk i1 - 1 into its slot now; i1 - 2 and i1 - 3 into registers
        load(xa, i1 - 1);
        put(xa, i1 - 1);
        load(xb, i1 - 2);
        load(xa, i1 - 3);
        lds_barrier();
        // per chunk i (descending): during (B) the slot of chunk i - 1 is written and chunk i - 3
        // is requested into the same registers; pairs with no branch inside, as in the forward pass
        for (int i = i1 - 1; i >= i0; i -= 2) {
            lds_barrier();                 // B1 of chunk i
            put(xb, i - 1);
            load(xb, i - 3);
            lds_barrier();                 // B2 of chunk i
            lds_barrier();                 // B1 of chunk i - 1
            put(xa, i - 2);
            load(xa, i - 4);
            lds_barrier();                 // B2 of chunk i - 1
        }
        return;
    }

    // ---------------------------------------------------- computing waves
    const int g = (tid & 63) >> 4, li = tid & 15, ct = w >> 2, rg = w & 3;
    const int r0 = rg * (D / 4) + 4 * g, col = jt * SW + 16 * ct + li;
    f4 dS[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) dS[q][v] = init ? init[(size_t)(r0 + 16 * q + v) * D + col] : 0.f;
    float dkeep[8];   // dE(8 g + j, col) of the chunk after this one (row group 0 stores it)
    auto store_de = [&](int ic) __attribute__((always_inline)) {
        if (rg == 0) {
            float* deout = a.debuf + cslot(a, c0 + ic, h) * BC * D + col;
#pragma unroll
            for (int j = 0; j < 8; ++j) deout[(size_t)(8 * g + j) * D] = dkeep[j];
        }
    };
    lds_barrier();   // chunk i1 - 1's slot is ready
    for (int i = i1 - 1; i >= i0; --i) {
        const float* sl = sSlot + (i & 1) * SL::SIZE;
        {   // this chunk's dS_next, the later chunk's dE
            float* slot = a.dstates + cslot(a, c0 + i, h) * DD + col;
#pragma unroll
            for (int q = 0; q < NT; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) slot[(size_t)(r0 + 16 * q + v) * D] = dS[q][v];
            if (i < i1 - 1) store_de(i + 1);
        }
        float ob[8];   // dO(8 g + j, col)
        ld8(ob, sl + SL::OT + (16 * ct + li) * SL::LV + 8 * g);
        // (A) dS_n and this wave's partial of dE = K'' dS_n (+ P^T dO), stored transposed
        f4 dSn[NT];
        {
            float en[4 * NT];
#pragma unroll
            for (int q = 0; q < NT; ++q) ld4(en + 4 * q, sl + SL::EN + r0 + 16 * q);
#pragma unroll
            for (int q = 0; q < NT; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) dSn[q][v] = dS[q][v] * en[4 * q + v];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float kpp[4 * NT];
#pragma unroll
            for (int q = 0; q < NT; ++q) ld4(kpp + 4 * q, sl + SL::KPP + (16 * tt + li) * SL::LK + r0 + 16 * q);
            f4 y = zero4();
            mma_xb<NT, SPLIT>(y, kpp, dSn);
            if (rg == tt) {   // P^T dO, token tile tt: A(t, s) = P(s, t)
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = sl[SL::P + (8 * g + j) * SL::LM + 16 * tt + li];
                mma8<SPLIT>(y, p, ob);
            }
            *reinterpret_cast<v4f*>(sY + (w * 16 + li) * LY + 16 * tt + 4 * g) = v4f{y[0], y[1], y[2], y[3]};
        }
        lds_barrier();   // B1
        // (B) dE (kept for the gradient step) and -dV = -Diag(beta) M^T dE; row groups 0 and 1 take
        // token tile rg of their column half
        if (rg < 2) {
            float yb[8];
            ld8(dkeep, sY + ((4 * ct) * 16 + li) * LY + 8 * g);
#pragma unroll
            for (int p = 1; p < 4; ++p) {
                ld8(yb, sY + ((4 * ct + p) * 16 + li) * LY + 8 * g);
#pragma unroll
                for (int j = 0; j < 8; ++j) dkeep[j] += yb[j];
            }
            float m[8], bt[4];
#pragma unroll
            for (int j = 0; j < 8; ++j) m[j] = sl[SL::M + (8 * g + j) * SL::LM + 16 * rg + li];   // M^T(t', t) = M(t, t')
            ld4(bt, sl + SL::BETA + 16 * rg + 4 * g);
            f4 x = zero4();
            mma8<SPLIT>(x, m, dkeep);
            *reinterpret_cast<v4f*>(sV + (16 * ct + li) * LY + 16 * rg + 4 * g) =
                v4f{-bt[0] * x[0], -bt[1] * x[1], -bt[2] * x[2], -bt[3] * x[3]};
        }
        lds_barrier();   // B2
        // (C) dS = Diag(e_m)(dS_n + Q'^T dO - K'^T dV) on this wave's rows
        float vb[8];
        ld8(vb, sV + (16 * ct + li) * LY + 8 * g);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            float qp[8], kp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int x = (8 * g + j) * SL::LK + rg * (D / 4) + 16 * q + li;
                qp[j] = sl[SL::QP + x];
                kp[j] = sl[SL::KP + x];
            }
            f4 acc = dSn[q];
            mma8<SPLIT>(acc, qp, ob);
            mma8<SPLIT>(acc, kp, vb);
            float em[4];
            ld4(em, sl + SL::EM + r0 + 16 * q);
#pragma unroll
            for (int v = 0; v < 4; ++v) dS[q][v] = acc[v] * em[v];
        }
    }
    if ((i1 - i0) & 1) {   // the loading waves' idle step
        lds_barrier();
        lds_barrier();
    }
    store_de(i0);
    if (out) {
#pragma unroll
        for (int q = 0; q < NT; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) out[(size_t)u * DD + (size_t)(r0 + 16 * q + v) * D + col] = dS[q][v];
    }
}

// Each wave owns one 16-column tile of D in GRAD_RTW of the chunk's two 16-row tiles (so 8 D /
// GRAD_RTW threads), and waves 0-3 also the four 16 x 16 tiles of the C x GW and C x C products.
// The two state passes of the same chunks in one launch: they are independent (the reverse
// pass reads only the records, dO and the later state gradient), so when each has fewer
// workgroups than the chip has compute units (few sequences and heads) they run side by side.
// Workgroups [0, nf) run the forward pass, the rest the reverse pass.
template <int D, class IN, int WM, bool WIN>
__global__ __launch_bounds__(STH) void state_pair_kernel(BackwardArgs a, int nf) {
    __shared__ union {
        FwdShared<D> f;
        RevShared<D> r;
    } sh;
    if (static_cast<int>(blockIdx.x) < nf) state_fwd_body<D, IN, WM>(a, sh.f, blockIdx.x, nf);
    else state_rev_body<D, IN, WIN>(a, sh.r, blockIdx.x - nf, gridDim.x - nf);
}

constexpr int GRAD_RTW = 2;
template <int D>
constexpr int grad_threads() { return 8 * D / GRAD_RTW; }

template <int D, class IN, bool OB, bool SG>
__global__ __launch_bounds__(grad_threads<D>()) void grad_kernel(BackwardArgs a) {
    constexpr bool SPLIT = !std::is_same<IN, F32>::value;   // split-bf16 products for BF16 and F32S
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
    Stage<BC, D, GT> rX;   // decay exponents (b - m) log2(e): Q', K', K'' now, the decay factors at the end
    {
        using SR = StageRows<IN, D, GT>;
        SR rq, rk;
        Stage<BC, BC, GT> r4, r6;
        rq.load(a.q, p.t0, p.len, a.H, h, D, 0);
        rk.load(a.k, p.t0, p.len, a.H, h, D, 0);
        rX.load(rec + Rec<D>::X, D);
        r4.load(rec + Rec<D>::M, BC);
        r6.load(rec + Rec<D>::L, BC);
        const float em = rec[Rec<D>::EM + (tid & (D - 1))], en = rec[Rec<D>::EN + (tid & (D - 1))];
        const float bt = rec[Rec<D>::BETA + (tid & (BC - 1))];
        fetch(0);
        static_assert(SR::IT == Stage<BC, D, GT>::IT && SR::C4 == Stage<BC, D, GT>::C4, "");
#pragma unroll
        for (int it = 0; it < SR::IT; ++it) {   // Q' = Q e^{b-m}, K' = K e^{b-m}, K'' = K e^{m-b}
            const int e = tid + it * GT, r = e / SR::C4, c = 4 * (e % SR::C4);
            if (SR::live(e)) {
                v4f qp, kp, kpp, unused;
                decay4(SR::widen(rq.x[it]), rX.x[it], r < p.len, qp, unused);
                decay4(SR::widen(rk.x[it]), rX.x[it], r < p.len, kp, kpp);
                *reinterpret_cast<v4f*>(sQp + r * LD + c) = qp;
                *reinterpret_cast<v4f*>(sKp + r * LD + c) = kp;
                *reinterpret_cast<v4f*>(sKpp + r * LD + c) = kpp;
            }
        }
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
            const float x2 = sX[r * LD + c], up = exp2_hw(x2), dn = exp2_hw(-x2);
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
        if (units > 0) state_pair_kernel<D, IN, 0, false><<<2 * units * (D / SW), STH, 0, st>>>(a, units * (D / SW));
        if (nc_max > 0) grad_kernel<D, IN, OB, SG><<<nc_max * a.H, grad_threads<D>(), 0, st>>>(a);
        return hipGetLastError();
    }
    // Windows of W chunks per sequence.  A forward sweep over windows 0..n_win-2 keeps only the
    // entry state of every later window; then, from the last window to the first, each window
    // rebuilds its chunk records and entry states, runs the reverse pass from the state gradient
    // the later window left, and takes its chunks' gradients.
    const int grid = a.N * a.W * a.H;
    // The checkpoints.  bf16 inputs (parity bound 2e-3): all windows' entry states at once, from
    // the prefill's segment summaries (segments = windows) chained by its combine, in scratch that
    // the window data takes over afterwards.  fp32 inputs, or when that scratch does not fit: a
    // sweep over the windows, each rebuilding its records and running the forward state pass.
    bool ckpt_done = false;
    if constexpr (std::is_same<IN, BF16>::value) {
        const size_t avail = static_cast<size_t>(reinterpret_cast<char*>(a.ckpt) - reinterpret_cast<char*>(a.prep));
        if (segment_states_workspace_bytes(a.N, a.H, D, n_win) <= avail) {
            PrefillArgs pa;
            pa.q = a.q; pa.k = a.k; pa.v = a.v; pa.g = a.g; pa.beta = a.beta;
            pa.S0 = a.S0; pa.cu = nullptr; pa.o = nullptr; pa.S_final = nullptr; pa.workspace = a.prep;
            pa.B = a.B; pa.T = a.T; pa.H = a.H; pa.D = D; pa.N = a.N;
            pa.in_bf16 = true; pa.out_bf16 = false; pa.scalar_gate = SG;
            const hipError_t e = launch_segment_states(pa, a.W, n_win, a.ckpt, st);
            if (e != hipSuccess) return e;
            ckpt_done = true;
        }
    }
    for (int wi = 0; !ckpt_done && wi + 1 < n_win; ++wi) {
        a.wi = wi;
        a.w0 = wi * a.W;
        prep_kernel<D, IN, SG><<<grid, BT, 0, st>>>(a);
        state_fwd_kernel<D, IN, 2><<<units * (D / SW), STH, 0, st>>>(a);
    }
    for (int wi = n_win - 1; wi >= 0; --wi) {
        a.wi = wi;
        a.w0 = wi * a.W;
        prep_kernel<D, IN, SG><<<grid, BT, 0, st>>>(a);
        state_pair_kernel<D, IN, 1, true><<<2 * units * (D / SW), STH, 0, st>>>(a, units * (D / SW));
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
    if (a.split_fp32 && !a.in_bf16) {
        KDA_BWD_CASE(128, F32S, false)
        KDA_BWD_CASE(128, F32S, true)
        KDA_BWD_CASE(64, F32S, false)
        KDA_BWD_CASE(64, F32S, true)
    }
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
