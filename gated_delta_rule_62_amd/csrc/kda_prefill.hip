// kda_prefill.hip -- chunkwise KDA prefill for gfx950 (MI355X).
//
// Method: the chunkwise parallel form of the fine-grained gated delta rule
// ("Decoding Hybrid Attention Architectures", intl.cloud.baidu.com article 9569726,
// section 4; "Technical Analysis and Engineering Practices for Novel Hybrid Linear
// Attention Architectures", article 9578008, section 3).  Per chunk of C tokens (32 by
// default, 64 on request) with entry state S (d_k x d_v, fp32) and chunk-local
// cumulative log-decay b_r = sum_{i<=r} g_i:
//
//   A    = StrictTril(Diag(beta) Kbar Ktil^T)           Kbar = K e^{b}, Ktil = K e^{-b}
//   T    = (I + A)^{-1} Diag(beta)
//   P    = Tril(Qbar Ktil^T)                             Qbar = Q e^{b}
//   Unew = T (V - Kbar S)                                (= U - W S with U = T V, W = T Kbar)
//   O    = Qbar S + P Unew
//   S   <- Diag(gamma) S + Khat^T Unew                   gamma = e^{b_n}, Khat = K e^{b_n - b}
//
// The pages leave U and W undefined and print the state term with (Gamma.K)^T;
// the reading used here (T as above, keys decayed to the chunk end) is the one
// that reproduces the token recurrence exactly.
//
// MI355X design.
//  * One workgroup runs the whole chunk loop of one (sequence, head[, segment]):
//    intra-chunk operands live in LDS, the state lives in MFMA accumulator
//    registers, and nothing but q, k, v, log_alpha, beta, o and the states
//    touches HBM.  Wave w owns 32 state columns.
//  * Every contraction runs on v_mfma_f32_16x16x32_bf16 with each fp32 operand
//    split into hi + lo bf16 (three MFMAs per product, fp32 accumulation).  A
//    single bf16 rounding of any computed operand would put the output error
//    near 1e-2 relative; the split keeps it near 3e-5.
//  * Accumulator tiles (S, Y, Unew) are fed straight back as MFMA B operands.
//    A 16x16 accumulator holds rows 4*(lane/16)+e of its tile, so two stacked
//    tiles form the 8 values a lane supplies for a 32-deep step once the
//    reduction index is taken in the order kpos() below; the LDS-resident A
//    operands are stored in that order, which costs nothing.
//  * Decay factors are formed relative to the chunk midpoint for the C x C
//    products (e^{b_r - b_m} and e^{b_m - b_i}), so their exponents stay within
//    half a chunk's summed decay.
//  * The (I + A)^{-1} solve is blocked 16 x 16: the diagonal blocks are inverted by
//    substitution in fp32 (X_bb = (I + A_bb)^{-1}), and Unew is formed block by block,
//    Unew_b = X_bb (beta_b R_b - sum_{k<b} A_bk Unew_k), so T itself is never formed.
//    The 32-token kernel inverts its two diagonal blocks on two producer waves (one
//    block-row per lane quad); the 64-token kernel inverts its four on one wave.
//  * Few long sequences (the 64K-token workload has 32 heads): each sequence is
//    cut into G segments.  Pass 1 runs segments from a zero state and also carries
//    the segment transition (the identity pushed through the same updates, which is
//    linear in the state); a combine kernel chains
//    S_entry(s+1) = Phi(s) S_entry(s) + S_loc(s); pass 2 reruns the segments from
//    their entry states.  Segment 0 needs no summary: with 32-token chunks its
//    output pass runs in the same launch as the summaries of segments 1..G-2 (its
//    workgroups take the first compute units), and pass 2 covers segments 1..G-1.
//    That fills the chip at the cost of a second pass; every kernel of a call runs
//    on the caller's stream.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// Position of reduction index L (0..31) inside a 32-deep MFMA step when the B
// operand comes from two stacked accumulator tiles.
__host__ __device__ constexpr int kpos(int L) {
    return L < 16 ? 8 * (L >> 2) + (L & 3) : 8 * ((L - 16) >> 2) + 4 + ((L - 16) & 3);
}
__host__ __device__ constexpr int kperm(int x) { return (x & ~31) | kpos(x & 31); }

__device__ __forceinline__ u16 bits(__bf16 h) { return __builtin_bit_cast(u16, h); }

constexpr float kLog2e = 1.4426950408889634f;
// 2^x on the hardware exp2 unit (v_exp_f32)
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 32-bit constant in a scalar register.  The bf16 pairs (-1, 0) and (0, -1) below must not
// become inline constants: an inline constant names a 32-bit float, not a bf16 pair.
__device__ __forceinline__ uint32_t sreg_const(uint32_t v) {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
    return r;
}

// Two values at once: hi = bf16(x) packed in one word, lo = bf16(x - hi) packed in another.
// x_i - hi_i is exact in fp32; v_dot2_f32_bf16 forms it in one instruction as
// hi . (-e_i) + x_i (the other product is hi_j * 0), so a pair costs two conversions and two
// dot products.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const bf16x2 hb = __builtin_bit_cast(bf16x2, h);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, sreg_const(0x0000bf80u)), x0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, sreg_const(0xbf800000u)), x1, false);
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// Four values -> packed hi and lo words (8 bytes each).
__device__ __forceinline__ void split_quad(float x0, float x1, float x2, float x3, uint2& hi, uint2& lo) {
    split_pair(x0, x1, hi.x, lo.x);
    split_pair(x2, x3, hi.y, lo.y);
}

__device__ __forceinline__ void split2(float x, u16& hi, u16& lo) {
    const __bf16 h = static_cast<__bf16>(x);
    hi = bits(h);
    lo = bits(static_cast<__bf16>(x - static_cast<float>(h)));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// (ah + al)(bh + bl) to fp32 accuracy, dropping only al*bl.
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma(al, bh, c);
    c = mfma(ah, bl, c);
    return mfma(ah, bh, c);
}

__device__ __forceinline__ bf16x8 frag(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 frag4(const u16* p) { return *reinterpret_cast<const bf16x4*>(p); }

// 16x16x16 products: a 16x16 accumulator tile is, as it stands, the K = 16 B operand
// (lane holds rows 4*(lane/16)+e of one column), so tiles chain with no reordering.
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma3_16(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
    c = mfma16(al, bh, c);
    c = mfma16(ah, bl, c);
    return mfma16(ah, bh, c);
}
__device__ __forceinline__ void split4(f32x4 t, bf16x4& hi, bf16x4& lo) {
    uint32_t h0, h1, l0, l1;
    split_pair(t[0], t[1], h0, l0);
    split_pair(t[2], t[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Four consecutive outputs (16-byte fp32 or 8-byte bf16 store; bf16 rounds to nearest even).
template <bool OUT_BF16>
__device__ __forceinline__ void store_out4(void* base, size_t idx, f32x4 x) {
    if constexpr (OUT_BF16) {
        const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
        const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = uint2{w0, w1};
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = x;
    }
}

// Workgroup barrier for LDS traffic only.  The waves of a workgroup exchange data
// through LDS alone, so the barrier waits for this wave's LDS operations and leaves
// global loads (the next chunk's inputs) in flight; __syncthreads() would also wait
// for every outstanding global load.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Counters in LDS that order the producer and consumer waves of a workgroup without a
// workgroup barrier.  A wave publishes with signal_count once its earlier LDS accesses are
// complete; a wave waits with wait_count until a counter reaches a target.  Global loads in
// flight are not waited on by either.  A wait is bounded: after a poll limit (2^16 polls,
// milliseconds, unless the host asks for fewer) it marks the workgroup broken and returns, and
// every later wait returns at once.  A broken workgroup writes NaN to every output row and state
// it stores from then on and sets the call's status word, so an ordering mistake shows as NaN
// results and a nonzero status, never as a stuck workgroup.
struct SyncCounters {
    int p1, p2, ready;   // producer waves done with phase 1, phase 2, a whole chunk
    int pt;              // consumer waves done with the P tiles of the chunk being built
    int done[2];         // consumer waves done with a chunk, per LDS buffer
    int broken;
};

__device__ __forceinline__ void signal_count(int* c) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Explicit LDS accesses (address space 3): a volatile access through a generic pointer
// would become a flat access, whose completion wait also waits for global loads in flight.
typedef __attribute__((address_space(3))) volatile int lds_vint;

__device__ __forceinline__ int lds_read(const int* p) { return *(const lds_vint*)(p); }

__device__ __forceinline__ void wait_count(const int* c, int target, int* broken, int limit) {
    for (int polls = 0;; ++polls) {
        if (__builtin_amdgcn_readfirstlane(lds_read(c)) >= target) break;
        // the first polls follow each other closely; later ones sleep between reads and
        // look at the broken flag every 64 polls
        if (polls >= 8) {
            if ((polls & 63) == 0 && __builtin_amdgcn_readfirstlane(lds_read(broken))) break;
            if (polls >= limit) {
                *(lds_vint*)(broken) = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    asm volatile("" ::: "memory");
}

// Order LDS accesses between lanes of one wave (no workgroup barrier involved).
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Two stacked accumulator tiles -> hi/lo B operands of one 32-deep step.
__device__ __forceinline__ void split_b(f32x4 t0, f32x4 t1, bf16x8& hi, bf16x8& lo) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_pair(t0[0], t0[1], h0, l0);
    split_pair(t0[2], t0[3], h1, l1);
    split_pair(t1[0], t1[1], h2, l2);
    split_pair(t1[2], t1[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

__device__ __forceinline__ void store4(u16* p, const u16 (&x)[4]) {
    uint2 w;
    w.x = static_cast<uint32_t>(x[0]) | (static_cast<uint32_t>(x[1]) << 16);
    w.y = static_cast<uint32_t>(x[2]) | (static_cast<uint32_t>(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = w;
}

template <typename IN>
__device__ __forceinline__ void load4(const typename IN::storage* p, size_t off, float (&out)[4]) {
    if constexpr (std::is_same<IN, F32>::value) {
        const float4 x = *reinterpret_cast<const float4*>(p + off);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p + off);
        out[0] = __uint_as_float(x.x << 16);
        out[1] = __uint_as_float(x.x & 0xffff0000u);
        out[2] = __uint_as_float(x.y << 16);
        out[3] = __uint_as_float(x.y & 0xffff0000u);
    }
}

// ------------------------------------------------------------------ compile-time shape
template <int D, int C, int MODE>
struct Cfg {
    // The output pass at the 32-token chunk gives each of D/16 waves 16 state columns
    // (one 16-wide tile); at the 64-token chunk, whose larger intra-chunk working set
    // needs the full register file, D/32 waves of 32 columns.  The summary pass carries
    // [S | Phi] (2D columns) on D/16 waves, 32 columns each.
    static constexpr int CT = (MODE == 0 && C == 32) ? 1 : 2;  // 16-column tiles per wave
    static constexpr int NW = (MODE == 0 ? D : 2 * D) / (16 * CT);
    static constexpr int NT = 64 * NW;
    static constexpr int CQ = D / 4;                           // channel quads
    // Element phase: each of the first NA threads owns one channel quad over TPG tokens; a
    // wave holds 8 quads for all C tokens (8 token groups), so the decay prefix over tokens
    // stays inside the wave.
    static constexpr int TPG = C / 8;                          // tokens per element-phase thread
    static constexpr int NA = 8 * CQ;                          // threads in the element phase
    static constexpr int NRT = C / 16, NKT = C / 32;           // token row tiles, 32-deep token steps
    static constexpr int RT = D / 16, KS = D / 32;             // state row tiles, 32-deep channel steps
    static constexpr int PK = D + 8;                           // pitch of [token][channel] planes
    static constexpr int PT = C + 8;                           // pitch of [row][token] planes
    static constexpr int NB = C / 16;                          // 16x16 blocks of the solve
    static constexpr int AP = C + 4;                           // pitch of the off-diagonal A planes
    static constexpr int XP = 20;                              // pitch of the diagonal-inverse planes
    static constexpr int NTRI = NRT * (NRT + 1) / 2;           // lower 16x16 tiles of a C x C product
    // Khat^T gets its own LDS region when it fits; otherwise it overwrites Ktil_m after the
    // C x C products that read it.
    static constexpr bool KT_SEP = false;
    static constexpr int KT = KT_SEP ? C * PK : ((C * PK > D * PT) ? C * PK : D * PT);
    static constexpr int KH = KT_SEP ? D * PT : 8;
    static constexpr int WPE = 1;   // one workgroup per compute unit (D/16 waves)
    static_assert(TPG % 4 == 0 && NA <= NT && NA % 64 == 0, "element-phase tiling");
};

// ------------------------------------------------------------------ LDS layout
template <int D, int C, int MODE>
struct Smem {
    using K = Cfg<D, C, MODE>;
    static constexpr int NQ = MODE == 0 ? 2 : 1, QE = MODE == 0 ? C * K::PK : 8;
    static constexpr int NP = MODE == 0 ? 2 : 1, PE = MODE == 0 ? C * K::PT : 8;
    u16 kb[2][C * K::PK];    // Kbar_m = K e^{b - b_m}                 [token][kperm(channel)]
    u16 qb[NQ][QE];          // Qbar_m = Q e^{b - b_m}                 [token][kperm(channel)]
    u16 kt[2][K::KT];        // Ktil_m = K e^{b_m - b} [token][kperm(channel)]; without a
                             // separate region, then Khat^T = (K e^{b_n - b})^T [channel][kperm(token)]
    u16 kh[K::KT_SEP ? 2 : 1][K::KH];   // Khat^T when it has its own region
    float a[K::NB][16][17];  // diagonal 16x16 blocks of A (fp32)
    u16 aoff[2][C * K::AP];  // -A off the diagonal blocks               [token][token]
    u16 xd[2][C * K::XP];    // X_bb = (I + A_bb)^{-1} per diagonal block [16 b + r][c]
    u16 p[NP][PE];           // P = Tril(Qbar Ktil^T)                   [token][kperm(token)]
    float beta[C];
    float em[D];             // e^{b_m}
    float gam[D];            // gamma = e^{b_n}
};

// Raw (undecoded) input registers: bf16 stays packed until it is used.
template <typename IN> struct Raw;
template <> struct Raw<BF16> {
    using quad = uint2;
    using elem = uint16_t;
    static __device__ __forceinline__ float get(const uint2& x, int ch) {
        const uint32_t w = ch < 2 ? x.x : x.y;
        return __uint_as_float((ch & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw<F32> {
    using quad = float4;
    using elem = float;
    static __device__ __forceinline__ float get(const float4& x, int ch) {
        return ch == 0 ? x.x : ch == 1 ? x.y : ch == 2 ? x.z : x.w;
    }
};

struct KernelArgs {
    const void *q, *k, *v, *g, *beta;
    const float* S0;
    const int32_t* cu;
    const int32_t* order;
    const int32_t* seg;   // segment table of a packed batch (nullptr: one pass per sequence)
    void* o;
    float* S_final;
    float* phi;     // [G-1][N*H][D][D] segment transitions
    float* sloc;    // [G-1][N*H][D][D] segment end states from a zero entry
    float* se;      // [G-1][N*H][D][D] entry states of segments 1..G-1
    int T, H, NH, G, cps, chunks;
    int cps0;       // chunks in segment 0 (cps unless the split schedule lengthens or shortens it)
    int seg0;       // segment of the launch's first workgroup row (equal-length batches)
    int split0;     // 1: segment 0's output pass writes its exit state as segment 1's entry
    int* status;    // call status word: set to 1 by a workgroup whose ordering wait gave up
    int wait_limit; // polls before an ordering wait gives up (2^16 unless the host asks for fewer)
    // fused prologue / epilogue (FUSE kernels only)
    int fuse_flags;           // kFuseQK | kFuseBeta | kFuseDecay
    float decay_bias, decay_scale;
    const void* out_gate;     // [B, T, H, D] gate logits or nullptr
};

// MODE 0: outputs (o, S_final) from a known entry state.
// MODE 1: segment summary (S_loc from a zero entry and the transition Phi).
template <int D, int C, typename IN, bool OUT_BF16, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg<D, C, MODE>::NT, Cfg<D, C, MODE>::NT),
                          amdgpu_waves_per_eu(Cfg<D, C, MODE>::NW * Cfg<D, C, MODE>::WPE / 4,
                                              Cfg<D, C, MODE>::NW * Cfg<D, C, MODE>::WPE / 4)))
void chunk_kernel(KernelArgs a) {
    using K = Cfg<D, C, MODE>;
    constexpr int NT = K::NT, NW = K::NW, CT = K::CT, TPG = K::TPG, NA = K::NA;
    constexpr int NRT = K::NRT, NKT = K::NKT, RT = K::RT, KS = K::KS, PK = K::PK, PT = K::PT;
    using ST = typename IN::storage;
    using R = Raw<IN>;
    using quad = typename R::quad;
    using elem = typename R::elem;

    __shared__ Smem<D, C, MODE> sm;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4, lr = l & 15;
    const int H = a.H;

    // ---------------------------------------------------------------- work unit
    int n, h, s, c_begin, c_end;
    long t0, t1;
    if (a.cu) {
        const int rank = blockIdx.x / H;
        h = blockIdx.x % H;
        n = a.order[rank];
        t0 = a.cu[n];
        t1 = a.cu[n + 1];
        s = 0;
        c_begin = 0;
        c_end = static_cast<int>((t1 - t0 + C - 1) / C);
    } else {
        const int unit = blockIdx.x % a.NH;
        s = a.seg0 + blockIdx.x / a.NH;
        n = unit / H;
        h = unit % H;
        t0 = static_cast<long>(n) * a.T;
        t1 = t0 + a.T;
        c_begin = s == 0 ? 0 : a.cps0 + (s - 1) * a.cps;
        c_end = min(s == 0 ? a.cps0 : c_begin + a.cps, a.chunks);
    }
    const int unit = n * H + h;
    const size_t ubase = static_cast<size_t>(unit) * D * D;

    const bool is_phi = MODE == 1 && w >= D / 32;
    const int j0 = MODE == 0 ? 16 * CT * w : 32 * (w % (NW / 2));
    const int cq = 8 * w + (l & 7), tg = l >> 3, c4 = 4 * cq;
    const bool loader = tid < NA;

    // ---------------------------------------------------------------- entry state
    f32x4 S[RT][CT];
    {
        const float* src = nullptr;
        if constexpr (MODE == 0) {
            if (s == 0) src = a.S0 ? a.S0 + ubase : nullptr;
            else src = a.se + (static_cast<size_t>(s - 1) * a.NH + unit) * D * D;
        }
        if (src) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[rt][ct][e] = src[(16 * rt + 4 * g4 + e) * D + j0 + 16 * ct + lr];
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[rt][ct][e] = (is_phi && 16 * rt + 4 * g4 + e == j0 + 16 * ct + lr) ? 1.f : 0.f;
        }
    }
    if constexpr (MODE == 0) {
        // P's strictly-upper 16x16 tiles inside the 32-deep steps are read but never written.
        for (int i = tid; i < 2 * C * PT; i += NT) sm.p[i / (C * PT)][i % (C * PT)] = 0;
    }

    // ---------------------------------------------------------------- input prefetch
    // Rows past the end of a ragged chunk load a valid row (clamped index) and are
    // zeroed when used, so every load is unconditional.
    quad pk[TPG], pq[TPG], pg[TPG];
    elem pb = 0;
    const int HD = H * D;   // elements between consecutive tokens of one head
    auto fetch = [&](int chunk) {
        const long ts = t0 + static_cast<long>(chunk) * C;
        const int last = static_cast<int>(min(static_cast<long>(C), t1 - ts)) - 1;
        const size_t base = (static_cast<size_t>(ts) * H + h) * D;   // uniform
        const ST* kp = static_cast<const ST*>(a.k) + base;
        const ST* gp = static_cast<const ST*>(a.g) + base;
        const ST* qp = static_cast<const ST*>(a.q) + base;
        if (loader) {
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                const unsigned off = static_cast<unsigned>(min(tg * TPG + i, last) * HD + c4);
                pk[i] = *reinterpret_cast<const quad*>(kp + off);
                pg[i] = *reinterpret_cast<const quad*>(gp + off);
                if constexpr (MODE == 0) pq[i] = *reinterpret_cast<const quad*>(qp + off);
            }
            if (last < C - 1) {   // ragged last chunk: padded rows read as zero
#pragma unroll
                for (int i = 0; i < TPG; ++i)
                    if (tg * TPG + i > last) pk[i] = pg[i] = pq[i] = quad{};
            }
        }
        if (tid < C) {
            pb = static_cast<const ST*>(a.beta)[static_cast<size_t>(ts + min(tid, last)) * H + h];
            if (tid > last) pb = elem{};
        }
    };
    if (c_begin < c_end) fetch(c_begin);
    lds_barrier();

    for (int chunk = c_begin; chunk < c_end; ++chunk) {
        const long ts = t0 + static_cast<long>(chunk) * C;
        const int ntok = static_cast<int>(min(static_cast<long>(C), t1 - ts));

        // ============================================================ phase A: decay prefix, decayed operands
        float ktk[TPG][4];   // Ktil_m kept for Khat^T after the C x C products
        float enm[4];
        if (loader) {
            float gr[TPG][4];
#pragma unroll
            for (int i = 0; i < TPG; ++i)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch)
                    gr[i][ch] = R::get(pg[i], ch) * kLog2e + (i ? gr[i - 1][ch] : 0.f);   // log2 units
            float off[4], bm[4], bn[4];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                // inclusive prefix over the wave's 8 token groups (lanes 8 apart)
                float incl = gr[TPG - 1][ch];
#pragma unroll
                for (int dd = 8; dd < 64; dd <<= 1) {
                    const float y = __shfl_up(incl, dd);
                    incl += l >= dd ? y : 0.f;
                }
                off[ch] = incl - gr[TPG - 1][ch];
                bm[ch] = __shfl(incl, 24 + (l & 7));   // through token C/2 - 1
                bn[ch] = __shfl(incl, 56 + (l & 7));   // through the chunk's last token
                enm[ch] = exp2f_hw(bn[ch] - bm[ch]);
            }
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                const int r = tg * TPG + i;
                u16 kh[4], kl[4], th[4], tl[4], qh[4], ql[4];
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const float b = gr[i][ch] + off[ch] - bm[ch];   // b_r - b_m, log2 units
                    const float em = exp2f_hw(b);
                    const float ei = exp2f_hw(-b);
                    const float kv = R::get(pk[i], ch);
                    split2(kv * em, kh[ch], kl[ch]);
                    ktk[i][ch] = kv * ei;
                    split2(ktk[i][ch], th[ch], tl[ch]);
                    if constexpr (MODE == 0) split2(R::get(pq[i], ch) * em, qh[ch], ql[ch]);
                }
                const int idx = r * PK + kperm(c4);
                store4(&sm.kb[0][idx], kh);
                store4(&sm.kb[1][idx], kl);
                store4(&sm.kt[0][idx], th);
                store4(&sm.kt[1][idx], tl);
                if constexpr (MODE == 0) {
                    store4(&sm.qb[0][idx], qh);
                    store4(&sm.qb[1][idx], ql);
                }
            }
            if (tg == 0) {
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    sm.em[c4 + ch] = exp2f_hw(bm[ch]);
                    sm.gam[c4 + ch] = exp2f_hw(bn[ch]);
                }
            }
        }
        if (tid < C) sm.beta[tid] = IN::to_f32(pb);
        lds_barrier();

        // V of this chunk (used by the state pass) and the next chunk's k, q, log_alpha,
        // beta stream in while the C x C products and the solve run.
        elem pv[NRT][CT][4];
        if (!is_phi) {
            const int last = ntok - 1;
            const ST* vp = static_cast<const ST*>(a.v) + (static_cast<size_t>(ts) * H + h) * D + j0 + lr;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pv[rt][ct][e] = vp[static_cast<unsigned>(min(16 * rt + 4 * g4 + e, last) * HD + 16 * ct)];
            if (last < C - 1) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * rt + 4 * g4 + e > last) pv[rt][ct][e] = elem{};
            }
        }
        if (chunk + 1 < c_end) fetch(chunk + 1);

        // ============================================================ phase B: C x C products on MFMA
        // job < NTRI: tile of A = StrictTril(Diag(beta) Kbar_m Ktil_m^T); otherwise a tile of
        // P = Tril(Qbar_m Ktil_m^T).  Tiles are the lower 16x16 tiles of the C x C product.
        auto cxc_job = [&](int job) {
            const bool isP = job >= K::NTRI;
            const int tj = isP ? job - K::NTRI : job;
            int rt = 0;
            while ((rt + 1) * (rt + 2) / 2 <= tj) ++rt;
            const int ct = tj - rt * (rt + 1) / 2;
            const u16* ah_base = &sm.kb[0][0];
            const u16* al_base = &sm.kb[1][0];
            if constexpr (MODE == 0) {
                if (isP) { ah_base = &sm.qb[0][0]; al_base = &sm.qb[1][0]; }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ao = (16 * rt + lr) * PK + 32 * ks + 8 * g4;
                const int bo = (16 * ct + lr) * PK + 32 * ks + 8 * g4;
                acc = mfma3(frag(ah_base + ao), frag(al_base + ao), frag(&sm.kt[0][bo]), frag(&sm.kt[1][bo]), acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * rt + 4 * g4 + e, col = 16 * ct + lr;
                if (!isP) {
                    if (rt == ct) {
                        sm.a[rt][4 * g4 + e][lr] = col < row ? acc[e] * sm.beta[row] : 0.f;
                    } else {
                        u16 hi, lo;
                        split2(-acc[e] * sm.beta[row], hi, lo);
                        sm.aoff[0][row * K::AP + col] = hi;
                        sm.aoff[1][row * K::AP + col] = lo;
                    }
                } else if constexpr (MODE == 0) {
                    u16 hi, lo;
                    split2(col <= row ? acc[e] : 0.f, hi, lo);
                    sm.p[0][row * PT + kperm(col)] = hi;
                    sm.p[1][row * PT + kperm(col)] = lo;
                }
            }
        };
        // Without a separate Khat^T region, P must finish before Khat^T overwrites Ktil_m.
        constexpr int NJOB_B = (MODE == 0 && !K::KT_SEP) ? 2 * K::NTRI : K::NTRI;
#pragma unroll
        for (int jj = 0; jj < (NJOB_B + NW - 1) / NW; ++jj)
            if (w + jj * NW < NJOB_B) cxc_job(w + jj * NW);
        lds_barrier();

        // ============================================================ phase C/D: Khat^T, P, and T
        // Khat^T from registers (all element-phase threads)
        {
            u16* khi = K::KT_SEP ? &sm.kh[0][0] : &sm.kt[0][0];
            u16* klo = K::KT_SEP ? &sm.kh[K::KT_SEP ? 1 : 0][0] : &sm.kt[1][0];
            if (loader) {
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const int c = c4 + ch;
#pragma unroll
                    for (int gq = 0; gq < TPG / 4; ++gq) {
                        u16 hi[4], lo[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) split2(ktk[4 * gq + j][ch] * enm[ch], hi[j], lo[j]);
                        const int idx = c * PT + kperm(tg * TPG + 4 * gq);
                        store4(khi + idx, hi);
                        store4(klo + idx, lo);
                    }
                }
            }
        }
        if (w == 0 && l < 16 * K::NB) {
            // X_bb = (I + A_bb)^{-1} for each diagonal 16x16 block: one lane per (block,
            // column), right-looking substitution (critical path: one FMA per column).
            const int o0 = 16 * (l >> 4), j = l & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = r == j ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
                for (int r = i + 1; r < 16; ++r) x[r] -= sm.a[l >> 4][r][i] * x[i];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                u16 hi, lo;
                split2(x[r], hi, lo);
                sm.xd[0][(o0 + r) * K::XP + j] = hi;
                sm.xd[1][(o0 + r) * K::XP + j] = lo;
            }
        }
        lds_barrier();

        // ============================================================ phase E: state pass (per wave)
        // Y = Kbar S and Z = Qbar S.  The B operands are Diag(e^{b_m}) S (e^{b_m} completes
        // Kbar_m / Qbar_m to Kbar / Qbar), split per 32-deep step to keep registers low.
        f32x4 Y[NRT][CT], Z[NRT][CT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Y[rt][ct] = Z[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 sbh[CT], sbl[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 x0 = S[2 * ks][ct], x1 = S[2 * ks + 1][ct];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[e] *= sm.em[32 * ks + 4 * g4 + e];
                    x1[e] *= sm.em[32 * ks + 16 + 4 * g4 + e];
                }
                split_b(x0, x1, sbh[ct], sbl[ct]);
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int ao = (16 * rt + lr) * PK + 32 * ks + 8 * g4;
                const bf16x8 kh = frag(&sm.kb[0][ao]), kl = frag(&sm.kb[1][ao]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Y[rt][ct] = mfma3(kh, kl, sbh[ct], sbl[ct], Y[rt][ct]);
                if constexpr (MODE == 0) {
                    const bf16x8 qh = frag(&sm.qb[0][ao]), ql = frag(&sm.qb[1][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = mfma3(qh, ql, sbh[ct], sbl[ct], Z[rt][ct]);
                }
            }
        }
        // Unew = (I + A)^{-1} Diag(beta) (V - Kbar S), one 16-token block at a time:
        //   Unew_b = X_bb (beta_b (V - Kbar S)_b - sum_{k<b} A_bk Unew_k)
        f32x4 V[NRT][CT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    V[rt][ct][e] = is_phi ? 0.f : IN::to_f32(pv[rt][ct][e]);
        f32x4 U[NRT][CT];
        bf16x4 uh[NRT][CT], ul[NRT][CT];
#pragma unroll
        for (int b = 0; b < NRT; ++b) {
            f32x4 acc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[ct][e] = sm.beta[16 * b + 4 * g4 + e] * (V[b][ct][e] - Y[b][ct][e]);
#pragma unroll
            for (int k = 0; k < b; ++k) {
                const int ao = (16 * b + lr) * K::AP + 16 * k + 4 * g4;
                const bf16x4 ah = frag4(&sm.aoff[0][ao]), al = frag4(&sm.aoff[1][ao]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma3_16(ah, al, uh[k][ct], ul[k][ct], acc[ct]);
            }
            const int xo = (16 * b + lr) * K::XP + 4 * g4;
            const bf16x4 xh = frag4(&sm.xd[0][xo]), xl = frag4(&sm.xd[1][xo]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                bf16x4 bh, bl;
                split4(acc[ct], bh, bl);
                U[b][ct] = mfma3_16(xh, xl, bh, bl, f32x4{0.f, 0.f, 0.f, 0.f});
                split4(U[b][ct], uh[b][ct], ul[b][ct]);
            }
        }
        // 32-deep B operands of Unew: two stacked tiles in kperm order
        bf16x8 ubh[NKT][CT], ubl[NKT][CT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                ubh[kt][ct] = cat8(uh[2 * kt][ct], uh[2 * kt + 1][ct]);
                ubl[kt][ct] = cat8(ul[2 * kt][ct], ul[2 * kt + 1][ct]);
            }

        if constexpr (MODE == 0) {
            // O = Qbar S + P Unew
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int kt = 0; kt <= (rt >> 1); ++kt) {
                    const int ao = (16 * rt + lr) * PT + 32 * kt + 8 * g4;
                    const bf16x8 ph = frag(&sm.p[0][ao]), pl = frag(&sm.p[1][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = mfma3(ph, pl, ubh[kt][ct], ubl[kt][ct], Z[rt][ct]);
                }
            const bool full = ntok == C;   // uniform: only a sequence's last chunk can be ragged
            const size_t obase = (static_cast<size_t>(ts) * H + h) * D + j0 + lr;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * rt + 4 * g4 + e;
                        if (full || row < ntok)
                            store_out<OUT_BF16>(a.o, obase + static_cast<unsigned>(row * HD + 16 * ct), Z[rt][ct][e]);
                    }
        }
        // S <- Diag(gamma) S + Khat^T Unew
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[rt][ct][e] *= sm.gam[16 * rt + 4 * g4 + e];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const int ao = (16 * rt + lr) * PT + 32 * kt + 8 * g4;
                const u16* khi = K::KT_SEP ? &sm.kh[0][0] : &sm.kt[0][0];
                const u16* klo = K::KT_SEP ? &sm.kh[K::KT_SEP ? 1 : 0][0] : &sm.kt[1][0];
                const bf16x8 kh = frag(khi + ao), kl = frag(klo + ao);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[rt][ct] = mfma3(kh, kl, ubh[kt][ct], ubl[kt][ct], S[rt][ct]);
            }
        lds_barrier();
    }

    // ---------------------------------------------------------------- exit state
    float* dst = nullptr;
    if constexpr (MODE == 0) {
        if ((a.cu || s == a.G - 1) && a.S_final) dst = a.S_final + ubase;
    } else {
        dst = (is_phi ? a.phi : a.sloc) + (static_cast<size_t>(s) * a.NH + unit) * D * D;
    }
    if (dst) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(16 * rt + 4 * g4 + e) * D + j0 + 16 * ct + lr] = S[rt][ct][e];
    }
}

// Value of lane S of this lane's group of 4 lanes (DPP quad_perm broadcast).
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), S * 0x55, 0xf, 0xf, true));
}

// Right-looking elimination steps K, K-1, .., 1 of x^T (I + A) = e_i^T for a strictly lower
// triangular 16 x 16 A, with row i of x spread over the 4 lanes of a quad: this lane holds
// x_{4 jg + c}, c = 0..3, and col[k][c] = A_{k, 4 jg + c}.  x_K lives in lane K / 4 of the quad.
// A_{k j} = 0 for j >= k, so every lane updates its 4 entries at every step.
template <int K>
__device__ __forceinline__ void quad_lower_solve(float (&y)[4], const f32x4 (&col)[16]) {
    const float nk = -quad_bcast<K / 4>(y[K % 4]);
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = __builtin_fmaf(col[K][c], nk, y[c]);
    if constexpr (K > 1) quad_lower_solve<K - 1>(y, col);
}

// ------------------------------------------------------------------ pipelined kernel (C = 32)
// The operands of a chunk depend only on that chunk's inputs, never on the state, so
// they are built one chunk ahead.  Producer waves (one per SIMD) build chunk c+1's
// decayed operands, the A tiles and the diagonal-block inverses into one LDS buffer
// while consumer waves run chunk c's state pass out of the other.  The two sides are
// ordered by counters in LDS (signal_count / wait_count), so that one side's vector-ALU
// work runs beside the other side's MFMA work without workgroup barriers:
//
//   step   producer (chunk c+1)                      consumer (chunk c)
//   1      decay prefix, decayed K/Q splits, rho     Y = Kbar S, Z = Qbar S
//   2      A tiles, next inputs requested            Unew block recurrence, O; P tiles of c+1
//   3      diagonal-block inverses, Ktil_m^T         state update, O stores, state split
// ------------------------------------------------------------------ fused prologue helpers
constexpr int kFuseQK = 1, kFuseBeta = 2, kFuseDecay = 4;

__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + exp2f_hw(-x * kLog2e)); }

// log2(sigmoid(x)) = min(x, 0) log2(e) - log2(1 + 2^{-|x| log2(e)}), without overflow for any x
__device__ __forceinline__ float log2_sigmoid(float x) {
    return fminf(x, 0.f) * kLog2e - __builtin_amdgcn_logf(1.f + exp2f_hw(-fabsf(x) * kLog2e));
}

// Sum over the N (4 or 8) lanes of an aligned lane group (DPP butterflies; every lane gets the sum).
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
    static_assert(N == 4 || N == 8, "lane groups of 4 or 8");
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                   0xf, 0xf, true));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
    if constexpr (N == 8) x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    return x;
}

// 1 / (sum over producer waves of the partial sums of squares of token r + 1e-12)
template <int NPW, int C>
__device__ __forceinline__ float inv_sumsq(const float (&part)[NPW][C], int r) {
    float t = 1e-12f;
#pragma unroll
    for (int i = 0; i < NPW; ++i) t += part[i][r];
    return __builtin_amdgcn_rcpf(t);
}

// CT: 16-column tiles per consumer wave.  The output pass runs D/32 consumer waves of 32 state
// columns (CT = 2) on its own, or D/16 waves of 16 (CT = 1) in the launch it shares with the
// summary pass, which carries [S | Phi] (2D columns) on D/16 waves of 32: there both passes have
// D/32 producer and D/16 consumer waves, so they fit one workgroup size and register budget.
// NPW: producer waves.  Producer wave w owns QPW channel quads (4 QPW key channels) over all C
// tokens: lane l takes quad QPW w + l % QPW and TPG consecutive tokens of token group l / QPW, so
// the decay prefix over tokens stays inside the wave.  D/32 waves give 8 quads x 4 tokens per
// lane; D/16 waves 4 quads x 2 tokens.
template <int D, int MODE, int CT_ = 2, int NPW_ = D / 32>
struct PCfg {
    static constexpr int C = 32;
    static constexpr int NPW = NPW_;                               // producer waves
    static constexpr int QPW = D / (4 * NPW);                      // channel quads per producer wave
    static constexpr int TGN = 64 / QPW;                           // token groups per producer wave
    static constexpr int CT = CT_;
    static constexpr int NCW = (MODE == 0 ? D : 2 * D) / (16 * CT);   // consumer waves
    static constexpr int NW = NPW + NCW;
    static constexpr int NT = 64 * NW;
    static constexpr int WPE = (NW + 3) / 4;                       // waves per SIMD
    static constexpr int TPG = C / TGN;                            // tokens per producer thread
    static_assert(TPG == 2 || TPG == 4, "producer lanes hold 2 or 4 tokens");
    static constexpr int NRT = C / 16, RT = D / 16, KS = D / 32;
    // LDS planes carry no padding; 16-byte slots are XOR-swizzled per row instead, so that the
    // MFMA fragment reads (16 rows x 4 slots per instruction) and the producers' 8-byte writes
    // both avoid bank conflicts.  [token][channel] planes: rows of D channels, slot ^= row.
    __device__ static int tok(int row, int col) {
        return row * D + ((((col >> 3) ^ row) & (D / 8 - 1)) << 3) + (col & 7);
    }
    // [row][token] planes (C = 32 tokens, four 16-byte slots per row)
    __device__ static int swz(int row) { return (((row >> 2) ^ (row >> 4)) & 3) ^ ((row >> 1) & 2); }
    __device__ static int chm(int row, int col) { return row * C + ((((col >> 3) ^ swz(row)) & 3) << 3) + (col & 7); }
    static constexpr int AP = C + 4;                               // pitch of the off-diagonal A planes
    static constexpr int XP = 24;                                  // pitch of the diagonal-inverse planes
    static constexpr int NJOB = 3;                                 // lower 16x16 tiles of a 32 x 32 product
};

// VLDS: bf16 inputs, whose V tiles the producer stages in LDS for the consumers.
template <int D, int MODE, bool VLDS, int NPW_ = D / 32>
struct alignas(16) PBuf {
    using K = PCfg<D, MODE, 2, NPW_>;
    static constexpr int NQ = MODE == 0 ? 2 : 1, QE = MODE == 0 ? K::C * D : 8;
    static constexpr int PE = MODE == 0 ? K::C * K::C : 8;
    u16 kb[2][K::C * D];        // Kbar_m = K e^{b - b_m}     [token][kperm(channel)]
    u16 qb[NQ][QE];             // Qbar_m = Q e^{b - b_m}     [token][kperm(channel)]
    u16 kt[2][K::C * D];        // Ktil_m = K e^{b_m - b} [token][kperm(channel)], then
                                // Ktil_m^T                   [channel][kperm(token)]
    u16 aoff[2][K::C * K::AP];  // -A off the diagonal blocks  [token][token]
    u16 xd[2][K::C * K::XP];    // X_bb = (I + A_bb)^{-1}      [16 b + r][c]
    u16 p[NQ][PE];              // P = Tril(Qbar Ktil^T)       [token][kperm(token)]
    u16 vt[VLDS ? D * K::C : 8];    // V^T (bf16)              [column][token]
    float beta[K::C];
    float betae[K::C];          // fused prologue: beta_r / |k_r|^2
    float vs[K::C];             // fused prologue: |k_r| (scales V rows)
    float os[K::C];             // fused prologue: 1 / |q_r| (scales O rows)
    float nk[K::NPW][K::C];     // fused prologue: per producer wave, partial sums of k_r^2 and q_r^2
    float nq[K::NPW][K::C];
    float fv[K::C];             // scalar gate: e^{b_m - b_r} (scales V rows)
    float fo[K::C];             // scalar gate: e^{b_r - b_m} (scales O rows)
    float em[D];                // e^{b_m}
    float rho[D];               // e^{b_m} of the next chunk times e^{b_n - b_m} (1 after the last)
    float rn[D];                // e^{b_n - b_m}
    int tiny[K::NPW];           // scalar gate, per producer wave: some channel's rho is below
                                // 2^-100, so the consumers apply its two factors one after the other
    // Per-channel decay: the carried state X holds S~ = Diag(F) X, and F is folded into the
    // chunk's decayed operands instead of scaling the state every chunk.  When F would leave the
    // range the operands need, the producer resets it to 1 and the consumers rescale X by
    // f1 f2 f3 (three factors, each inside fp32 range) before this chunk.
    float f1[D], f2[D], f3[D];
    int renorm[K::NPW];         // per producer wave: some channel of the wave is rescaled
    float fin1[D], fin2[D];     // after the last chunk: S = Diag(fin1 fin2) X
};

template <int D, int MODE, bool VLDS, int NPW_ = D / 32>
struct PSmem {
    PBuf<D, MODE, VLDS, NPW_> buf[2];
    float a[2][16][20];         // diagonal 16x16 blocks of A (fp32), producer-private
    SyncCounters sync;
};

// One workgroup's share of a call: segment s, chunks [c_begin, c_end), of the (sequence n,
// head h) pair whose tokens are [t0, t1), with where its entry state comes from and where its
// result goes.  MODE 0 reads `entry` (nullptr: zero) and writes its exit state to `exit`
// (nullptr: none); MODE 1 writes S_loc to `exit` and Phi to `phi`.
struct Unit {
    int n, h, s, c_begin, c_end;
    long t0, t1;
    const float* entry;
    float* exit;
    float* phi;
};

// Segment table of a packed batch (int32, in the workspace), ranks r = 0..N-1 longest first:
//   [0]                 L, the segment length in chunks (segments 1.. of every sequence)
//   [4 + r]             the sequence of rank r
//   [4 + N + r]         chunks in its segment 0
//   [4 + 2N + r]        its segments after segment 0 (G_n - 1)
//   [4 + 3N + r], r<=N  exclusive prefix over ranks of its pass-1 workgroups, max(1, G_n - 1)
//   [4 + 4N + 1 + r]    exclusive prefix over ranks of its pass-2 workgroups, G_n - 1; also its
//                       first state slot (segment s >= 1 of rank r uses slot p2[r] + s - 1)
constexpr int kSegHdr = 4;
inline size_t seg_table_ints(int N) { return kSegHdr + 5 * static_cast<size_t>(N) + 2; }

// Largest r in [0, N) with pre[r] <= j, for a non-decreasing prefix array with pre[0] = 0 <= j
// < pre[N]: the rank whose range [pre[r], pre[r + 1]) holds item j.
__device__ __forceinline__ int seg_rank(const int32_t* pre, int N, int j) {
    int lo = 0, hi = N;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= j) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Equal-length batches: workgroup `block` of a launch whose first workgroup row is segment
// a.seg0; rows of N*H units.
template <int D, int C, int MODE>
__device__ __forceinline__ Unit unit_equal(const KernelArgs& a, int block) {
    Unit u;
    const int unit = block % a.NH;
    u.s = a.seg0 + block / a.NH;
    u.n = unit / a.H;
    u.h = unit % a.H;
    u.t0 = static_cast<long>(u.n) * a.T;
    u.t1 = u.t0 + a.T;
    u.c_begin = u.s == 0 ? 0 : a.cps0 + (u.s - 1) * a.cps;
    u.c_end = min(u.s == 0 ? a.cps0 : u.c_begin + a.cps, a.chunks);
    const size_t ub = static_cast<size_t>(unit) * D * D;
    u.entry = nullptr;
    u.exit = nullptr;
    u.phi = nullptr;
    if constexpr (MODE == 0) {
        if (u.s == 0) u.entry = a.S0 ? a.S0 + ub : nullptr;
        else u.entry = a.se + (static_cast<size_t>(u.s - 1) * a.NH + unit) * D * D;
        if (u.s == a.G - 1 && a.S_final) u.exit = a.S_final + ub;
        else if (u.s == 0 && a.split0) u.exit = a.se + ub;   // segment 1's entry state
    } else {
        const size_t sb = (static_cast<size_t>(u.s) * a.NH + unit) * D * D;
        u.exit = a.sloc + sb;
        u.phi = a.phi + sb;
    }
    return u;
}

// Packed sequences, one pass: workgroup `block` runs the whole of one (sequence, head), the
// sequences taken longest first.
template <int D, int C>
__device__ __forceinline__ Unit unit_packed(const KernelArgs& a, int block) {
    Unit u;
    u.n = a.order[block / a.H];
    u.h = block % a.H;
    u.s = 0;
    u.t0 = a.cu[u.n];
    u.t1 = a.cu[u.n + 1];
    u.c_begin = 0;
    u.c_end = static_cast<int>((u.t1 - u.t0 + C - 1) / C);
    const size_t ub = (static_cast<size_t>(u.n) * a.H + u.h) * D * D;
    u.entry = a.S0 ? a.S0 + ub : nullptr;
    u.exit = a.S_final ? a.S_final + ub : nullptr;
    u.phi = nullptr;
    return u;
}

// Packed sequences, segmented: item j = block / H of head h = block % H.  Pass 1 (pass2 false)
// holds, per rank, segment 0's output pass and then the summaries of segments 1..G_n-2; pass 2
// the output passes of segments 1..G_n-1.  Returns the item's mode (0 output, 1 summary), or -1
// for a workgroup past the last item.
template <int D, int C>
__device__ __forceinline__ int unit_segmented(const KernelArgs& a, int block, bool pass2, Unit& u) {
    const int32_t* tab = a.seg;
    const int N = a.NH / a.H;
    const int32_t* p1 = tab + kSegHdr + 3 * N;
    const int32_t* p2 = p1 + N + 1;
    const int32_t* pre = pass2 ? p2 : p1;
    const int j = block / a.H;
    if (j >= pre[N]) return -1;
    const int r = seg_rank(pre, N, j);
    const int L = tab[0], cps0 = tab[kSegHdr + N + r], more = tab[kSegHdr + 2 * N + r];
    u.n = tab[kSegHdr + r];
    u.h = block % a.H;
    u.t0 = a.cu[u.n];
    u.t1 = a.cu[u.n + 1];
    const int nc = static_cast<int>((u.t1 - u.t0 + C - 1) / C);
    u.s = j - pre[r] + (pass2 ? 1 : 0);
    u.c_begin = u.s == 0 ? 0 : cps0 + (u.s - 1) * L;
    u.c_end = u.s == 0 ? cps0 : min(u.c_begin + L, nc);
    const size_t ub = (static_cast<size_t>(u.n) * a.H + u.h) * D * D;
    // state slot of segment s (>= 1): the entry state of segment s, or the summary of segment s
    const size_t slot = (static_cast<size_t>(p2[r] + u.s - 1) * a.H + u.h) * D * D;
    u.entry = nullptr;
    u.exit = nullptr;
    u.phi = nullptr;
    if (u.s == 0) {
        u.entry = a.S0 ? a.S0 + ub : nullptr;
        if (more == 0) u.exit = a.S_final ? a.S_final + ub : nullptr;
        else u.exit = a.se + (static_cast<size_t>(p2[r]) * a.H + u.h) * D * D;   // segment 1's entry
        return 0;
    }
    if (!pass2) {
        u.exit = a.sloc + slot;
        u.phi = a.phi + slot;
        return 1;
    }
    u.entry = a.se + slot;
    if (u.s == more) u.exit = a.S_final ? a.S_final + ub : nullptr;
    return 0;
}

// SG (scalar gate): log_alpha is one value per (token, head), [B, T, H] -- the gated delta
// rule of Gated DeltaNet.  With f_r = e^{b_r - b_m} a scalar per token, the decay factors move
// off the contractions: A = StrictTril(Diag(beta) K K^T) and P = Tril(Q K^T) carry no decay,
// and with U' = Diag(1/f) Unew, S~ = e^{b_m} S,
//     U' = (I + A)^{-1} Diag(beta) (Diag(1/f) V - K S~),   O = Diag(f) (Q S~ + P U'),
//     S~ <- rho (S~ + K^T U'),   rho = e^{b_m'} e^{b_n - b_m} (a scalar).
// With bf16 inputs K and Q are exact MFMA operands, so every product that has them on one side
// needs two MFMAs (or one) instead of three, and the producer has no per-element decay.
//
// FUSE (fused prologue / epilogue, flags in KernelArgs): q and k arrive unnormalised, beta and
// log_alpha as logits, and o may be gated.  The L2 norms enter as per-token scalars only: with
// n_r = |k_r| and m_r = |q_r| (over the key channels, plus 1e-12 under the root),
//     A = Diag(beta / n^2) StrictTril(Kbar Ktil^T),  U' = T (Diag(n) V - Kbar S),
//     O = Diag(1/m) (Qbar S + P U'),  S <- Diag(gamma) S + Khat^T U'
// with the unnormalised Kbar, Ktil, Khat, Qbar, P (U' = Diag(1/n) Unew of the normalised keys),
// so the producer only adds per-token sums of squares to its decay phase.
template <int D, typename IN, bool OUT_BF16, int MODE, bool SG, bool FUSE, int CT_, int NPW_ = D / 32>
__device__ __forceinline__ void pipe_body(const KernelArgs& a,
                                          PSmem<D, MODE, std::is_same<IN, BF16>::value, NPW_>& sm,
                                          const Unit& u) {
    using K = PCfg<D, MODE, CT_, NPW_>;
    constexpr int C = K::C, NPW = K::NPW, CT = K::CT, TPG = K::TPG, QPW = K::QPW, TGN = K::TGN;
    constexpr int NRT = K::NRT, RT = K::RT, KS = K::KS;
    using ST = typename IN::storage;
    using R = Raw<IN>;
    using quad = typename R::quad;
    using elem = typename R::elem;
    constexpr bool VLDS = std::is_same<IN, BF16>::value;
    // scalar gate with bf16 inputs: K and Q are exact bf16 MFMA operands (no low parts)
    constexpr bool EXACT = SG && std::is_same<IN, BF16>::value;
    using Buf = PBuf<D, MODE, VLDS, NPW_>;

    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, lr = l & 15;
    const int wl = a.wait_limit;
    // wave index in a scalar register: the producer / consumer split below is a uniform
    // branch, so each side runs its own loop with its own registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    const bool producer = w < NPW;
    // The last two producer waves invert the two diagonal blocks (one each) in phase 3.
    const bool solver = w >= NPW - 2;

    // ---------------------------------------------------------------- work unit
    const int h = u.h, c_begin = u.c_begin, c_end = u.c_end;
    const long t0 = u.t0, t1 = u.t1;
    const int HD = H * D;   // elements between consecutive tokens of one head

    // consumer identity: 16 CT state columns starting at j0 (of S, or of Phi in the summary pass)
    const int ci = producer ? 0 : w - NPW;
    const bool is_phi = MODE == 1 && ci >= D / (16 * CT);
    const int j0 = 16 * CT * (ci % (D / (16 * CT)));
    // producer identity: channel quad cq, token group tg (TPG tokens)
    const int cq = QPW * w + (l % QPW), tg = l / QPW, c4 = 4 * cq;

    if constexpr (MODE == 0) {
        // P's strictly-upper 16x16 tile inside the 32-deep step is read but never written.
        for (int i = tid; i < 2 * 2 * C * C; i += K::NT) {
            const int b = i / (2 * C * C), r = i % (2 * C * C);
            sm.buf[b].p[r / (C * C)][r % (C * C)] = 0;
        }
    }
    if (tid == 0) sm.sync = SyncCounters{0, 0, 0, 0, {0, 0}, 0};
    lds_barrier();
    int* const broken = &sm.sync.broken;

    // ================================================================ producer state
    quad pk[TPG], pq[TPG], pg[TPG], pvq[TPG];
    elem pgs[TPG];   // scalar gate: log_alpha of this lane's tokens
    elem pb = 0;
    uint2 kth[TPG], ktl[TPG];   // split Ktil_m words, kept from phase 1 for Ktil_m^T in phase 3
    float enm[4] = {1.f, 1.f, 1.f, 1.f};   // e^{b_n - b_m} of the chunk last produced
    // per-channel decay: log2 F of the chunk last produced and log2 e^{b_n - b_m} of it
    float lf[4] = {0.f, 0.f, 0.f, 0.f}, lrn[4] = {0.f, 0.f, 0.f, 0.f};
    // part 0: k and log_alpha; part 1: q, v and beta; -1: everything.  The two parts are requested
    // in different phases so the chip's memory requests are spread over the chunk loop.
    auto fetch = [&](int chunk, int part) {
        const long ts = t0 + static_cast<long>(chunk) * C;
        const int last = static_cast<int>(min(static_cast<long>(C), t1 - ts)) - 1;
        const size_t base = (static_cast<size_t>(ts) * H + h) * D;   // uniform
        // uniform bases plus a 32-bit byte offset per lane (scalar base + vector offset addressing)
        const char* kp = reinterpret_cast<const char*>(static_cast<const ST*>(a.k) + base);
        const char* gp = reinterpret_cast<const char*>(static_cast<const ST*>(a.g) + base);
        const char* qp = reinterpret_cast<const char*>(static_cast<const ST*>(a.q) + base);
        const char* vp = reinterpret_cast<const char*>(static_cast<const ST*>(a.v) + base);
        // Rows past a ragged end load a valid row here and are zeroed where they are used:
        // touching a loaded value now would make the wave wait for the loads.
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            const unsigned off = static_cast<unsigned>(min(tg * TPG + i, last) * HD + c4) * sizeof(ST);
            if (part != 1) {
                if constexpr (SG)
                    pgs[i] = static_cast<const ST*>(a.g)[static_cast<size_t>(ts + min(tg * TPG + i, last)) * H + h];
                else
                    pg[i] = *reinterpret_cast<const quad*>(gp + off);
                pk[i] = *reinterpret_cast<const quad*>(kp + off);
            }
            if (part != 0) {
                if constexpr (MODE == 0) pq[i] = *reinterpret_cast<const quad*>(qp + off);
                if constexpr (VLDS) pvq[i] = *reinterpret_cast<const quad*>(vp + off);
            }
        }
        if (part != 0 && tid < C) pb = static_cast<const ST*>(a.beta)[static_cast<size_t>(ts + min(tid, last)) * H + h];
    };

    // V^T staged in LDS for the consumers (bf16 inputs)
    auto stage_v = [&](Buf& B) {
        if constexpr (VLDS) {
            // V^T: channel ch of token i is the low (even ch) or high (odd ch) half of word ch / 2
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const unsigned sel = (ch & 1) ? 0x07060302u : 0x05040100u;
                auto word = [&](int t) { return ch < 2 ? pvq[t].x : pvq[t].y; };
                if constexpr (TPG == 4) {
                    *reinterpret_cast<uint2*>(&B.vt[K::chm(c4 + ch, tg * TPG)]) =
                        uint2{__builtin_amdgcn_perm(word(1), word(0), sel), __builtin_amdgcn_perm(word(3), word(2), sel)};
                } else {
                    *reinterpret_cast<uint32_t*>(&B.vt[K::chm(c4 + ch, tg * TPG)]) =
                        __builtin_amdgcn_perm(word(1), word(0), sel);
                }
            }
        }
    };

    // phase 1: decay prefix (in log2 units) and the decayed, split K / Q planes.  With
    // the previous chunk's buffer `prev`, also that chunk's state factor rho.
    // fused prologue: per-token sums of squares of k and q over this wave's 32 channels (8 lanes
    // share a token group), one partial per producer wave
    auto fused_sumsq = [&](Buf& B) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                sk += R::get(pk[i], ch) * R::get(pk[i], ch);
                if constexpr (MODE == 0) sq += R::get(pq[i], ch) * R::get(pq[i], ch);
            }
            sk = sum_lanes<QPW>(sk);
            if constexpr (MODE == 0) sq = sum_lanes<QPW>(sq);
            if ((l % QPW) == 0) {
                B.nk[w][tg * TPG + i] = sk;
                if constexpr (MODE == 0) B.nq[w][tg * TPG + i] = sq;
            }
        }
    };
    // beta of the chunk's tokens (sigmoid of the logits with the fused prologue; padded rows 0)
    auto stage_beta = [&](Buf& B, int last) __attribute__((always_inline)) {
        if (tid < C) {
            float bt = IN::to_f32(pb);
            if constexpr (FUSE) {
                if ((a.fuse_flags & kFuseBeta) && tid <= last) bt = sigmoid_f(bt);
            }
            B.beta[tid] = bt;
        }
    };
    auto produce_decay = [&](Buf& B, int chunk, Buf* prev) {
        const long ts = t0 + static_cast<long>(chunk) * C;
        const int last = static_cast<int>(min(static_cast<long>(C), t1 - ts)) - 1;
        if constexpr (SG) {
            // scalar gate: decay prefix of the chunk's tokens, the per-token factors f and 1/f,
            // and K, Q as they are (split into hi / lo only for fp32 inputs)
            if (last < C - 1) {
#pragma unroll
                for (int i = 0; i < TPG; ++i)
                    if (tg * TPG + i > last) {
                        pk[i] = pq[i] = quad{};
                        pgs[i] = elem{};
                    }
                if (tid > last) pb = elem{};
            }
            float gs[TPG];
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                float g2 = IN::to_f32(pgs[i]) * kLog2e;   // log2 of this token's decay
                if constexpr (FUSE) {
                    if ((a.fuse_flags & kFuseDecay) && tg * TPG + i <= last)
                        g2 = log2_sigmoid(IN::to_f32(pgs[i]) + a.decay_bias) / a.decay_scale;
                }
                gs[i] = g2 + (i ? gs[i - 1] : 0.f);
            }
            if constexpr (FUSE) fused_sumsq(B);
            float incl = gs[TPG - 1];
#pragma unroll
            for (int dd = QPW; dd < 64; dd <<= 1) {
                const float y = __shfl_up(incl, dd);
                incl += l >= dd ? y : 0.f;
            }
            const float bm = __shfl(incl, (TGN / 2 - 1) * QPW), bn = __shfl(incl, (TGN - 1) * QPW);
            const float off = incl - gs[TPG - 1] - bm;   // b_r - b_m = gs + off
            if (tg == 0) {
                const float em = exp2f_hw(bm);
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    B.em[c4 + ch] = em;
                    if (prev) {
                        prev->rho[c4 + ch] = em * enm[0];
                        prev->rn[c4 + ch] = enm[0];
                    }
                }
                if (prev && l == 0) prev->tiny[w] = em * enm[0] < 0x1p-100f;
            }
            const float en = exp2f_hw(bn - bm);
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) enm[ch] = en;
            if (w == 0 && (l % QPW) == 0) {
#pragma unroll
                for (int i = 0; i < TPG; ++i) {
                    const float b = gs[i] + off;
                    B.fo[tg * TPG + i] = exp2f_hw(b);
                    B.fv[tg * TPG + i] = exp2f_hw(-b);
                }
            }
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                const int idx = K::tok(tg * TPG + i, kperm(c4));
                if constexpr (EXACT) {
                    *reinterpret_cast<quad*>(&B.kb[0][idx]) = pk[i];
                    kth[i] = pk[i];
                    if constexpr (MODE == 0) *reinterpret_cast<quad*>(&B.qb[0][idx]) = pq[i];
                } else {
                    uint2 hi, lo;
                    split_quad(R::get(pk[i], 0), R::get(pk[i], 1), R::get(pk[i], 2), R::get(pk[i], 3), kth[i], ktl[i]);
                    *reinterpret_cast<uint2*>(&B.kb[0][idx]) = kth[i];
                    *reinterpret_cast<uint2*>(&B.kb[1][idx]) = ktl[i];
                    if constexpr (MODE == 0) {
                        split_quad(R::get(pq[i], 0), R::get(pq[i], 1), R::get(pq[i], 2), R::get(pq[i], 3), hi, lo);
                        *reinterpret_cast<uint2*>(&B.qb[0][idx]) = hi;
                        *reinterpret_cast<uint2*>(&B.qb[1][idx]) = lo;
                    }
                }
            }
            stage_v(B);
            stage_beta(B, last);
            return;
        }
        if (last < C - 1) {   // ragged last chunk: padded rows read as zero
#pragma unroll
            for (int i = 0; i < TPG; ++i)
                if (tg * TPG + i > last) pk[i] = pg[i] = pq[i] = quad{};
            if (tid > last) pb = elem{};
        }
        float gr[TPG][4];
#pragma unroll
        for (int i = 0; i < TPG; ++i)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                float g2 = R::get(pg[i], ch) * kLog2e;   // log2 of this token's decay
                if constexpr (FUSE) {
                    if ((a.fuse_flags & kFuseDecay) && tg * TPG + i <= last)
                        g2 = log2_sigmoid(R::get(pg[i], ch) + a.decay_bias) / a.decay_scale;
                }
                gr[i][ch] = g2 + (i ? gr[i - 1][ch] : 0.f);
            }
        if constexpr (FUSE) fused_sumsq(B);
        float off[4], bm[4], bn[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            // inclusive prefix over the wave's TGN token groups (lanes QPW apart)
            float incl = gr[TPG - 1][ch];
#pragma unroll
            for (int dd = QPW; dd < 64; dd <<= 1) {
                const float y = __shfl_up(incl, dd);
                incl += l >= dd ? y : 0.f;
            }
            off[ch] = incl - gr[TPG - 1][ch];
            bm[ch] = __shfl(incl, (TGN / 2 - 1) * QPW + (l % QPW));   // through token C/2 - 1
            bn[ch] = __shfl(incl, (TGN - 1) * QPW + (l % QPW));       // through the chunk's last token
            off[ch] -= bm[ch];                     // b_r - b_m = gr + off
        }
        // F of this chunk (log2): the previous chunk's F times its rho = e^{b_m} e^{b_n - b_m} of the
        // previous chunk and this one.  The decayed operands take exponents (b_r - b_m) + log2 F
        // (K, Q) and -(b_r - b_m) - log2 F (Ktil), kept within +-100 (the carried state X = S~ / F
        // then stays below 2^100 |S~|); b_r - b_m spans [b_n - b_m, -b_m] and log2 F <= 0, so F is
        // reset to 1 (and X rescaled) when log2 F < -100 + |b_n - b_m|.  The first chunk starts from
        // F = 1 (the consumers scale the entry state by e^{b_m}).
        bool rescale = false;
        float f1v[4] = {1.f, 1.f, 1.f, 1.f}, f2v[4] = {1.f, 1.f, 1.f, 1.f}, f3v[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            float lnew = 0.f;
            if (prev) {
                lnew = lf[ch] + lrn[ch] + bm[ch];
                if (lnew < -100.f + fabsf(bn[ch] - bm[ch])) {
                    f1v[ch] = exp2f_hw(lf[ch]);
                    f2v[ch] = exp2f_hw(lrn[ch]);
                    f3v[ch] = exp2f_hw(bm[ch]);
                    rescale = true;
                    lnew = 0.f;
                }
            }
            lf[ch] = lnew;
            lrn[ch] = bn[ch] - bm[ch];
            off[ch] += lnew;                       // (b_r - b_m) + log2 F = gr + off
        }
        // every lane holds its channels' values; lanes with tg == 0 cover the wave's channels once
        const bool any_rescale = __builtin_amdgcn_ballot_w64(rescale) != 0;
        if (tg == 0) {   // every wave writes its factors (1 where unchanged): any wave's reset rescales all rows
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                B.em[c4 + ch] = exp2f_hw(bm[ch]);
                B.f1[c4 + ch] = f1v[ch];
                B.f2[c4 + ch] = f2v[ch];
                B.f3[c4 + ch] = f3v[ch];
            }
            if (l == 0) B.renorm[w] = any_rescale;
        }
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            const int r = tg * TPG + i;
            float kb[4], kt[4], qb[4];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const float b = gr[i][ch] + off[ch];   // b_r - b_m
                const float em = exp2f_hw(b);
                const float ei = exp2f_hw(-b);
                const float kv = R::get(pk[i], ch);
                kb[ch] = kv * em;
                kt[ch] = kv * ei;
                if constexpr (MODE == 0) qb[ch] = R::get(pq[i], ch) * em;
            }
            const int idx = K::tok(r, kperm(c4));
            uint2 hi, lo;
            split_quad(kb[0], kb[1], kb[2], kb[3], hi, lo);
            *reinterpret_cast<uint2*>(&B.kb[0][idx]) = hi;
            *reinterpret_cast<uint2*>(&B.kb[1][idx]) = lo;
            split_quad(kt[0], kt[1], kt[2], kt[3], kth[i], ktl[i]);
            *reinterpret_cast<uint2*>(&B.kt[0][idx]) = kth[i];
            *reinterpret_cast<uint2*>(&B.kt[1][idx]) = ktl[i];
            if constexpr (MODE == 0) {
                split_quad(qb[0], qb[1], qb[2], qb[3], hi, lo);
                *reinterpret_cast<uint2*>(&B.qb[0][idx]) = hi;
                *reinterpret_cast<uint2*>(&B.qb[1][idx]) = lo;
            }
        }
        stage_v(B);
        stage_beta(B, last);
    };

    // Tiles of A^T and P^T: tile (rt, ct), ct <= rt, is Ktil_m[ct] against Kbar_m[rt] (or
    // Qbar_m[rt]); the accumulator of lane (g4, lr) then holds row 16 rt + lr, columns
    // 16 ct + 4 g4 + e, so each lane stores 4 consecutive entries of one row.  Tile index
    // job: 0 -> (1, 0), 1 -> (0, 0), 2 -> (1, 1).
    auto tile_of = [](int job, int& rt, int& ct) {
        rt = job == 1 ? 0 : 1;
        ct = job == 2 ? 1 : 0;
    };
    // phase 2 (producer): the three A tiles
    auto produce_products = [&](Buf& B) {
        for (int job = w; job < 3; job += NPW) {
            int rt, ct;
            tile_of(job, rt, ct);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ao = K::tok(16 * ct + lr, 32 * ks + 8 * g4);
                const int bo = K::tok(16 * rt + lr, 32 * ks + 8 * g4);
                if constexpr (EXACT)
                    acc = mfma(frag(&B.kb[0][ao]), frag(&B.kb[0][bo]), acc);
                else if constexpr (SG)
                    acc = mfma3(frag(&B.kb[0][ao]), frag(&B.kb[1][ao]), frag(&B.kb[0][bo]), frag(&B.kb[1][bo]), acc);
                else
                    acc = mfma3(frag(&B.kt[0][ao]), frag(&B.kt[1][ao]), frag(&B.kb[0][bo]), frag(&B.kb[1][bo]), acc);
            }
            const int row = 16 * rt + lr;
            float br = B.beta[row];
            if constexpr (FUSE) {
                if (a.fuse_flags & kFuseQK) br *= inv_sumsq(B.nk, row);
            }
            if (rt == ct) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = 4 * g4 + e < lr ? acc[e] * br : 0.f;
                *reinterpret_cast<f32x4*>(&sm.a[rt][lr][4 * g4]) = v;
            } else {
                uint2 hi, lo;
                split_quad(-acc[0] * br, -acc[1] * br, -acc[2] * br, -acc[3] * br, hi, lo);
                const int idx = row * K::AP + 16 * ct + 4 * g4;
                *reinterpret_cast<uint2*>(&B.aoff[0][idx]) = hi;
                *reinterpret_cast<uint2*>(&B.aoff[1][idx]) = lo;
            }
        }
    };
    // phase 2 (producer, fused prologue): per-token scalars for the consumers
    auto produce_token_scales = [&](Buf& B) {
        if constexpr (FUSE) {
            if (w == NPW - 1 && l < C) {
                const bool qk = a.fuse_flags & kFuseQK;
                const float ik = qk ? inv_sumsq(B.nk, l) : 1.f;
                B.betae[l] = B.beta[l] * ik;
                B.vs[l] = qk ? __builtin_amdgcn_rsqf(ik) : 1.f;
                if constexpr (MODE == 0) B.os[l] = qk ? __builtin_amdgcn_sqrtf(inv_sumsq(B.nq, l)) : 1.f;
            }
        }
    };
    // consumers, output pass: the three P tiles of the chunk the producers are building, once
    // its planes are written (phase 1) and before phase 3 turns Ktil_m into Ktil_m^T
    auto consume_ptiles = [&](Buf& B) {
        if constexpr (MODE == 0) {
            for (int job = ci; job < 3; job += K::NCW) {
                int rt, ct;
                tile_of(job, rt, ct);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int ao = K::tok(16 * ct + lr, 32 * ks + 8 * g4);
                    const int bo = K::tok(16 * rt + lr, 32 * ks + 8 * g4);
                    if constexpr (EXACT)
                        acc = mfma(frag(&B.kb[0][ao]), frag(&B.qb[0][bo]), acc);
                    else if constexpr (SG)
                        acc = mfma3(frag(&B.kb[0][ao]), frag(&B.kb[1][ao]), frag(&B.qb[0][bo]), frag(&B.qb[1][bo]), acc);
                    else
                        acc = mfma3(frag(&B.kt[0][ao]), frag(&B.kt[1][ao]), frag(&B.qb[0][bo]), frag(&B.qb[1][bo]), acc);
                }
                f32x4 pv4;
#pragma unroll
                for (int e = 0; e < 4; ++e) pv4[e] = (rt > ct || 4 * g4 + e <= lr) ? acc[e] : 0.f;
                uint2 hi, lo;
                split_quad(pv4[0], pv4[1], pv4[2], pv4[3], hi, lo);
                const int idx = K::chm(16 * rt + lr, 8 * g4 + 4 * ct);   // kperm(16 ct + 4 g4 + e) = 8 g4 + 4 ct + e
                *reinterpret_cast<uint2*>(&B.p[0][idx]) = hi;
                *reinterpret_cast<uint2*>(&B.p[1][idx]) = lo;
            }
        }
    };
    // phase 3: Ktil_m^T over Ktil_m (read by the products), regrouped from the split words
    // of phase 1
    auto produce_transpose = [&](Buf& B) {
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const int c = c4 + ch;
            // channel ch of token i sits in the low (even ch) or high (odd ch) half of word ch / 2
            const unsigned sel = (ch & 1) ? 0x07060302u : 0x05040100u;
            auto hw = [&](int t) { return (ch < 2) ? kth[t].x : kth[t].y; };
            auto lw = [&](int t) { return (ch < 2) ? ktl[t].x : ktl[t].y; };
            const int idx = K::chm(c, kperm(tg * TPG));
            if constexpr (TPG == 4) {
                *reinterpret_cast<uint2*>(&B.kt[0][idx]) =
                    uint2{__builtin_amdgcn_perm(hw(1), hw(0), sel), __builtin_amdgcn_perm(hw(3), hw(2), sel)};
                if constexpr (!EXACT)
                    *reinterpret_cast<uint2*>(&B.kt[1][idx]) =
                        uint2{__builtin_amdgcn_perm(lw(1), lw(0), sel), __builtin_amdgcn_perm(lw(3), lw(2), sel)};
            } else {
                *reinterpret_cast<uint32_t*>(&B.kt[0][idx]) = __builtin_amdgcn_perm(hw(1), hw(0), sel);
                if constexpr (!EXACT) *reinterpret_cast<uint32_t*>(&B.kt[1][idx]) = __builtin_amdgcn_perm(lw(1), lw(0), sel);
            }
        }
    };
    // phase 3: X_bb = (I + A_bb)^{-1} on the two solver waves
    auto produce_inverse = [&](Buf& B) {
        if (solver) {
            // Block blk: lane (i, jg) = (l / 4, l % 4) solves columns 4 jg .. 4 jg + 3 of row i
            // of X_bb = (I + A_bb)^{-1} (x^T (I + A) = e_i^T).
            const int blk = w - (NPW - 2), jg = l & 3;
            int i = l >> 2;
            asm volatile("" : "+v"(i));   // keep the unit-vector set-up inside the loop
            f32x4 col[16];
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) col[kk] = *reinterpret_cast<const f32x4*>(&sm.a[blk][kk][4 * jg]);
            float y[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) y[c] = 4 * jg + c == i ? 1.f : 0.f;
            quad_lower_solve<15>(y, col);
            uint2 hi, lo;
            split_quad(y[0], y[1], y[2], y[3], hi, lo);
            const int idx = (16 * blk + i) * K::XP + 4 * jg;
            *reinterpret_cast<uint2*>(&B.xd[0][idx]) = hi;
            *reinterpret_cast<uint2*>(&B.xd[1][idx]) = lo;
        }
    };

    // ================================================================ consumer state
    f32x4 S[RT][CT];
    if (!producer) {
        const float* src = MODE == 0 ? u.entry : nullptr;
        if (src) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[rt][ct][e] = src[(16 * rt + 4 * g4 + e) * D + j0 + 16 * ct + lr];
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[rt][ct][e] = (is_phi && 16 * rt + 4 * g4 + e == j0 + 16 * ct + lr) ? 1.f : 0.f;
        }
    }
    f32x4 Y[NRT][CT], Z[NRT][CT];
    elem pv[NRT][CT][4];
    bf16x8 ubh[CT], ubl[CT];
    // The consumers carry St = Diag(e^{b_m}) S, with b_m the midpoint decay of the chunk about to
    // be processed: then Kbar S = Kbar_m St and Qbar S = Qbar_m St, and since
    // gamma = e^{b_m} e^{b_n - b_m} and Khat = Ktil_m e^{b_n - b_m}, the chunk update is
    //   St <- Diag(rho) (St + Ktil_m^T Unew),  rho = e^{b_m'} e^{b_n - b_m}
    // with b_m' the next chunk's midpoint decay (rho = e^{b_n - b_m} after the last chunk, which
    // leaves S itself).  The output pass splits St for the coming chunk right after the update,
    // so step 1 holds only MFMA work beside the producer's vector-ALU work; the summary pass,
    // with twice the columns per compute unit, has no registers to spare for it.
    constexpr bool PRESPLIT = MODE == 0 && NPW == D / 32;
    bf16x8 sph[PRESPLIT ? KS : 1][CT], spl[PRESPLIT ? KS : 1][CT];
    auto split_state = [&]() {
        if constexpr (PRESPLIT) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) split_b(S[2 * ks][ct], S[2 * ks + 1][ct], sph[ks][ct], spl[ks][ct]);
        }
    };

    // consumer step 1: V loads, Y = Kbar_m St and Z = Qbar_m St.
    auto consume_project = [&](const Buf& B, int chunk) {
        const long ts = t0 + static_cast<long>(chunk) * C;
        const int last = static_cast<int>(min(static_cast<long>(C), t1 - ts)) - 1;
        if (!VLDS && !is_phi) {
            const ST* vp = static_cast<const ST*>(a.v) + (static_cast<size_t>(ts) * H + h) * D + j0 + lr;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pv[rt][ct][e] = vp[static_cast<unsigned>(min(16 * rt + 4 * g4 + e, last) * HD + 16 * ct)];
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Y[rt][ct] = Z[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 sbh[CT], sbl[CT];
            if constexpr (PRESPLIT) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    sbh[ct] = sph[ks][ct];
                    sbl[ct] = spl[ks][ct];
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) split_b(S[2 * ks][ct], S[2 * ks + 1][ct], sbh[ct], sbl[ct]);
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int ao = K::tok(16 * rt + lr, 32 * ks + 8 * g4);
                if constexpr (EXACT) {
                    const bf16x8 kh = frag(&B.kb[0][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[rt][ct] = mfma(kh, sbh[ct], mfma(kh, sbl[ct], Y[rt][ct]));
                } else {
                    const bf16x8 kh = frag(&B.kb[0][ao]), kl = frag(&B.kb[1][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[rt][ct] = mfma3(kh, kl, sbh[ct], sbl[ct], Y[rt][ct]);
                }
                if constexpr (MODE == 0) {
                    // Z^T = St^T Qbar_m^T: the split state serves as the A operand,
                    // so lane (g4, lr) ends up with token 16 rt + lr, columns 16 ct + 4 g4 + e
                    if constexpr (EXACT) {
                        const bf16x8 qh = frag(&B.qb[0][ao]);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = mfma(sbh[ct], qh, mfma(sbl[ct], qh, Z[rt][ct]));
                    } else {
                        const bf16x8 qh = frag(&B.qb[0][ao]), ql = frag(&B.qb[1][ao]);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = mfma3(sbh[ct], sbl[ct], qh, ql, Z[rt][ct]);
                    }
                }
            }
        }
        // Y <- V - Kbar S (frees the raw V registers before the solve)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 vv = {0.f, 0.f, 0.f, 0.f};
                if constexpr (VLDS) {
                    if (!is_phi) {
                        const uint2 w = *reinterpret_cast<const uint2*>(&B.vt[K::chm(j0 + 16 * ct + lr, 16 * rt + 4 * g4)]);
                        vv = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
                    }
                } else if (!is_phi) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) vv[e] = IN::to_f32(pv[rt][ct][e]);
                }
                if constexpr (SG) {
                    if (!is_phi) vv *= *reinterpret_cast<const f32x4*>(&B.fv[16 * rt + 4 * g4]);
                }
                if constexpr (FUSE) {
                    if (!is_phi) vv *= *reinterpret_cast<const f32x4*>(&B.vs[16 * rt + 4 * g4]);
                }
                Y[rt][ct] = vv - Y[rt][ct];
            }
    };

    // consumer step 2: Unew = (I + A)^{-1} Diag(beta) (V - Kbar S) one 16-token block at a time,
    //   Unew_b = X_bb (beta_b (V - Kbar S)_b - sum_{k<b} A_bk Unew_k),
    // then O = Z + P Unew (stored in step 3).
    auto consume_solve = [&](const Buf& B) {
        bf16x4 uh[NRT][CT], ul[NRT][CT];
#pragma unroll
        for (int b = 0; b < NRT; ++b) {
            const f32x4 bb = *reinterpret_cast<const f32x4*>(FUSE ? &B.betae[16 * b + 4 * g4] : &B.beta[16 * b + 4 * g4]);
            f32x4 acc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[ct][e] = bb[e] * Y[b][ct][e];
#pragma unroll
            for (int k = 0; k < b; ++k) {
                const int ao = (16 * b + lr) * K::AP + 16 * k + 4 * g4;
                const bf16x4 ah = frag4(&B.aoff[0][ao]), al = frag4(&B.aoff[1][ao]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma3_16(ah, al, uh[k][ct], ul[k][ct], acc[ct]);
            }
            const int xo = (16 * b + lr) * K::XP + 4 * g4;
            const bf16x4 xh = frag4(&B.xd[0][xo]), xl = frag4(&B.xd[1][xo]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                bf16x4 bh, bl;
                split4(acc[ct], bh, bl);
                const f32x4 u = mfma3_16(xh, xl, bh, bl, f32x4{0.f, 0.f, 0.f, 0.f});
                split4(u, uh[b][ct], ul[b][ct]);
            }
        }
        // 32-deep B operands of Unew: two stacked tiles in kperm order
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            ubh[ct] = cat8(uh[0][ct], uh[1][ct]);
            ubl[ct] = cat8(ul[0][ct], ul[1][ct]);
        }
        if constexpr (MODE == 0) {
            // O^T = Z^T + Unew^T P^T
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int ao = K::chm(16 * rt + lr, 8 * g4);
                const bf16x8 ph = frag(&B.p[0][ao]), pl = frag(&B.p[1][ao]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = mfma3(ubh[ct], ubl[ct], ph, pl, Z[rt][ct]);
            }
        }
    };

    // The output-gate logits of a chunk's rows (fused output pass only; rows past the end of a
    // ragged chunk read its last row and are not stored), requested before the solve so that
    // their latency overlaps the solve and the state update that precede the O store.
    using GRaw = typename std::conditional<std::is_same<IN, F32>::value, f32x4, uint2>::type;
    GRaw graw[NRT][CT];
    auto request_gate = [&](int chunk) __attribute__((always_inline)) {
        if constexpr (MODE == 0 && FUSE) {
            if (a.out_gate) {
                const long ts = t0 + static_cast<long>(chunk) * C;
                const int ntok = static_cast<int>(min(static_cast<long>(C), t1 - ts));
                const size_t obase = (static_cast<size_t>(ts) * H + h) * D + j0 + 4 * g4;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const int row = min(16 * rt + lr, ntok - 1);
                        graw[rt][ct] = *reinterpret_cast<const GRaw*>(static_cast<const ST*>(a.out_gate) + obase +
                                                                      static_cast<unsigned>(row * HD + 16 * ct));
                    }
            }
        }
    };
    // consumer step 3: the state update and the output rows of the chunk.  Per-channel decay: the
    // carried state takes X <- X + Ktil^T Unew with F folded into Ktil by the producer (no per-chunk
    // scaling), and is rescaled only when the next chunk resets F.  Scalar gate: St <- rho (St +
    // K^T U'), rho = e^{b_m'} e^{b_n - b_m}, applied as two factors when it falls below fp32 range
    // (steep decays, a chunk's summed log-decay below about -87).
    auto consume_update = [&](const Buf& B, const Buf& next, int chunk, bool last) {
        if constexpr (SG) {
            int tiny = 0;
#pragma unroll
            for (int pw = 0; pw < NPW; ++pw) tiny |= B.tiny[pw];
            tiny = __builtin_amdgcn_readfirstlane(tiny);
            // the first factor: rho, or e^{b_n - b_m} when the two are applied one after the other
            const float* r1 = tiny ? &B.rn[0] : &B.rho[0];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 rh = *reinterpret_cast<const f32x4*>(r1 + 16 * rt + 4 * g4);
                const int ao = K::chm(16 * rt + lr, 8 * g4);
                if constexpr (EXACT) {
                    const bf16x8 kh = frag(&B.kt[0][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) S[rt][ct] = mfma(kh, ubh[ct], mfma(kh, ubl[ct], S[rt][ct])) * rh;
                } else {
                    const bf16x8 kh = frag(&B.kt[0][ao]), kl = frag(&B.kt[1][ao]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) S[rt][ct] = mfma3(kh, kl, ubh[ct], ubl[ct], S[rt][ct]) * rh;
                }
            }
            if (tiny && !last) {   // the second factor, e^{b_m} of the next chunk
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const f32x4 r2 = *reinterpret_cast<const f32x4*>(&next.em[16 * rt + 4 * g4]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) S[rt][ct] *= r2;
                }
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int ao = K::chm(16 * rt + lr, 8 * g4);
                const bf16x8 kh = frag(&B.kt[0][ao]), kl = frag(&B.kt[1][ao]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[rt][ct] = mfma3(kh, kl, ubh[ct], ubl[ct], S[rt][ct]);
            }
            if (!last) {
                int rs = 0;
#pragma unroll
                for (int pw = 0; pw < NPW; ++pw) rs |= next.renorm[pw];
                if (__builtin_amdgcn_readfirstlane(rs)) {   // the next chunk resets F
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const int o = 16 * rt + 4 * g4;
                        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&next.f1[o]);
                        const f32x4 a2 = *reinterpret_cast<const f32x4*>(&next.f2[o]);
                        const f32x4 a3 = *reinterpret_cast<const f32x4*>(&next.f3[o]);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) S[rt][ct] = ((S[rt][ct] * a1) * a2) * a3;
                    }
                }
            }
        }
        if constexpr (MODE == 0) {
            const long ts = t0 + static_cast<long>(chunk) * C;
            const int ntok = static_cast<int>(min(static_cast<long>(C), t1 - ts));
            // a workgroup whose ordering broke stores NaN rows from here on
            if (__builtin_amdgcn_readfirstlane(lds_read(broken)) != 0) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Z[rt][ct] = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                                        __builtin_nanf(""), __builtin_nanf("")};
            }
            // lane (g4, lr) holds 4 consecutive columns of token 16 rt + lr
            const size_t obase = (static_cast<size_t>(ts) * H + h) * D + j0 + 4 * g4;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int row = 16 * rt + lr;
                if (row < ntok) {
                    float fo = 1.f;
                    if constexpr (SG) fo = B.fo[row];
                    if constexpr (FUSE) fo = SG ? fo * B.os[row] : B.os[row];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        f32x4 ov = Z[rt][ct] * fo;
                        if constexpr (FUSE) {
                            if (a.out_gate) {
                                f32x4 gv;
                                if constexpr (std::is_same<IN, F32>::value) {
                                    gv = graw[rt][ct];
                                } else {
                                    const uint2 x = graw[rt][ct];
                                    gv = f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                                               __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e) ov[e] *= sigmoid_f(gv[e]);
                            }
                        }
                        store_out4<OUT_BF16>(a.o, obase + static_cast<unsigned>(row * HD + 16 * ct), ov);
                    }
                }
            }
        }
    };

    // ================================================================ chunk loops
    // Producer and consumer waves run separate loops, ordered by the LDS counters alone (no
    // workgroup barrier).  The producers build chunk i in three phases, each closed by a count
    // that the other producers wait for: phase 1 (decay, planes, and the previous chunk's rho),
    // phase 2 (A tiles), phase 3 (diagonal inverses, then Ktil_m^T over Ktil_m once the
    // consumers have taken the P tiles from it; closes `ready`).  Before phase 1 of chunk i they
    // wait until every consumer is done with chunk i - 2, the last user of the same buffer.  A
    // consumer runs chunk i once it is `ready`; after its solve it waits for the producers'
    // phase 1 of chunk i + 1, forms that chunk's P tiles (closing `pt`), and then runs the
    // state update, which needs chunk i's rho from that same phase.
    const int n_chunks = c_end - c_begin;
    if (producer) {
        if (n_chunks > 0) fetch(c_begin, -1);
        for (int i = 0; i < n_chunks; ++i) {
            const int chunk = c_begin + i;
            Buf& B = sm.buf[chunk & 1];
            if (i >= 2) wait_count(&sm.sync.done[chunk & 1], K::NCW * (i / 2), broken, wl);
            produce_decay(B, chunk, i > 0 ? &sm.buf[(chunk & 1) ^ 1] : nullptr);
            signal_count(&sm.sync.p1);
            wait_count(&sm.sync.p1, NPW * (i + 1), broken, wl);
            // The inputs of the next chunk are requested outside the decay phase: k and
            // log_alpha (used first) here, q, v and beta before phase 3, except on the waves
            // that solve the diagonal blocks in phase 3, which request all here.
            if (chunk + 1 < c_end) fetch(chunk + 1, solver ? -1 : 0);
            produce_products(B);
            produce_token_scales(B);
            signal_count(&sm.sync.p2);
            wait_count(&sm.sync.p2, NPW * (i + 1), broken, wl);
            if (!solver && chunk + 1 < c_end) fetch(chunk + 1, 1);
            produce_inverse(B);
            wait_count(&sm.sync.pt, K::NCW * (i + 1), broken, wl);
            produce_transpose(B);
            signal_count(&sm.sync.ready);
        }
        if (n_chunks > 0) {
            // rho of the last chunk (no next midpoint): e^{b_n - b_m}, which leaves S itself
            if (tg == 0) {
                Buf& lb = sm.buf[(c_end - 1) & 1];
                if constexpr (SG) {
#pragma unroll
                    for (int ch = 0; ch < 4; ++ch) lb.rho[c4 + ch] = enm[ch];
                    if (l == 0) lb.tiny[w] = 0;
                } else {
                    // S = Diag(F e^{b_n - b_m}) X after the last chunk
#pragma unroll
                    for (int ch = 0; ch < 4; ++ch) {
                        lb.fin1[c4 + ch] = exp2f_hw(lf[ch]);
                        lb.fin2[c4 + ch] = exp2f_hw(lrn[ch]);
                    }
                }
            }
            signal_count(&sm.sync.p1);
        }
        return;
    }
    // With the scalar gate the producers have little vector work and the consumers' chain sets
    // the pace: the consumer waves issue first when both sides are ready (2.6% faster on the
    // long-context shape; the per-channel kernels gain nothing from either side's priority and
    // lose 5% when the consumers go first).
    if constexpr (SG) __builtin_amdgcn_s_setprio(2);
    if (n_chunks > 0) {
        wait_count(&sm.sync.p1, NPW, broken, wl);
        consume_ptiles(sm.buf[c_begin & 1]);
        signal_count(&sm.sync.pt);
        wait_count(&sm.sync.ready, NPW, broken, wl);
        const Buf& first = sm.buf[c_begin & 1];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 em = *reinterpret_cast<const f32x4*>(&first.em[16 * rt + 4 * g4]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[rt][ct] *= em;
        }
        split_state();
    }
    for (int i = 0; i < n_chunks; ++i) {
        const int chunk = c_begin + i;
        const Buf& cur = sm.buf[chunk & 1];
        if (i > 0) wait_count(&sm.sync.ready, NPW * (i + 1), broken, wl);
        consume_project(cur, chunk);
        request_gate(chunk);
        consume_solve(cur);
        wait_count(&sm.sync.p1, NPW * (i + 2), broken, wl);
        if (i + 1 < n_chunks) {
            consume_ptiles(sm.buf[(chunk & 1) ^ 1]);
            signal_count(&sm.sync.pt);
        }
        consume_update(cur, sm.buf[(chunk & 1) ^ 1], chunk, i + 1 == n_chunks);
        signal_count(&sm.sync.done[chunk & 1]);
        if (i + 1 < n_chunks) split_state();
    }

    // ---------------------------------------------------------------- exit state
    if constexpr (!SG) {
        if (n_chunks > 0) {   // S = Diag(F e^{b_n - b_m}) X after the last chunk
            const Buf& lb = sm.buf[(c_end - 1) & 1];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(&lb.fin1[16 * rt + 4 * g4]);
                const f32x4 a2 = *reinterpret_cast<const f32x4*>(&lb.fin2[16 * rt + 4 * g4]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[rt][ct] = (S[rt][ct] * a1) * a2;
            }
        }
    }
    float* const dst = MODE == 1 && is_phi ? u.phi : u.exit;
    const bool poison = __builtin_amdgcn_readfirstlane(lds_read(broken)) != 0;
    if (poison && l == 0 && a.status) *reinterpret_cast<volatile int*>(a.status) = 1;
    if (dst) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(16 * rt + 4 * g4 + e) * D + j0 + 16 * ct + lr] = poison ? __builtin_nanf("") : S[rt][ct][e];
    }
}

template <int D, typename IN, bool OUT_BF16, int MODE, bool SG = false, bool FUSE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(PCfg<D, MODE>::NT, PCfg<D, MODE>::NT),
                          amdgpu_waves_per_eu(PCfg<D, MODE>::WPE, PCfg<D, MODE>::WPE)))
void pipe_kernel(KernelArgs a) {
    __shared__ PSmem<D, MODE, std::is_same<IN, BF16>::value> sm;
    constexpr int C = PCfg<D, MODE>::C;
    Unit u;
    if constexpr (MODE == 0) {
        if (a.seg) {
            if (unit_segmented<D, C>(a, blockIdx.x, true, u) < 0) return;
        } else {
            u = a.cu ? unit_packed<D, C>(a, blockIdx.x) : unit_equal<D, C, 0>(a, blockIdx.x);
        }
    } else {
        u = unit_equal<D, C, 1>(a, blockIdx.x);
    }
    pipe_body<D, IN, OUT_BF16, MODE, SG, FUSE, PCfg<D, MODE>::CT>(a, sm, u);
}

// Pass 1 of the split schedule in one launch: workgroups [0, NH) run segment 0's output pass
// from S0 (writing o and, as segment 1's entry state, its exit state) with 16-column consumer
// waves; the others run the summaries of segments 1..G-2.  Both have D/32 producer and D/16
// consumer waves, and the launch order puts segment 0's workgroups first.  For a packed batch
// the segment table assigns the two kinds of work per sequence.
template <int D, typename IN, bool OUT_BF16, bool SG = false, bool FUSE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(PCfg<D, 1>::NT, PCfg<D, 1>::NT),
                          amdgpu_waves_per_eu(PCfg<D, 1>::WPE, PCfg<D, 1>::WPE)))
void pipe_pass1_kernel(KernelArgs a) {
    static_assert(PCfg<D, 0, 1>::NT == PCfg<D, 1>::NT, "both passes need the same workgroup size");
    constexpr bool VLDS = std::is_same<IN, BF16>::value;
    __shared__ union Both {
        PSmem<D, 0, VLDS> out;
        PSmem<D, 1, VLDS> sum;
    } sm;
    constexpr int C = PCfg<D, 1>::C;
    const int block = blockIdx.x;
    Unit u;
    int mode;
    if (a.seg) {
        mode = unit_segmented<D, C>(a, block, false, u);
        if (mode < 0) return;
    } else if (block < a.NH) {
        KernelArgs a0 = a;
        a0.seg0 = 0;
        a0.split0 = 1;
        u = unit_equal<D, C, 0>(a0, block);
        mode = 0;
    } else {
        KernelArgs a1 = a;
        a1.seg0 = 1;
        u = unit_equal<D, C, 1>(a1, block - a.NH);
        mode = 1;
    }
    if (mode == 0) pipe_body<D, IN, OUT_BF16, 0, SG, FUSE, 1>(a, sm.out, u);
    else pipe_body<D, IN, OUT_BF16, 1, SG, FUSE, 2>(a, sm.sum, u);
}

// Entry states of segments s_first..G-1:  S_e(s) = Phi(s-1) S_e(s-1) + S_loc(s-1), starting from
// S_e(s_first - 1) = init (S0, or segment 1's entry when segment 0 ran its output pass first;
// null: zero).  One workgroup per (unit, 16-column slice).  Phi(s-1) is staged through LDS with
// coalesced loads, and the next segment's Phi and S_loc are requested while this one is applied;
// the products run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), D/64 16-row tiles per wave.
// With a segment table (packed batches), unit r * H + h is rank r's sequence: its own G and
// state slots, and s_first = 2 (segment 0's output pass left segment 1's entry state).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ init, const float* __restrict__ phi,
                                                      const float* __restrict__ sloc, float* __restrict__ se,
                                                      int NH, int G, int s_first, const int32_t* __restrict__ seg,
                                                      int H) {
    constexpr int LP = D + 4;              // row pitch of Phi in LDS
    constexpr int LC = 20;                 // row pitch of the 16-column state slice
    constexpr int RT = D / 64;             // row tiles per wave
    constexpr int NF = D * D / 4 / 256;    // float4 of Phi per thread
    using fx4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;
    __shared__ __attribute__((aligned(16))) float sphi[D * LP];
    __shared__ __attribute__((aligned(16))) float cur[2][D * LC];
    const int unit = blockIdx.x, c0 = blockIdx.y * 16, tid = threadIdx.x, w = tid >> 6;
    const int i = tid & 15, kq = (tid & 63) >> 4;
    // step s reads Phi and S_loc of segment s-1 at slot p0 + (s-1) st and writes segment s's
    // entry state at slot e0 + (s-1) st (slots of D x D floats)
    long p0 = unit, e0 = unit, st = NH;
    const float* ini = init ? init + static_cast<size_t>(unit) * D * D : nullptr;
    if (seg) {
        const int N = NH / H, r = unit / H, h = unit % H;
        G = 1 + seg[kSegHdr + 2 * N + r];
        if (G < 3) return;
        const long base = seg[kSegHdr + 4 * N + 1 + r];
        s_first = 2;
        p0 = (base - 1) * H + h;
        e0 = base * H + h;
        st = H;
        ini = se + static_cast<size_t>(e0) * D * D;
    }
    for (int e = tid; e < D * 16; e += 256) cur[0][(e >> 4) * LC + (e & 15)] = ini ? ini[(e >> 4) * D + c0 + (e & 15)] : 0.f;
    fx4 pf[NF];
    float pl[RT][4];
    auto fetch = [&](int s) __attribute__((always_inline)) {
        const size_t sb = static_cast<size_t>(p0 + (s - 1) * st) * D * D;
        const fx4* src = reinterpret_cast<const fx4*>(phi + sb);
#pragma unroll
        for (int f = 0; f < NF; ++f) pf[f] = src[tid + 256 * f];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) pl[t][v] = sloc[sb + static_cast<size_t>(16 * (w * RT + t) + 4 * kq + v) * D + c0 + i];
    };
    if (s_first < G) fetch(s_first);
    int b = 0;
    for (int s = s_first; s < G; ++s) {
        __syncthreads();   // the last step's reads of sphi are done and its slice is complete
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int e = tid + 256 * f;
            *reinterpret_cast<fx4*>(sphi + (e / (D / 4)) * LP + 4 * (e % (D / 4))) = pf[f];
        }
        fx4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = pl[t][v];
        __syncthreads();
        if (s + 1 < G) fetch(s + 1);
        // lane (i, kq) supplies key index k = 16 s2 + 4 kq + e of row i and of column i in the
        // e-th product of step s2, so its Phi values are four consecutive floats
#pragma unroll 2
        for (int s2 = 0; s2 < D / 16; ++s2) {
            fx4 a4[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t)
                a4[t] = *reinterpret_cast<const fx4*>(sphi + (16 * (w * RT + t) + i) * LP + 16 * s2 + 4 * kq);
            const float* bc = cur[b] + (16 * s2 + 4 * kq) * LC + i;
            const float b0 = bc[0], b1 = bc[LC], b2 = bc[2 * LC], b3 = bc[3 * LC];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[t][0], b0, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[t][1], b1, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[t][2], b2, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[t][3], b3, acc[t], 0, 0, 0);
            }
        }
        const size_t sb = static_cast<size_t>(e0 + (s - 1) * st) * D * D;
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * (w * RT + t) + 4 * kq + v;
                cur[b ^ 1][row * LC + i] = acc[t][v];
                se[sb + static_cast<size_t>(row) * D + c0 + i] = acc[t][v];
            }
        b ^= 1;
    }
}

// Longest-first order of packed sequences (ties by index).  Each thread ranks one sequence
// against all others, O(N) per thread over a grid of N threads: for batches of up to
// kOrderExactMax sequences.  Larger batches take the bucketed order below.
__global__ __launch_bounds__(256) void order_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ order, int N) {
    __shared__ int len[kOrderExactMax];   // every sequence's length, read once per workgroup
    for (int m = threadIdx.x; m < N; m += blockDim.x) len[m] = cu[m + 1] - cu[m];
    __syncthreads();
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int li = len[i];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int lm = len[m];
        rank += (lm > li) || (lm == li && m < i);
    }
    order[rank] = i;
}

// Bucketed longest-first order for large packed batches: sequences go to kOrderBuckets buckets
// by length / 32 (the top bucket takes everything from 32 * (kOrderBuckets - 1) tokens on), in
// decreasing bucket order; within a bucket the order is that of the atomic cursor.  The order
// only decides which workgroup runs which (sequence, head) when, never what it computes, so the
// outputs do not depend on it.  Four launches: clear the counters (a fill kernel, no memset),
// count, exclusive scan, scatter.
__device__ __forceinline__ int order_bucket(const int32_t* cu, int i) {
    const int len = cu[i + 1] - cu[i];
    return kOrderBuckets - 1 - min(max(len, 0) >> 5, kOrderBuckets - 1);   // longest first
}

__global__ __launch_bounds__(kOrderBuckets) void order_clear_kernel(int32_t* __restrict__ cnt) {
    cnt[threadIdx.x] = 0;
    cnt[kOrderBuckets + threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void order_count_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ cnt,
                                                          int N) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) atomicAdd(&cnt[order_bucket(cu, i)], 1);
}

// cnt[kOrderBuckets + b] <- sum of cnt[b'] over b' < b (one workgroup)
__global__ __launch_bounds__(kOrderBuckets) void order_scan_kernel(int32_t* __restrict__ cnt) {
    __shared__ int32_t buf[kOrderBuckets];
    const int t = threadIdx.x;
    const int c = cnt[t];
    buf[t] = c;
    __syncthreads();
    for (int off = 1; off < kOrderBuckets; off <<= 1) {
        const int x = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += x;
        __syncthreads();
    }
    cnt[kOrderBuckets + t] = buf[t] - c;
}

__global__ __launch_bounds__(256) void order_scatter_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ order, int N) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) order[atomicAdd(&cnt[kOrderBuckets + order_bucket(cu, i)], 1)] = i;
}

// Segment plan of a packed batch whose (sequence, head) pairs are too few to fill the chip, in
// one workgroup (one thread per sequence, N <= 256).  A sequence of c chunks is cut into a
// segment 0 of about t = round(ratio L) chunks (t = L for L < 64) and G - 1 = ceil((c - t) / L)
// segments of L chunks after it (none when c <= t), segment 0 taking the remainder.  L is the
// smallest length >= Lmin for which the pass-1 workgroups, the sum over sequences of
// max(1, G - 1), fit `items` per head, raised to Lc, the smallest length with 25 Lc^2 >=
// 9 c_max, when that fits too: the combine chains a sequence's segments one after another, at
// about 0.8 of a chunk's time per segment on MI355X, so with segment 0 about L long the call
// takes about 2.2 L + 0.8 c_max / L chunk-times, least near L = 0.6 sqrt(c_max).  When the
// result leaves no gain over one pass per sequence (2 L + 8 >= c_max), no sequence is cut.
// Ranks are longest first (ties by index), as in the one-pass order.
__global__ __launch_bounds__(256) void seg_plan_kernel(const int32_t* __restrict__ cu, int N, int C, int items,
                                                       int Lmin, float ratio, int32_t* __restrict__ tab) {
    __shared__ int red[2][4];   // per-wave partials, two sets so consecutive reductions need one barrier each
    __shared__ int more_r[256];
    __shared__ int lens[256];
    const int i = threadIdx.x;
    const bool act = i < N;
    const int len = act ? cu[i + 1] - cu[i] : 0;
    lens[i] = len;
    const int c = (len + C - 1) / C;
    int parity = 0;
    // over the 256 threads: a wave reduction, then the four waves' partials through LDS
    auto reduce = [&](int x, bool take_max) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const int y = __shfl_xor(x, o, 64);
            x = take_max ? max(x, y) : x + y;
        }
        if ((i & 63) == 0) red[parity][i >> 6] = x;
        __syncthreads();
        const int* p = red[parity];
        parity ^= 1;
        return take_max ? max(max(p[0], p[1]), max(p[2], p[3])) : (p[0] + p[1]) + (p[2] + p[3]);
    };
    auto more_of = [&](int L) {
        const int t = L >= 64 ? max(1, static_cast<int>(rintf(ratio * L))) : L;
        int m = c > t ? (c - t + L - 1) / L : 0;
        if (m > 0 && c - m * L < 1) --m;   // segment 0 keeps at least one chunk
        return m;
    };
    const int maxc = reduce(c, true);
    int lo = Lmin, hi = max(Lmin, maxc);   // at L = max(Lmin, maxc) every sequence needs one item
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (reduce(act ? max(1, more_of(mid)) : 0, false) <= items) hi = mid;
        else lo = mid + 1;
    }
    int L = lo;
    int Lc = static_cast<int>(sqrtf(0.36f * static_cast<float>(maxc)));
    while (25LL * Lc * Lc < 9LL * maxc) ++Lc;
    while (Lc > 1 && 25LL * (Lc - 1) * (Lc - 1) >= 9LL * maxc) --Lc;
    if (Lc > L && reduce(act ? max(1, more_of(Lc)) : 0, false) <= items) L = Lc;
    const bool cut = 2 * L + 8 < maxc;
    if (act) {
        int rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = lens[m];
            rank += (lm > len) || (lm == len && m < i);
        }
        const int m = cut ? more_of(L) : 0;
        tab[kSegHdr + rank] = i;
        tab[kSegHdr + N + rank] = c - m * L;
        tab[kSegHdr + 2 * N + rank] = m;
        more_r[rank] = m;
    }
    __syncthreads();
    if (i <= N) {
        int s1 = 0, s2 = 0;
        for (int r = 0; r < i; ++r) {
            s1 += max(1, more_r[r]);
            s2 += more_r[r];
        }
        tab[kSegHdr + 3 * N + i] = s1;
        tab[kSegHdr + 4 * N + 1 + i] = s2;
    }
    if (i == 0) tab[0] = L;
}

// Clears the call's status word before its kernels run (a fill kernel rather than a memset, so
// that the call stays free of memset nodes under stream capture).
__global__ void status_clear_kernel(int* status) {
    if (threadIdx.x == 0) *status = 0;
}

template <int D, int C, typename IN, bool OB, bool SG = false, bool FUSE = false>
hipError_t launch_variant(const PrefillArgs& pa, const PrefillPlan& plan, hipStream_t stream) {
    static_assert(!FUSE || C == 32, "the fused prologue runs on the pipelined 32-token kernel");
    static_assert(!SG || C == 32, "the scalar gate runs on the pipelined 32-token kernel");
    KernelArgs a;
    a.q = pa.q; a.k = pa.k; a.v = pa.v; a.g = pa.g; a.beta = pa.beta;
    a.S0 = pa.S0; a.cu = pa.cu; a.o = pa.o; a.S_final = pa.S_final;
    a.T = pa.T; a.H = pa.H; a.NH = pa.N * pa.H; a.G = plan.G; a.cps = plan.cps; a.chunks = plan.chunks;
    a.cps0 = plan.cps;
    a.seg0 = 0;
    a.split0 = 0;
    a.fuse_flags = pa.fuse_flags; a.decay_bias = pa.decay_bias; a.decay_scale = pa.decay_scale;
    a.out_gate = pa.out_gate;
    a.wait_limit = pa.wait_limit;
    char* ws = static_cast<char*>(pa.workspace);
    a.status = reinterpret_cast<int*>(ws + plan.off_status);
    a.order = pa.cu ? reinterpret_cast<const int32_t*>(ws + plan.off_order) : nullptr;
    a.seg = nullptr;
    const bool states = plan.G > 1 || plan.seg_items > 0;
    a.phi = states ? reinterpret_cast<float*>(ws + plan.off_phi) : nullptr;
    a.sloc = states ? reinterpret_cast<float*>(ws + plan.off_sloc) : nullptr;
    a.se = states ? reinterpret_cast<float*>(ws + plan.off_se) : nullptr;
    const int NH = a.NH;
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, stream, a.status);
    // The 32-token chunk runs the producer/consumer kernel; the 64-token chunk, whose
    // operands do not fit twice in LDS, the single-buffered one.
    auto pass = [&](int mode, int grid, const KernelArgs& ka) {
        if constexpr (C == 32) {
            if (mode == 0)
                hipLaunchKernelGGL((pipe_kernel<D, IN, OB, 0, SG, FUSE>), dim3(grid), dim3(PCfg<D, 0>::NT), 0, stream, ka);
            else
                hipLaunchKernelGGL((pipe_kernel<D, IN, OB, 1, SG, FUSE>), dim3(grid), dim3(PCfg<D, 1>::NT), 0, stream, ka);
        } else {
            if (mode == 0)
                hipLaunchKernelGGL((chunk_kernel<D, C, IN, OB, 0>), dim3(grid), dim3(Cfg<D, C, 0>::NT), 0, stream, ka);
            else
                hipLaunchKernelGGL((chunk_kernel<D, C, IN, OB, 1>), dim3(grid), dim3(Cfg<D, C, 1>::NT), 0, stream, ka);
        }
    };
    // Segment 0's output pass runs beside the summaries of later segments, so it may be as long
    // as the ratio of a summary chunk's cost to an output chunk's (measured on MI355X: plain
    // 1.18, scalar gate 1.08, fused output pass with its gate 0.95); the other segments share
    // the rest equally.  Only for segments of 64 chunks or more, where the per-chunk costs
    // outweigh the fixed ones of a segment (state loads and stores, the pipeline's fill).
    constexpr double kSeg0Ratio = FUSE ? 0.95 : (SG ? 1.08 : 1.18);
    if (pa.cu) {
        if constexpr (C == 32) {
            if (plan.seg_items > 0) {
                // Packed batch with too few (sequence, head) pairs to fill the chip: the split
                // schedule per sequence, from the segment table the first kernel writes.
                int32_t* tab = reinterpret_cast<int32_t*>(ws + plan.off_order);
                hipLaunchKernelGGL(seg_plan_kernel, dim3(1), dim3(256), 0, stream, pa.cu, pa.N, C,
                                   plan.seg_items, kMinChunksPerSegment, static_cast<float>(kSeg0Ratio), tab);
                a.seg = tab;
                a.order = nullptr;
                const int grid = plan.seg_items * pa.H;
                hipLaunchKernelGGL((pipe_pass1_kernel<D, IN, OB, SG, FUSE>), dim3(grid), dim3(PCfg<D, 1>::NT), 0,
                                   stream, a);
                hipLaunchKernelGGL(combine_kernel<D>, dim3(NH, D / 16), dim3(256), 0, stream, nullptr, a.phi,
                                   a.sloc, a.se, NH, 0, 2, a.seg, pa.H);
                pass(0, grid, a);
                return hipGetLastError();
            }
        }
        int32_t* order = reinterpret_cast<int32_t*>(ws + plan.off_order);
        const dim3 grid((pa.N + 255) / 256);
        if (pa.N <= kOrderExactMax) {
            hipLaunchKernelGGL(order_kernel, grid, dim3(256), 0, stream, pa.cu, order, pa.N);
        } else {
            int32_t* cnt = reinterpret_cast<int32_t*>(ws + plan.off_buckets);
            hipLaunchKernelGGL(order_clear_kernel, dim3(1), dim3(kOrderBuckets), 0, stream, cnt);
            hipLaunchKernelGGL(order_count_kernel, grid, dim3(256), 0, stream, pa.cu, cnt, pa.N);
            hipLaunchKernelGGL(order_scan_kernel, dim3(1), dim3(kOrderBuckets), 0, stream, cnt);
            hipLaunchKernelGGL(order_scatter_kernel, grid, dim3(256), 0, stream, pa.cu, cnt, order, pa.N);
        }
        pass(0, NH, a);
        return hipGetLastError();
    }
    if constexpr (C == 32) {
        if (plan.G > 1 && plan.split0) {
            // G, and with it the workspace, is unchanged by the longer segment 0.
            const int cps = static_cast<int>(std::ceil(plan.chunks / (plan.G - 1 + kSeg0Ratio)));
            const int cps0 = plan.chunks - (plan.G - 1) * cps;
            if (plan.cps >= 64 && cps0 >= 1) {
                a.cps = cps;
                a.cps0 = cps0;
            }
            // one launch: segment 0's output pass (exit state -> segment 1's entry) and the
            // summaries of segments 1..G-2
            hipLaunchKernelGGL((pipe_pass1_kernel<D, IN, OB, SG, FUSE>), dim3(NH * (plan.G - 1)), dim3(PCfg<D, 1>::NT),
                               0, stream, a);
            if (plan.G > 2)
                hipLaunchKernelGGL(combine_kernel<D>, dim3(NH, D / 16), dim3(256), 0, stream, a.se, a.phi, a.sloc,
                                   a.se, NH, plan.G, 2, nullptr, pa.H);
            KernelArgs a1 = a;   // output passes of segments 1..G-1
            a1.seg0 = 1;
            pass(0, NH * (plan.G - 1), a1);
            return hipGetLastError();
        }
    }
    if (plan.G > 1) {
        pass(1, NH * (plan.G - 1), a);
        hipLaunchKernelGGL(combine_kernel<D>, dim3(NH, D / 16), dim3(256), 0, stream, pa.S0, a.phi, a.sloc, a.se,
                           NH, plan.G, 1, nullptr, pa.H);
    }
    pass(0, NH * plan.G, a);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

PrefillPlan plan_prefill(int B, int T, int H, int D, int N, bool varlen, int chunk) {
    PrefillPlan p;
    p.chunk = chunk == 0 ? kDefaultChunk : chunk;
    // Every plan starts with the call's status word (256 bytes reserved).
    p.off_status = 0;
    if (varlen) {
        p.G = 1;
        p.off_order = kStatusBytes;
        const long pairs = static_cast<long>(N) * H;
        const long tc = (static_cast<long>(T) + p.chunk - 1) / p.chunk;   // >= the longest sequence's chunks
        if (p.chunk == 32 && pairs > 0 && pairs < kComputeUnits && tc >= 2 * kMinChunksPerSegment) {
            // Too few (sequence, head) pairs to fill the chip: each sequence is cut into segments
            // on the device, with at most kComputeUnits / H pass-1 workgroups per head (N of them
            // at least, which N * H < kComputeUnits allows) and as many state slots.
            p.seg_items = kComputeUnits / H;
            const size_t mat = static_cast<size_t>(p.seg_items) * H * D * D * sizeof(float);
            const size_t tab = align256(seg_table_ints(N) * sizeof(int32_t));
            p.off_phi = kStatusBytes + tab;
            p.off_sloc = p.off_phi + align256(mat);
            p.off_se = p.off_sloc + align256(mat);
            p.workspace_bytes = p.off_se + align256(mat);
            return p;
        }
        p.workspace_bytes = kStatusBytes + align256(static_cast<size_t>(N) * sizeof(int32_t));
        if (N > kOrderExactMax) {   // bucket counters and cursors of the bucketed order
            p.off_buckets = p.workspace_bytes;
            p.workspace_bytes += align256(2 * kOrderBuckets * sizeof(int32_t));
        }
        return p;
    }
    (void)B;
    p.chunks = (T + p.chunk - 1) / p.chunk;
    const long units = static_cast<long>(N) * H;
    // workgroups that fill the chip: one per compute unit
    const long target = static_cast<long>(kComputeUnits);
    int G = 1;
    bool split = false;
    if (units > 0 && units < target && p.chunks >= 2 * kMinChunksPerSegment) {
        G = static_cast<int>((target + units - 1) / units);
        G = std::min(G, p.chunks / kMinChunksPerSegment);
        G = std::max(G, 1);
        // The pipelined kernel's split schedule: segment 0's output pass beside the summaries of
        // segments 1..G-2, then the output passes of segments 1..G-1; each fills the chip with
        // floor(target / units) segments, one more than the plain schedule's summary pass.
        if (p.chunk == 32) {
            const int gs = std::min(static_cast<int>(target / units) + 1, p.chunks / kMinChunksPerSegment);
            if (gs >= 3) {
                G = gs;
                split = true;
            }
        }
    }
    p.cps = p.chunks > 0 ? (p.chunks + G - 1) / G : 0;
    p.G = p.cps > 0 ? (p.chunks + p.cps - 1) / p.cps : 1;
    p.split0 = split && p.G >= 3;
    p.workspace_bytes = kStatusBytes;
    if (p.G > 1) {
        const size_t mat = static_cast<size_t>(units) * (p.G - 1) * D * D * sizeof(float);
        p.off_phi = kStatusBytes;
        p.off_sloc = kStatusBytes + align256(mat);
        p.off_se = kStatusBytes + 2 * align256(mat);
        p.workspace_bytes = kStatusBytes + 3 * align256(mat);
    }
    return p;
}

hipError_t clear_prefill_status(void* workspace, const PrefillPlan& plan, hipStream_t stream) {
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, stream,
                       reinterpret_cast<int*>(static_cast<char*>(workspace) + plan.off_status));
    return hipGetLastError();
}

namespace {
template <int D, typename IN, bool SG>
hipError_t segment_states_typed(const PrefillArgs& pa, int W, int G, float* entry, hipStream_t stream) {
    KernelArgs a;
    a.q = pa.q; a.k = pa.k; a.v = pa.v; a.g = pa.g; a.beta = pa.beta;
    a.S0 = pa.S0; a.cu = nullptr; a.order = nullptr; a.seg = nullptr; a.o = nullptr; a.S_final = nullptr;
    a.T = pa.T; a.H = pa.H; a.NH = pa.N * pa.H; a.G = G; a.cps = W; a.cps0 = W;
    a.chunks = (pa.T + 31) / 32; a.seg0 = 0; a.split0 = 0;
    a.fuse_flags = 0; a.decay_bias = 0.f; a.decay_scale = 1.f; a.out_gate = nullptr;
    a.wait_limit = pa.wait_limit;
    char* ws = static_cast<char*>(pa.workspace);
    const size_t mat = align256(static_cast<size_t>(a.NH) * (G - 1) * D * D * sizeof(float));
    a.status = reinterpret_cast<int*>(ws);
    a.phi = reinterpret_cast<float*>(ws + kStatusBytes);
    a.sloc = reinterpret_cast<float*>(ws + kStatusBytes + mat);
    a.se = entry;
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, stream, a.status);
    hipLaunchKernelGGL((pipe_kernel<D, IN, false, 1, SG, false>), dim3(a.NH * (G - 1)), dim3(PCfg<D, 1>::NT), 0,
                       stream, a);
    hipLaunchKernelGGL(combine_kernel<D>, dim3(a.NH, D / 16), dim3(256), 0, stream, pa.S0, a.phi, a.sloc, entry,
                       a.NH, G, 1, nullptr, pa.H);
    return hipGetLastError();
}
}  // namespace

size_t segment_states_workspace_bytes(int N, int H, int D, int G) {
    if (G < 2) return kStatusBytes;
    return kStatusBytes + 2 * align256(static_cast<size_t>(N) * H * (G - 1) * D * D * sizeof(float));
}

hipError_t launch_segment_states(const PrefillArgs& a, int W, int G, float* entry, hipStream_t stream) {
    if (G < 2 || a.N * a.H == 0) return hipSuccess;
#define KDA_SEG_CASE(DD, INT)                                                                      \
    if (a.D == DD && a.in_bf16 == std::is_same<INT, BF16>::value)                                  \
        return a.scalar_gate ? segment_states_typed<DD, INT, true>(a, W, G, entry, stream)        \
                             : segment_states_typed<DD, INT, false>(a, W, G, entry, stream);
    KDA_SEG_CASE(128, BF16)
    KDA_SEG_CASE(128, F32)
    KDA_SEG_CASE(64, BF16)
    KDA_SEG_CASE(64, F32)
#undef KDA_SEG_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream) {
#define KDA_PREFILL_CASE(DD, CC, INT, OB)                                                              \
    if (a.D == DD && plan.chunk == CC && a.in_bf16 == std::is_same<INT, BF16>::value && a.out_bf16 == OB) { \
        if (a.scalar_gate || a.fuse_flags || a.out_gate) {                                             \
            if constexpr (CC == 32) {                                                                  \
                if (a.scalar_gate && !a.fuse_flags && !a.out_gate)                                     \
                    return launch_variant<DD, CC, INT, OB, true>(a, plan, stream);                      \
                if (a.scalar_gate) return launch_variant<DD, CC, INT, OB, true, true>(a, plan, stream);  \
                return launch_variant<DD, CC, INT, OB, false, true>(a, plan, stream);                   \
            }                                                                                          \
            return hipErrorInvalidValue;                                                               \
        }                                                                                              \
        return launch_variant<DD, CC, INT, OB>(a, plan, stream);                                       \
    }
#define KDA_PREFILL_D(DD, CC)              \
    KDA_PREFILL_CASE(DD, CC, BF16, true)   \
    KDA_PREFILL_CASE(DD, CC, BF16, false)  \
    KDA_PREFILL_CASE(DD, CC, F32, true)    \
    KDA_PREFILL_CASE(DD, CC, F32, false)
    KDA_PREFILL_D(128, 32)
    KDA_PREFILL_D(128, 64)
    KDA_PREFILL_D(64, 32)
    KDA_PREFILL_D(64, 64)
#undef KDA_PREFILL_D
#undef KDA_PREFILL_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
