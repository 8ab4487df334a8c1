// kda_api.hip -- host side of libkda.so: argument checks, workspace carving and
// kernel launches for the C ABI declared in include/kda.h.
//
// Every check that can be made from the arguments runs before the first HIP
// call, so a rejected call touches no device state.  Nothing here allocates or
// synchronises.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "kda.h"
#include "kda_launch.h"
#include "kda_backward.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(kda_dtype d) { return d == KDA_BF16 ? 2 : 4; }

bool dtype_ok(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }

bool head_ok(int Dk, int Dv) { return Dk == Dv && (Dk == 64 || Dk == 128); }

// [a, a+na) and [b, b+nb) overlap?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

extern "C" size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                                int has_cu_seqlens, int chunk) {
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0 || !head_ok(Dk, Dv)) return 0;
    if (!kda::chunk_supported(chunk)) return 0;
    kda::PrefillPlan plan = kda::plan_prefill(B, T, H, Dk, num_seqs, has_cu_seqlens != 0, chunk);
    return plan.workspace_bytes;
}

namespace {

// Prefill for either decay layout: per key channel (KDA, log_alpha [B, T, H, Dk]) or one value
// per token and head (scalar gate, log_alpha [B, T, H]).
// Validated fusion options (nullptr when none are requested).
bool fusion_ok(const kda_fusion* f) {
    if (!f) return true;
    if (f->flags & ~(KDA_FUSE_QK_L2NORM | KDA_FUSE_BETA_SIGMOID | KDA_FUSE_DECAY_LOGSIGMOID)) return false;
    if ((f->flags & KDA_FUSE_DECAY_LOGSIGMOID) && !(f->decay_scale > 0.f && f->decay_scale < 3.0e38f)) return false;
    if ((f->flags & KDA_FUSE_DECAY_LOGSIGMOID) && !(f->decay_bias > -3.0e38f && f->decay_bias < 3.0e38f)) return false;
    return f->out_gate == nullptr || aligned16(f->out_gate);
}

kda::Fusion to_fusion(const kda_fusion* f) {
    kda::Fusion x;
    if (f) {
        x.flags = f->flags;
        x.decay_bias = f->decay_bias;
        x.decay_scale = (f->flags & KDA_FUSE_DECAY_LOGSIGMOID) ? f->decay_scale : 1.f;
        x.out_gate = f->out_gate;
    }
    return x;
}

kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const int32_t* cu_seqlens, int B, int T, int H, int Dk, int Dv,
                          int num_seqs, int chunk, kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                          void* workspace, size_t workspace_bytes, kda_stream_t stream, bool scalar_gate,
                          const kda_fusion* fusion = nullptr) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || num_seqs < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_ok(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::chunk_supported(chunk)) return KDA_ERR_UNSUPPORTED;
    if (!fusion_ok(fusion)) return KDA_ERR_INVALID_ARGUMENT;
    const bool fused = fusion && (fusion->flags || fusion->out_gate);
    if ((scalar_gate || fused) && chunk != 0 && chunk != 32) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARGUMENT;
    } else if (num_seqs != B) {
        return KDA_ERR_INVALID_ARGUMENT;
    }
    const size_t tokens = static_cast<size_t>(B) * static_cast<size_t>(T);
    if (tokens > 0 && num_seqs > 0) {
        if (!q || !k || !v || !log_alpha || !beta || !o) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(o))
            return KDA_ERR_INVALID_ARGUMENT;
        // beta rows are [B, T, H]: 16-byte alignment of the base is enough for the
        // kernels' scalar reads, but keep the documented contract uniform.
        if (!aligned16(beta)) return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return KDA_ERR_INVALID_ARGUMENT;

    const size_t ein = elem_size(in_dtype), eout = elem_size(out_dtype);
    const size_t n_qk = tokens * H * Dk * ein, n_v = tokens * H * Dv * ein, n_b = tokens * H * ein;
    const size_t n_g = scalar_gate ? n_b : n_qk;
    const size_t n_o = tokens * H * Dv * eout;
    const size_t n_s = static_cast<size_t>(num_seqs) * H * Dk * Dv * sizeof(float);
    if (tokens > 0) {
        const void* ins[5] = {q, k, v, log_alpha, beta};
        const size_t nin[5] = {n_qk, n_qk, n_v, n_g, n_b};
        for (int i = 0; i < 5; ++i)
            if (overlap(ins[i], nin[i], o, n_o) || overlap(ins[i], nin[i], S_final, n_s))
                return KDA_ERR_INVALID_ARGUMENT;
        if (fused && fusion->out_gate) {
            const size_t n_gate = tokens * H * Dv * ein;
            if (overlap(fusion->out_gate, n_gate, o, n_o) || overlap(fusion->out_gate, n_gate, S_final, n_s))
                return KDA_ERR_INVALID_ARGUMENT;
        }
    }
    if (overlap(S0, n_s, S_final, n_s) || overlap(S0, n_s, o, n_o) || overlap(o, n_o, S_final, n_s))
        return KDA_ERR_INVALID_ARGUMENT;

    kda::PrefillPlan plan = kda::plan_prefill(B, T, H, Dk, num_seqs, cu_seqlens != nullptr, chunk);
    if (workspace_bytes < plan.workspace_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (plan.workspace_bytes > 0 && (!workspace || !aligned16(workspace))) return KDA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return KDA_OK;
    if (overlap(workspace, plan.workspace_bytes, o, n_o) || overlap(workspace, plan.workspace_bytes, S_final, n_s))
        return KDA_ERR_INVALID_ARGUMENT;

    // A batch of equal-length sequences of at most kRecurrentMaxT tokens (new tokens on top of a
    // carried state) runs token by token with the state on chip: a chunk would be mostly padding.
    if (!cu_seqlens && T > 0 && T <= kda::kRecurrentMaxT && !fused) {
        const size_t units = static_cast<size_t>(B) * H;
        if (units > 0x7fffffffu) return KDA_ERR_UNSUPPORTED;
        hipError_t err = kda::launch_recurrent_fwd(Dk, in_dtype == KDA_BF16, out_dtype == KDA_BF16, q, k, v,
                                                   log_alpha, beta, S0, nullptr, T, H, static_cast<int>(units), o,
                                                   S_final, reinterpret_cast<hipStream_t>(stream), scalar_gate);
        return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.beta = beta;
    a.S0 = S0; a.cu = cu_seqlens; a.o = o; a.S_final = S_final;
    a.B = B; a.T = T; a.H = H; a.D = Dk; a.N = num_seqs;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.scalar_gate = scalar_gate;
    const kda::Fusion fz = to_fusion(fused ? fusion : nullptr);
    a.fuse_flags = fz.flags;
    a.decay_bias = fz.decay_bias;
    a.decay_scale = fz.decay_scale;
    a.out_gate = fz.out_gate;
    a.workspace = workspace;
    hipError_t err = kda::launch_prefill(a, plan, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status recurrent_step_impl(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S_in, float* S_out, int N, int H, int Dk, int Dv,
                               kda_dtype in_dtype, kda_dtype out_dtype, void* o, kda_stream_t stream,
                               bool scalar_gate, const kda_fusion* fusion = nullptr) {
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_ok(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
    if (!fusion_ok(fusion)) return KDA_ERR_INVALID_ARGUMENT;
    const bool fused = fusion && (fusion->flags || fusion->out_gate);
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S_in || !S_out || !o) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(beta) ||
        !aligned16(S_in) || !aligned16(S_out) || !aligned16(o))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t units = static_cast<size_t>(N) * H;
    const size_t ein = elem_size(in_dtype), eout = elem_size(out_dtype);
    const size_t n_s = units * Dk * Dv * sizeof(float), n_o = units * Dv * eout;
    if (S_in != S_out && overlap(S_in, n_s, S_out, n_s)) return KDA_ERR_INVALID_ARGUMENT;
    const void* ins[5] = {q, k, v, log_alpha, beta};
    const size_t nin[5] = {units * Dk * ein, units * Dk * ein, units * Dv * ein,
                           scalar_gate ? units * ein : units * Dk * ein, units * ein};
    for (int i = 0; i < 5; ++i)
        if (overlap(ins[i], nin[i], S_out, n_s) || overlap(ins[i], nin[i], o, n_o)) return KDA_ERR_INVALID_ARGUMENT;
    if (overlap(o, n_o, S_out, n_s) || overlap(o, n_o, S_in, n_s)) return KDA_ERR_INVALID_ARGUMENT;
    if (fused && fusion->out_gate) {
        const size_t n_gate = units * Dv * ein;
        if (overlap(fusion->out_gate, n_gate, o, n_o) || overlap(fusion->out_gate, n_gate, S_out, n_s))
            return KDA_ERR_INVALID_ARGUMENT;
    }
    if (units > 0x7fffffffu) return KDA_ERR_UNSUPPORTED;

    const kda::Fusion fz = to_fusion(fused ? fusion : nullptr);
    hipError_t err = kda::launch_decode(Dk, in_dtype == KDA_BF16, out_dtype == KDA_BF16, q, k, v, log_alpha,
                                        beta, S_in, S_out, o, static_cast<int>(units),
                                        reinterpret_cast<hipStream_t>(stream), scalar_gate, fused ? &fz : nullptr);
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status recurrent_fwd_impl(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                              const float* S0, const int32_t* cu_seqlens, int B, int T, int H, int Dk, int Dv,
                              int num_seqs, kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                              kda_stream_t stream, bool scalar_gate) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || num_seqs < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_ok(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens) {
        if (B != 1 || !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARGUMENT;
    } else if (num_seqs != B) {
        return KDA_ERR_INVALID_ARGUMENT;
    }
    const size_t tokens = static_cast<size_t>(B) * static_cast<size_t>(T);
    if (tokens > 0 && num_seqs > 0) {
        if (!q || !k || !v || !log_alpha || !beta || !o) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(beta) ||
            !aligned16(o))
            return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ein = elem_size(in_dtype), eout = elem_size(out_dtype);
    const size_t n_qk = tokens * H * Dk * ein, n_v = tokens * H * Dv * ein, n_b = tokens * H * ein;
    const size_t n_g = scalar_gate ? n_b : n_qk;
    const size_t n_o = tokens * H * Dv * eout;
    const size_t n_s = static_cast<size_t>(num_seqs) * H * Dk * Dv * sizeof(float);
    if (tokens > 0) {
        const void* ins[5] = {q, k, v, log_alpha, beta};
        const size_t nin[5] = {n_qk, n_qk, n_v, n_g, n_b};
        for (int i = 0; i < 5; ++i)
            if (overlap(ins[i], nin[i], o, n_o) || overlap(ins[i], nin[i], S_final, n_s))
                return KDA_ERR_INVALID_ARGUMENT;
    }
    // S_final == S0 (in place) is allowed; any other overlap is not
    if ((S0 != S_final && overlap(S0, n_s, S_final, n_s)) || overlap(S0, n_s, o, n_o) ||
        overlap(o, n_o, S_final, n_s))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t units = static_cast<size_t>(num_seqs) * H;
    if (units == 0) return KDA_OK;
    if (units > 0x7fffffffu) return KDA_ERR_UNSUPPORTED;
    hipError_t err = kda::launch_recurrent_fwd(Dk, in_dtype == KDA_BF16, out_dtype == KDA_BF16, q, k, v, log_alpha,
                                               beta, S0, cu_seqlens, T, H, static_cast<int>(units), o, S_final,
                                               reinterpret_cast<hipStream_t>(stream), scalar_gate);
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                    kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                                    void* workspace, size_t workspace_bytes, kda_stream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, chunk, in_dtype,
                          out_dtype, o, S_final, workspace, workspace_bytes, stream, false);
}

extern "C" kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* log_alpha,
                                         const void* beta, const float* S_in, float* S_out,
                                         int N, int H, int Dk, int Dv,
                                         kda_dtype in_dtype, kda_dtype out_dtype,
                                         void* o, kda_stream_t stream) {
    return recurrent_step_impl(q, k, v, log_alpha, beta, S_in, S_out, N, H, Dk, Dv, in_dtype, out_dtype, o, stream,
                               false);
}

extern "C" kda_status kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                        const void* beta, const float* S0, const int32_t* cu_seqlens,
                                        int B, int T, int H, int Dk, int Dv, int num_seqs,
                                        kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                                        kda_stream_t stream) {
    return recurrent_fwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, in_dtype,
                              out_dtype, o, S_final, stream, false);
}

extern "C" kda_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                    kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                                    void* workspace, size_t workspace_bytes, kda_stream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, chunk, in_dtype,
                          out_dtype, o, S_final, workspace, workspace_bytes, stream, true);
}

extern "C" kda_status gdn_recurrent_step(const void* q, const void* k, const void* v, const void* log_alpha,
                                         const void* beta, const float* S_in, float* S_out,
                                         int N, int H, int Dk, int Dv,
                                         kda_dtype in_dtype, kda_dtype out_dtype,
                                         void* o, kda_stream_t stream) {
    return recurrent_step_impl(q, k, v, log_alpha, beta, S_in, S_out, N, H, Dk, Dv, in_dtype, out_dtype, o, stream,
                               true);
}

extern "C" kda_status gdn_recurrent_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                        const void* beta, const float* S0, const int32_t* cu_seqlens,
                                        int B, int T, int H, int Dk, int Dv, int num_seqs,
                                        kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                                        kda_stream_t stream) {
    return recurrent_fwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, in_dtype,
                              out_dtype, o, S_final, stream, true);
}

extern "C" kda_status kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                          const void* beta, const float* S0, const int32_t* cu_seqlens,
                                          int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                          kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* S_final,
                                          void* workspace, size_t workspace_bytes, const kda_fusion* fusion,
                                          kda_stream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, B, T, H, Dk, Dv, num_seqs, chunk, in_dtype,
                          out_dtype, o, S_final, workspace, workspace_bytes, stream, false, fusion);
}

extern "C" kda_status kda_recurrent_step_fused(const void* q, const void* k, const void* v, const void* log_alpha,
                                               const void* beta, const float* S_in, float* S_out,
                                               int N, int H, int Dk, int Dv,
                                               kda_dtype in_dtype, kda_dtype out_dtype,
                                               void* o, const kda_fusion* fusion, kda_stream_t stream) {
    return recurrent_step_impl(q, k, v, log_alpha, beta, S_in, S_out, N, H, Dk, Dv, in_dtype, out_dtype, o, stream,
                               false, fusion);
}

extern "C" size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                                int has_cu_seqlens, int chunk) {
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0 || !head_ok(Dk, Dv)) return 0;
    if (chunk != 0 && chunk != 32) return 0;
    return kda::plan_backward(B, T, H, Dk, num_seqs, has_cu_seqlens != 0).workspace_bytes;
}

namespace {

kda_status chunk_bwd_impl(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const int32_t* cu_seqlens, const void* d_o, const float* dS_final,
                          int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk, kda_dtype in_dtype,
                          kda_dtype grad_dtype, void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta,
                          float* dS0, void* workspace, size_t workspace_bytes, kda_stream_t stream,
                          bool scalar_gate) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || num_seqs < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(in_dtype) || !dtype_ok(grad_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_ok(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 0 && chunk != 32) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens) {
        if (B != 1 || !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARGUMENT;
    } else if (num_seqs != B) {
        return KDA_ERR_INVALID_ARGUMENT;
    }
    const size_t tokens = static_cast<size_t>(B) * static_cast<size_t>(T);
    const bool work = tokens > 0 && num_seqs > 0;
    const void* ins[6] = {q, k, v, log_alpha, beta, d_o};
    void* outs[5] = {dq, dk, dv, dlog_alpha, dbeta};
    if (work) {
        for (const void* x : ins)
            if (!x || !aligned16(x)) return KDA_ERR_INVALID_ARGUMENT;
        for (const void* x : outs)
            if (!x || !aligned16(x)) return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)))
        return KDA_ERR_INVALID_ARGUMENT;

    const size_t ein = elem_size(in_dtype), eg = elem_size(grad_dtype);
    const size_t n_x = tokens * H * Dk, n_b = tokens * H;
    const size_t n_s = static_cast<size_t>(num_seqs) * H * Dk * Dv * sizeof(float);
    const size_t n_g = scalar_gate ? n_b : n_x;   // log_alpha and dlog_alpha
    const size_t nin[6] = {n_x * ein, n_x * ein, n_x * ein, n_g * ein, n_b * ein, n_x * ein};
    const size_t nout[5] = {n_x * eg, n_x * eg, n_x * eg, n_g * eg, n_b * eg};
    kda::BackwardPlan plan = kda::plan_backward(B, T, H, Dk, num_seqs, cu_seqlens != nullptr);
    // every output is disjoint from every input, from the other outputs and from the workspace
    for (int o = 0; o < 6; ++o) {
        const void* po = o < 5 ? outs[o] : dS0;
        const size_t no = o < 5 ? (work ? nout[o] : 0) : n_s;
        for (int i = 0; i < 6; ++i)
            if (overlap(ins[i], work ? nin[i] : 0, po, no)) return KDA_ERR_INVALID_ARGUMENT;
        if (overlap(S0, n_s, po, no) || overlap(dS_final, n_s, po, no)) return KDA_ERR_INVALID_ARGUMENT;
        for (int o2 = o + 1; o2 < 6; ++o2) {
            const void* p2 = o2 < 5 ? outs[o2] : dS0;
            const size_t n2 = o2 < 5 ? (work ? nout[o2] : 0) : n_s;
            if (overlap(po, no, p2, n2)) return KDA_ERR_INVALID_ARGUMENT;
        }
        if (overlap(workspace, plan.workspace_bytes, po, no)) return KDA_ERR_INVALID_ARGUMENT;
    }
    if (workspace_bytes < plan.workspace_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (plan.workspace_bytes > 0 && (!workspace || !aligned16(workspace))) return KDA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return KDA_OK;
    // grid sizes and token indices are 32-bit on the device
    const size_t units = static_cast<size_t>(num_seqs) * H;
    if (plan.nc_max * H > 0x7fffffffu || units * (Dk / 16) > 0x7fffffffu || tokens > 0x7fffffffu)
        return KDA_ERR_UNSUPPORTED;

    kda::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.beta = beta; a.dO = d_o;
    a.S0 = S0; a.dS_final = dS_final; a.cu = cu_seqlens;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dlog_alpha; a.dbeta = dbeta; a.dS0 = dS0;
    a.B = B; a.T = T; a.H = H; a.D = Dk; a.N = num_seqs;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = grad_dtype == KDA_BF16;
    a.scalar_gate = scalar_gate;
    hipError_t err = kda::launch_backward(a, plan, workspace, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    const void* d_o, const float* dS_final,
                                    int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                    kda_dtype in_dtype, kda_dtype grad_dtype,
                                    void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                                    void* workspace, size_t workspace_bytes, kda_stream_t stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, dS_final, B, T, H, Dk, Dv, num_seqs,
                          chunk, in_dtype, grad_dtype, dq, dk, dv, dlog_alpha, dbeta, dS0, workspace,
                          workspace_bytes, stream, false);
}

extern "C" kda_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    const void* d_o, const float* dS_final,
                                    int B, int T, int H, int Dk, int Dv, int num_seqs, int chunk,
                                    kda_dtype in_dtype, kda_dtype grad_dtype,
                                    void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta, float* dS0,
                                    void* workspace, size_t workspace_bytes, kda_stream_t stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, dS_final, B, T, H, Dk, Dv, num_seqs,
                          chunk, in_dtype, grad_dtype, dq, dk, dv, dlog_alpha, dbeta, dS0, workspace,
                          workspace_bytes, stream, true);
}
