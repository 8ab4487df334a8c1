// kda_device.h -- small device helpers shared by the KDA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// ---------------------------------------------------------------- element types
// Inputs arrive as fp32 or bf16 (carried as raw 16-bit patterns).
struct F32 {
    using storage = float;
    static __device__ __forceinline__ float to_f32(float x) { return x; }
};
struct BF16 {
    using storage = uint16_t;
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return __uint_as_float(static_cast<uint32_t>(x) << 16);
    }
};

// Output stores: fp32 or bf16 (round to nearest even, the hardware conversion of gfx950).
template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* base, size_t idx, float x) {
    if constexpr (OUT_BF16) static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(x);
    else static_cast<float*>(base)[idx] = x;
}

// exp(x) on the hardware exp2 unit (v_exp_f32) with a log2(e) pre-scale.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace kda
