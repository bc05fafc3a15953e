// Internal helpers of the dllm library (device types, conversions, host checks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm.h"

namespace dllm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// MI355X: 256 compute units in 8 accelerator dies (XCDs), each with its own L2.
constexpr int kNumXcd = 8;
constexpr int kNumCu = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (finite values; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Map a launch index to a logical work index so that consecutive logical
// items land on the same XCD (hardware dispatches workgroup i to XCD i % 8).
// Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    int x = bid % kNumXcd;
    int j = bid / kNumXcd;
    int per = total / kNumXcd;
    int extra = total % kNumXcd;
    return x * per + (x < extra ? x : extra) + j;
}

}  // namespace dllm

#define DLLM_CHECK_ARG(cond) \
    do { if (!(cond)) return DLLM_ERR_INVALID_ARG; } while (0)
#define DLLM_CHECK_SUP(cond) \
    do { if (!(cond)) return DLLM_ERR_UNSUPPORTED; } while (0)
#define DLLM_CHECK_LAUNCH() \
    do { if (hipGetLastError() != hipSuccess) return DLLM_ERR_HIP; } while (0)
