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

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two fp32 values -> packed bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Low-bit cache codes: OCP 8-bit float E4M3 (bit 7 sign, 4 exponent bits with
// bias 7, 3 mantissa bits; no infinities).  Encoding rounds to nearest, ties
// to even, and saturates at +-448 (the hardware conversion rounds the same
// way but turns overflow into NaN, hence the clamp); decoding is exact, and
// every code's value is also exactly a bf16 value.
__device__ __forceinline__ float e4m3_clamp(float v) { return fminf(fmaxf(v, -448.f), 448.f); }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return (uint32_t)w;
}
// eight codes (two words, code k in byte k % 4 of word k / 4) -> bf16x8
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    u32x4 u;
    u[0] = pack_bf16x2(a[0], a[1]);
    u[1] = pack_bf16x2(b[0], b[1]);
    u[2] = pack_bf16x2(c[0], c[1]);
    u[3] = pack_bf16x2(d[0], d[1]);
    return __builtin_bit_cast(bf16x8, u);
}

// Sum over the 16 lanes of each row of the wave (lanes 16r .. 16r+15); every
// lane of the row receives the sum.  Four DPP adds, no LDS traffic.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)); // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)); // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
    return v;
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


// s_waitcnt immediate: vector-memory count vm, LDS/scalar count lgkm, no wait
// on the export counter
__device__ __forceinline__ constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS copies issued from inline assembly: lane i's bytes land at
// LDS byte address base + size * i (base wave-uniform).  The compiler does
// not see these loads, so it adds no waits for them: the caller orders them
// with explicit s_waitcnt and barriers; the memory clobber keeps LDS reads
// from moving across a copy.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(base) : "memory", "m0");
}
// The same with the non-temporal hint, for data read once: the lines do not
// displace what the caches hold for data that is read again.
__device__ __forceinline__ void copy16_to_lds_nt(const void* gptr, uint32_t base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(gptr), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void* gptr, uint32_t base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(gptr), "s"(base) : "memory", "m0");
}

// A 16-byte load the compiler does not track (so it adds no wait for it, and
// counts none of it in the waits it adds): the caller waits with an explicit
// s_waitcnt and then passes the value through fence_value() before using it.
// Nothing stops the register allocator from copying the destination before
// that wait; a build-time walk over the generated assembly checks, on every
// control-flow path, that no instruction touches the destination registers
// before a wait that covers the load.
__device__ __forceinline__ u32x4 load_untracked_x4(const void* p) {
    u32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
    return v;
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Keeps later uses of v from being scheduled above the preceding wait.
__device__ __forceinline__ u32x4 fence_value(u32x4 v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Workgroup barrier that orders LDS only: the fences wait for this wave's
// LDS operations, not for its global loads in flight (a plain __syncthreads
// would drain those too).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tuning overrides (tuning.hip): the forced attention split count (0 =
// automatic) and the forced projection kernel name (nullptr = automatic),
// from DLLM_ATTN_SPLITS / DLLM_QKV_KERNEL read once per process, or from
// dllm_set_tuning.
int tuning_attn_splits();
const char* tuning_qkv_kernel();

}  // namespace dllm

#define DLLM_CHECK_ARG(cond) \
    do { if (!(cond)) return DLLM_ERR_INVALID_ARG; } while (0)
#define DLLM_CHECK_SUP(cond) \
    do { if (!(cond)) return DLLM_ERR_UNSUPPORTED; } while (0)
#define DLLM_CHECK_LAUNCH() \
    do { if (hipGetLastError() != hipSuccess) return DLLM_ERR_HIP; } while (0)
