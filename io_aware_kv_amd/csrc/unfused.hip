// The unfused comparison arm of a1-a3: the rotary embedding and the cache
// write as launches of their own, after a projection that leaves unrotated
// q|k|v rows in HBM (dllm_qkv_project).
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page).  研究动机: the
// four-kernel chain (projection, rotary, cache write, attention) moves every
// intermediate through global memory; 核心方法: the fused kernel removes those
// round trips.  This arm exists to measure that difference on MI355X with the
// same projection kernels (their epilogue reduced to a plain row store).
//
// Both kernels are memory-bound elementwise passes: 16-byte loads and stores,
// one thread per 8 rotation pairs (rotary) or per 16-byte piece (cache write).
#include <math.h>

#include "common.h"

namespace {

using namespace dllm;

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr int kThreadsU = 256;

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
        f[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
    }
}

// one thread per (row, q or k, head, piece of 8 rotation pairs): q rotated
// into q_out [R, n_out], k rotated in place inside qkv [R, 3 n_out]
__global__ __launch_bounds__(kThreadsU) void rope_kernel(int R, int n_heads, int head_dim,
                                                         float rope_base, const int32_t* __restrict__ pos,
                                                         uint16_t* qkv, uint16_t* __restrict__ q_out) {
    const int half = head_dim / 2, pieces = half / 8;
    const int n_out = n_heads * head_dim;
    const int64_t total = (int64_t)R * 2 * n_heads * pieces;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int pc = (int)(idx % pieces);
    const int h = (int)((idx / pieces) % n_heads);
    const int part = (int)((idx / ((int64_t)pieces * n_heads)) % 2);
    const int64_t r = idx / ((int64_t)pieces * n_heads * 2);
    uint16_t* src = qkv + r * 3 * n_out + part * n_out + h * head_dim + pc * 8;
    float lo[8], hi[8];
    unpack8(*(const u32x4*)src, lo);
    unpack8(*(const u32x4*)(src + half), hi);
    const double p = (double)pos[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = pc * 8 + e;
        double ang = p * pow((double)rope_base, -2.0 * i / head_dim);
        ang -= rint(ang * (1.0 / kTwoPi)) * kTwoPi;
        // hardware sin/cos take revolutions; |rev| <= 1/2 after the fp64 reduction
        const float rev = (float)(ang * (1.0 / kTwoPi));
        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
        const float x0 = lo[e], x1 = hi[e];
        lo[e] = x0 * cs - x1 * sn;
        hi[e] = x1 * cs + x0 * sn;
    }
    u32x4 plo, phi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        plo[e] = pack_bf16x2(lo[2 * e], lo[2 * e + 1]);
        phi[e] = pack_bf16x2(hi[2 * e], hi[2 * e + 1]);
    }
    uint16_t* dst = part == 0 ? q_out + r * n_out + h * head_dim + pc * 8 : src;
    *(u32x4*)dst = plo;
    *(u32x4*)(dst + half) = phi;
}

// one thread per (row, k or v, 16-byte piece): the row's k|v part of qkv to
// its cache slot (rows with a slot outside the cache are skipped)
__global__ __launch_bounds__(kThreadsU) void cache_write_kernel(int R, int n_out,
                                                                const uint16_t* __restrict__ qkv,
                                                                const int32_t* __restrict__ slot,
                                                                uint16_t* __restrict__ k_cache,
                                                                uint16_t* __restrict__ v_cache,
                                                                int64_t cache_rows) {
    const int pieces = n_out / 8;
    const int64_t total = (int64_t)R * 2 * pieces;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % pieces);
    const int part = (int)((idx / pieces) % 2);
    const int64_t r = idx / ((int64_t)pieces * 2);
    const int s = slot[r];
    if (s < 0 || (int64_t)s >= cache_rows) return;
    const u32x4 v = *(const u32x4*)(qkv + r * 3 * n_out + (1 + part) * n_out + c * 8);
    *(u32x4*)((part == 0 ? k_cache : v_cache) + (int64_t)s * n_out + c * 8) = v;
}

}  // namespace

extern "C" int dllm_rope_apply(dllm_dtype dt, int n_rows, int n_heads, int head_dim, float rope_base,
                               const int32_t* pos, void* qkv, void* q_out, hipStream_t stream) {
    DLLM_CHECK_ARG(n_rows >= 0 && n_heads > 0 && head_dim > 0 && rope_base > 0.f);
    DLLM_CHECK_SUP(dt == DLLM_BF16 && (head_dim == 64 || head_dim == 128));
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(pos && qkv && q_out);
    const int64_t total = (int64_t)n_rows * 2 * n_heads * (head_dim / 16);
    const int64_t blocks = (total + kThreadsU - 1) / kThreadsU;
    DLLM_CHECK_SUP(blocks < (1ll << 31));
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kThreadsU), 0, stream, n_rows, n_heads,
                       head_dim, rope_base, pos, (uint16_t*)qkv, (uint16_t*)q_out);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

extern "C" int dllm_cache_write(dllm_dtype dt, int n_rows, int n_heads, int head_dim, const void* qkv,
                                const int32_t* slot, void* k_cache, void* v_cache, int64_t cache_rows,
                                hipStream_t stream) {
    DLLM_CHECK_ARG(n_rows >= 0 && n_heads > 0 && head_dim > 0 && cache_rows >= 0);
    DLLM_CHECK_SUP(dt == DLLM_BF16 && (n_heads * head_dim) % 8 == 0);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(qkv && slot && k_cache && v_cache);
    const int n_out = n_heads * head_dim;
    const int64_t total = (int64_t)n_rows * 2 * (n_out / 8);
    const int64_t blocks = (total + kThreadsU - 1) / kThreadsU;
    DLLM_CHECK_SUP(blocks < (1ll << 31));
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreadsU), 0, stream, n_rows, n_out,
                       (const uint16_t*)qkv, slot, (uint16_t*)k_cache, (uint16_t*)v_cache, cache_rows);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
