// a6: per-sequence top-k of the tracked-set score.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page), 方法步骤详情 step 4:
// the k decoded tokens with the largest formula-(2) score, together with the
// newly decoded ones, are the next step's tracked set.
//
// One workgroup per sequence.  The score of position i is the sum over heads
// (ascending head order, fp32) of the per-head accumulators the attention
// kernel wrote.  Each candidate becomes a 64-bit key whose high
// word orders scores descending and whose low word is the position, so an
// ascending bitonic sort in LDS yields scores high-to-low with ties broken
// towards the lower position; non-candidates sort last.
#include "common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxCap = 4096;
constexpr int kMaxK = 256;

__device__ __forceinline__ uint32_t order_desc(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in f
    return ~asc;                                                  // descending in f
}

__global__ __launch_bounds__(kThreads) void topk_kernel(int n_heads, int n_cap, int k, float* mass,
                                                        const uint8_t* eligible, int32_t* idx,
                                                        float* val, int32_t* count,
                                                        int clear_mass) {
    __shared__ uint64_t keys[kMaxCap];
    __shared__ float score[kMaxCap];
    __shared__ int s_cnt;
    const int b = blockIdx.x, tid = threadIdx.x;
    float* mseq = mass + (int64_t)b * n_heads * n_cap;
    const uint8_t* erow = eligible + (int64_t)b * n_cap;
    int n2 = 1;
    while (n2 < n_cap) n2 <<= 1;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    int local = 0;
    for (int i = tid; i < n2; i += kThreads) {
        uint64_t key = ~0ull;
        if (i < n_cap) {
            float sc = 0.f;
            for (int hh = 0; hh < n_heads; ++hh) sc += mseq[(int64_t)hh * n_cap + i];
            score[i] = sc;
            if (erow[i]) {
                key = ((uint64_t)order_desc(sc) << 32) | (uint32_t)i;
                ++local;
            }
        }
        keys[i] = key;
    }
    atomicAdd(&s_cnt, local);
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n2 / 2; i += kThreads) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;
                uint64_t x = keys[lo], y = keys[hi];
                if ((x > y) == up) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    const int n = min(k, s_cnt);
    for (int j = tid; j < k; j += kThreads) {
        if (j < n) {
            int pos = (int)(keys[j] & 0xffffffffu);
            idx[(int64_t)b * k + j] = pos;
            val[(int64_t)b * k + j] = score[pos];
        } else {
            idx[(int64_t)b * k + j] = -1;
            val[(int64_t)b * k + j] = 0.f;
        }
    }
    if (tid == 0) count[b] = n;
    if (clear_mass) {
        __syncthreads();
        for (int i = tid; i < n_heads * n_cap; i += kThreads) mseq[i] = 0.f;
    }
}

}  // namespace

extern "C" int dllm_topk_tracked(int n_seq, int n_heads, int n_cap, int k, float* mass,
                                 const uint8_t* eligible, int32_t* idx, float* val, int32_t* count,
                                 int clear_mass, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq > 0 && n_heads > 0 && n_cap > 0 && k > 0);
    DLLM_CHECK_SUP(k <= kMaxK && n_cap <= kMaxCap);
    DLLM_CHECK_ARG(mass && eligible && idx && val && count);
    hipLaunchKernelGGL(topk_kernel, dim3(n_seq), dim3(kThreads), 0, stream, n_heads, n_cap, k, mass,
                       eligible, idx, val, count, clear_mass);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
