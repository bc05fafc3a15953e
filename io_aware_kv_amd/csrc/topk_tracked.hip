// a6: per-sequence top-k of the tracked-set score.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page), 方法步骤详情 step 4:
// the k decoded tokens with the largest formula-(2) score, together with the
// newly decoded ones, are the next step's tracked set.
//
// One workgroup per sequence.  The score of position i is the sum over heads
// (ascending head order, fp32) of the per-head accumulators the attention
// kernel wrote.  Selection is a radix select rather than a sort: each
// candidate's score becomes a 32-bit key that orders scores descending, and
// four 8-bit histogram passes (LDS) find the k-th smallest key T.  Keys below
// T are taken; among keys equal to T the lowest positions are taken (one block
// scan in position order), which is the tie rule of the sorted order.  The at
// most k taken entries are then placed by counting rank over (key, position),
// so the output runs from the highest score down, ties towards the lower
// position.  About a dozen barriers, against ~45 for a bitonic sort of 512.
#include "common.h"

namespace {

constexpr int kThreads = 512;
constexpr int kMaxCap = 4096;
constexpr int kMaxK = 256;

__device__ __forceinline__ uint32_t order_desc(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in f
    return ~asc;                                                  // descending in f
}

// exclusive block scan of one int per thread (512 threads, 8 waves)
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(x, off);
        if (lane >= off) x += t;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const int c = s_wave[w];
        base += w < wave ? c : 0;
        tot += c;
    }
    total = tot;
    __syncthreads();                                      // s_wave is free for the next scan
    return base + x - v;
}

template <int kPer>   // positions per thread (contiguous), kPer * kThreads >= n_cap
__global__ __launch_bounds__(kThreads) void topk_kernel(int n_heads, int n_cap, int k, float* mass,
                                                        const uint8_t* eligible, int32_t* idx,
                                                        float* val, int32_t* count,
                                                        int clear_mass) {
    __shared__ int hist[2][256];
    __shared__ int s_wave[kThreads / 64];
    __shared__ uint32_t s_prefix, s_krem;
    __shared__ uint32_t sel_key[kMaxK];
    __shared__ int sel_idx[kMaxK];
    __shared__ float sel_val[kMaxK];
    __shared__ int s_nsel;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    float* mseq = mass + (int64_t)b * n_heads * n_cap;
    const uint8_t* erow = eligible + (int64_t)b * n_cap;
    const int per = kPer;
    const int i0 = tid * per;

    // ---- scores of this thread's positions i0 .. i0 + per - 1 ----
    float sc[kPer];
    uint32_t key[kPer];
    bool cand[kPer];
    int ncand = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        sc[e] = 0.f;
        cand[e] = false;
        key[e] = 0xffffffffu;
    }
    // heads in groups of kGroup: the group's loads are independent and in
    // flight together (a plain running sum would serialise every load), then
    // added in ascending head order
    constexpr int kGroup = 32 / kPer;
    const int nvalid = max(0, min(per, n_cap - i0));
    for (int h0 = 0; h0 < n_heads; h0 += kGroup) {
        float v[kGroup][kPer];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const int hh = min(h0 + j, n_heads - 1);
            const float* mh = mseq + (int64_t)hh * n_cap + min(i0, n_cap - 1);
#pragma unroll
            for (int e = 0; e < kPer; ++e) v[j][e] = mh[min(e, max(nvalid - 1, 0))];
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (h0 + j < n_heads && e < nvalid) sc[e] += v[j][e];
    }
    if (clear_mass) {                                     // this thread's entries only: no hazard
        for (int hh = 0; hh < n_heads; ++hh) {
            float* mh = mseq + (int64_t)hh * n_cap;
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (e < per && i0 + e < n_cap) mh[i0 + e] = 0.f;
        }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        if (e < per && i0 + e < n_cap && erow[i0 + e]) {
            cand[e] = true;
            key[e] = order_desc(sc[e]);
            ++ncand;
        }
    }
    int total_cand;
    (void)block_exclusive_scan(ncand, s_wave, total_cand);
    const int kk = min(k, total_cand);

    // ---- radix select: the kk-th smallest key T (kk >= 1), 8 bits at a time ----
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)kk;
    if (kk > 0 && kk < total_cand) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            int* h = hist[pass & 1];
            for (int j = tid; j < 256; j += kThreads) h[j] = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (cand[e] && (key[e] & pmask) == prefix) atomicAdd(&h[(key[e] >> shift) & 255u], 1);
            __syncthreads();
            if (tid < 64) {
                // lane l owns bins 4l .. 4l+3; find the bin where the running count reaches krem
                int c[4], run = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) c[q] = h[4 * lane + q];
                const int own = c[0] + c[1] + c[2] + c[3];
                int incl = own;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t = __shfl_up(incl, off);
                    if (lane >= off) incl += t;
                }
                const int excl = incl - own;
                // the lane whose range holds the krem-th element
                const bool mine = excl < (int)krem && (int)krem <= incl;
                if (mine) {
                    run = excl;
                    int bin = 4 * lane;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (run + c[q] >= (int)krem) { bin = 4 * lane + q; break; }
                        run += c[q];
                    }
                    s_prefix = prefix | ((uint32_t)bin << shift);
                    s_krem = krem - (uint32_t)run;
                }
            }
            __syncthreads();
            prefix = s_prefix;
            krem = s_krem;
            pmask |= 0xffu << shift;
        }
    }
    // kk == total_cand: every candidate is taken (T above every key)
    const uint32_t T = (kk < total_cand && kk > 0) ? prefix : 0xffffffffu;
    const bool take_all = !(kk < total_cand && kk > 0);

    // ---- take keys < T, and the lowest positions among keys == T ----
    int neq = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) neq += (cand[e] && key[e] == T && !take_all) ? 1 : 0;
    int neq_total;
    int eq_rank = block_exclusive_scan(neq, s_wave, neq_total);
    if (tid == 0) s_nsel = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        if (!cand[e]) continue;
        bool take = take_all || key[e] < T;
        if (!take_all && key[e] == T) {
            take = eq_rank < (int)krem;
            ++eq_rank;
        }
        if (take && kk > 0) {
            const int slot = atomicAdd(&s_nsel, 1);
            if (slot < kMaxK) {
                sel_key[slot] = key[e];
                sel_idx[slot] = i0 + e;
                sel_val[slot] = sc[e];
            }
        }
    }
    __syncthreads();
    const int nsel = min(s_nsel, kk);
    // ---- order by (key, position): counting rank ----
    for (int j = tid; j < nsel; j += kThreads) {
        const uint32_t kj = sel_key[j];
        const int ij = sel_idx[j];
        int rank = 0;
        for (int i = 0; i < nsel; ++i) {
            const uint32_t ki = sel_key[i];
            rank += (ki < kj || (ki == kj && sel_idx[i] < ij)) ? 1 : 0;
        }
        idx[(int64_t)b * k + rank] = ij;
        val[(int64_t)b * k + rank] = sel_val[j];
    }
    for (int j = nsel + tid; j < k; j += kThreads) {
        idx[(int64_t)b * k + j] = -1;
        val[(int64_t)b * k + j] = 0.f;
    }
    if (tid == 0) count[b] = nsel;
    (void)lane;
}

}  // namespace

extern "C" int dllm_topk_tracked(int n_seq, int n_heads, int n_cap, int k, float* mass,
                                 const uint8_t* eligible, int32_t* idx, float* val, int32_t* count,
                                 int clear_mass, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq > 0 && n_heads > 0 && n_cap > 0 && k > 0);
    DLLM_CHECK_SUP(k <= kMaxK && n_cap <= kMaxCap);
    DLLM_CHECK_ARG(mass && eligible && idx && val && count);
    const int per = (n_cap + kThreads - 1) / kThreads;
    if (per <= 1)
        hipLaunchKernelGGL(topk_kernel<1>, dim3(n_seq), dim3(kThreads), 0, stream, n_heads, n_cap, k, mass,
                           eligible, idx, val, count, clear_mass);
    else if (per <= 2)
        hipLaunchKernelGGL(topk_kernel<2>, dim3(n_seq), dim3(kThreads), 0, stream, n_heads, n_cap, k, mass,
                           eligible, idx, val, count, clear_mass);
    else if (per <= 4)
        hipLaunchKernelGGL(topk_kernel<4>, dim3(n_seq), dim3(kThreads), 0, stream, n_heads, n_cap, k, mass,
                           eligible, idx, val, count, clear_mass);
    else
        hipLaunchKernelGGL(topk_kernel<8>, dim3(n_seq), dim3(kThreads), 0, stream, n_heads, n_cap, k, mass,
                           eligible, idx, val, count, clear_mass);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
