// a6: per-sequence top-k of the tracked-set score.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page), 方法步骤详情 step 4:
// the k decoded tokens with the largest formula-(2) score, together with the
// newly decoded ones, are the next step's tracked set.
//
// One workgroup per sequence.  The score of position i is the sum over heads
// (ascending head order, fp32) of the per-head accumulators the attention
// kernel wrote.  Each candidate's score becomes a 32-bit key that orders
// scores descending; with the position appended (key << 32 | position) the
// wanted set is the k smallest 64-bit composites, and their rank among
// themselves is the output order (highest score first, ties towards the lower
// position).
//
// Selection is a radix select over 4-bit digits, most significant first.  A
// wave counts its candidates per digit from four bit-plane ballots (no LDS
// atomics, so no serialisation when scores share their leading bits: digit
// d's lanes are the AND of the planes, or their complements, that spell d);
// the eight waves' counts meet in LDS behind one barrier, and every wave then
// finds the digit bin that holds the k-th key itself.  The select stops at the first pass whose bin is
// taken whole (then "key below a strict bound" is the whole rule); only when
// the k-th key is tied after all eight passes are the equal keys taken in
// position order, ranked through an LDS bitmap of the tied positions.  The first pass counts every
// candidate, which gives min(k, candidates).  The taken entries (at most 256)
// are ranked by counting over their packed composites, eight per step.
#include "common.h"

namespace {

using dllm::f32x4;
using dllm::u32x4;

constexpr int kMaxThreads = 1024;
constexpr int kMaxCap = 4096;
constexpr int kMaxK = 256;

__device__ __forceinline__ uint32_t order_desc(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in f
    return ~asc;                                                  // descending in f
}

// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// inclusive prefix sum inside each row of 16 lanes (DPP row shifts; a lane
// shifted in from outside the row contributes 0)
__device__ __forceinline__ int row16_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    return v;
}

// wave-wide minimum and maximum (row shifts, then row broadcasts; lane 63
// ends with the result)
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x111, 0xF, 0xF, false));   // row_shr:1
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x112, 0xF, 0xF, false));   // row_shr:2
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x114, 0xF, 0xF, false));   // row_shr:4
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x118, 0xF, 0xF, false));   // row_shr:8
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(~0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// LDS-only workgroup barrier: orders LDS, leaves global stores in flight
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Position of slot e of thread t.  One or two slots: strided over the
// threads (a wave's load is 64 consecutive scores).  Four or eight: runs of
// four consecutive positions (one 16-byte load per run when rows are aligned).
template <int kPer, int kThr>
__device__ __forceinline__ int slot_pos(int t, int e) {
    if constexpr (kPer >= 4) return 4 * t + 4 * kThr * (e >> 2) + (e & 3);
    else return t + kThr * e;
}

template <int kPer, int kThr>   // positions per thread, threads; kPer * kThr >= n_cap
__global__ __launch_bounds__(kThr) void topk_kernel(int n_heads, int n_cap, int k, float* mass,
                                                        const uint8_t* eligible, int32_t* idx,
                                                        float* val, int32_t* count,
                                                        int clear_mass) {
    constexpr int kWaves = kThr / 64;
    __shared__ int s_cnt[2][kWaves][16];
    __shared__ int s_nsel;
    __shared__ uint32_t s_eqbits[kMaxCap / 32];
    __shared__ int s_eqpre[kMaxCap / 32];
    __shared__ __attribute__((aligned(16))) unsigned long long s_sel[kMaxK + 8];
    __shared__ float s_selv[kMaxK];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float* mseq = mass + (int64_t)b * n_heads * n_cap;
    const uint8_t* erow = eligible + (int64_t)b * n_cap;
    const bool vec = kPer >= 4 && (n_cap & 3) == 0;      // 16-byte aligned runs (uniform)

    // ---- eligibility and scores of this thread's positions (loads in flight together) ----
    uint8_t el[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int p = slot_pos<kPer, kThr>(tid, e);
        el[e] = p < n_cap ? erow[p] : 0;
    }
    __builtin_amdgcn_sched_barrier(0);                   // issued ahead of the score loads
    float sc[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) sc[e] = 0.f;
    // heads in groups of kGroup: the group's loads are independent, then added
    // in ascending head order
    constexpr int kGroup = kPer == 1 ? 32 : 64 / kPer;     // one group covers 32 heads
    for (int h0 = 0; h0 < n_heads; h0 += kGroup) {
        float v[kGroup][kPer];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const float* mh = mseq + (int64_t)min(h0 + j, n_heads - 1) * n_cap;
            if (vec) {
#pragma unroll
                for (int r = 0; r < kPer / 4; ++r) {
                    const int p = slot_pos<kPer, kThr>(tid, 4 * r);
                    const f32x4 q = p < n_cap ? *(const f32x4*)(mh + p) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[j][4 * r + c] = q[c];
                }
            } else {
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
                    const int p = slot_pos<kPer, kThr>(tid, e);
                    v[j][e] = mh[min(p, n_cap - 1)];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if (h0 + j < n_heads) sc[e] += v[j][e];
    }
    if (clear_mass) {                                     // this thread's entries only: no hazard
        for (int hh = 0; hh < n_heads; ++hh) {
            float* mh = mseq + (int64_t)hh * n_cap;
            if (vec) {
#pragma unroll
                for (int r = 0; r < kPer / 4; ++r) {
                    const int p = slot_pos<kPer, kThr>(tid, 4 * r);
                    if (p < n_cap) *(f32x4*)(mh + p) = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
                    const int p = slot_pos<kPer, kThr>(tid, e);
                    if (p < n_cap) mh[p] = 0.f;
                }
            }
        }
    }
    uint32_t key[kPer];
    bool cand[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        cand[e] = slot_pos<kPer, kThr>(tid, e) < n_cap && el[e] != 0;
        key[e] = order_desc(sc[e]);
    }

    // ---- candidates, and the leading digits every candidate shares ----
    __shared__ uint32_t s_pre[kWaves][3];
    {
        int c = 0;
        uint32_t lo = ~0u, hi = 0u;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            c += __popcll(__ballot(cand[e]));
            lo = cand[e] ? min(lo, key[e]) : lo;
            hi = cand[e] ? max(hi, key[e]) : hi;
        }
        lo = wave_min_u32(lo);
        hi = wave_max_u32(hi);
        if (lane == 0) {
            s_pre[wave][0] = (uint32_t)c;
            s_pre[wave][1] = lo;
            s_pre[wave][2] = hi;
        }
    }
    lds_barrier();
    int total = 0;
    uint32_t gmin = ~0u, gmax = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        total += (int)s_pre[w][0];
        gmin = min(gmin, s_pre[w][1]);
        gmax = max(gmax, s_pre[w][2]);
    }
    const int kk = min(k, total);

    if constexpr (kPer == 1) {
        // ---- one position per thread: sort, then rank by searching ----
        // Each wave sorts its 64 composites (key << 32 | position; positions that
        // are not candidates take the largest value) ascending with a bitonic
        // network over lane exchanges, and publishes the sorted list.  A
        // composite's rank among all of them is the number of smaller ones, found
        // by a binary search in every wave's list (the eight searches
        // interleaved); candidates ranked below kk write their output there.
        // Composites of candidates are distinct, so ranks are too.
        __shared__ unsigned long long s_sorted[kWaves][64];
        unsigned long long c = cand[0] ? (((unsigned long long)key[0] << 32) | (uint32_t)tid) : ~0ull;
#pragma unroll
        for (int kb = 2; kb <= 64; kb <<= 1)
#pragma unroll
            for (int j = kb >> 1; j > 0; j >>= 1) {
                const unsigned long long o = __shfl_xor(c, j);
                const bool keep_min = ((lane & j) == 0) == ((lane & kb) == 0);
                c = keep_min ? (o < c ? o : c) : (o > c ? o : c);
            }
        s_sorted[wave][lane] = c;
        lds_barrier();
        int pos[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) pos[w] = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1)
#pragma unroll
            for (int w = 0; w < kWaves; ++w) pos[w] += s_sorted[w][pos[w] + step - 1] < c ? step : 0;
        int rank = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) rank += pos[w] + (s_sorted[w][pos[w]] < c ? 1 : 0);
        // the score travels with its composite: fetch it from the lane the
        // position started in (same wave), with every lane taking part
        const float cv = __shfl(sc[0], (int)((uint32_t)c & 63u));
        if (c != ~0ull && rank < kk) {
            idx[(int64_t)b * k + rank] = (int32_t)(uint32_t)(c & 0xffffffffu);
            val[(int64_t)b * k + rank] = cv;
        }
        for (int j = kk + tid; j < k; j += kThr) {
            idx[(int64_t)b * k + j] = -1;
            val[(int64_t)b * k + j] = 0.f;
        }
        if (tid == 0) count[b] = kk;
        return;
    }

    // ---- radix select: take keys below t_strict, plus (ties) krem keys equal to prefix ----
    int krem = kk;
    unsigned long long t_strict = 1ull << 32;             // take key < t_strict
    bool ties = false;
    uint32_t prefix = 0;
    if (kk < total) {                                     // uniform; else every candidate (or none) is taken
        // digits above the first one where the smallest and largest keys differ are common
        const int start = gmin == gmax ? 8 : __builtin_clz(gmin ^ gmax) / 4;
        uint32_t pmask = start == 0 ? 0u : (start >= 8 ? ~0u : ~0u << (32 - 4 * start));
        prefix = gmin & pmask;
        t_strict = prefix;                                // all equal (start == 8): ties at gmin
        ties = start >= 8;
        for (int pass = start; pass < 8; ++pass) {
            const int shift = 28 - 4 * pass;
            int dg[kPer];
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                dg[e] = (cand[e] && (key[e] & pmask) == prefix) ? (int)((key[e] >> shift) & 15u) : 16;
            // per digit, this wave's count: four bit-plane ballots per slot, then
            // the 16 digit masks by AND-ing planes (scalar work, no LDS atomics)
            int cnt[16];
#pragma unroll
            for (int d = 0; d < 16; ++d) cnt[d] = 0;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const unsigned long long mv = __ballot(dg[e] < 16);
                const unsigned long long p0 = __ballot(dg[e] & 1), p1 = __ballot(dg[e] & 2);
                const unsigned long long p2 = __ballot(dg[e] & 4), p3 = __ballot(dg[e] & 8);
                unsigned long long m1[2], m2[4], m3[8];
                m1[0] = mv & ~p0;
                m1[1] = mv & p0;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    m2[q] = m1[q] & ~p1;
                    m2[q + 2] = m1[q] & p1;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    m3[q] = m2[q] & ~p2;
                    m3[q + 4] = m2[q] & p2;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    cnt[q] += __popcll(m3[q] & ~p3);
                    cnt[q + 8] += __popcll(m3[q] & p3);
                }
            }
            int mine = 0;                                 // lane d < 16: this wave's count of digit d
#pragma unroll
            for (int d = 0; d < 16; ++d) mine = lane == d ? cnt[d] : mine;
            if (lane < 16) s_cnt[pass & 1][wave][lane] = mine;
            lds_barrier();
            // every wave: bin totals over the waves, inclusive scan over the 16 bins
            int tot = 0;
            if (lane < 16) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) tot += s_cnt[pass & 1][w][lane];
            }
            const int incl = row16_scan(tot);
            const int excl = incl - tot;
            const unsigned long long hit = __ballot(lane < 16 && excl < krem && krem <= incl);
            const int bin = hit ? __builtin_ctzll(hit) : 15;   // hit != 0: 1 <= krem <= candidates in prefix
            const int cnt_bin = __builtin_amdgcn_readlane(tot, bin), excl_bin = __builtin_amdgcn_readlane(excl, bin);
            krem -= excl_bin;
            prefix |= (uint32_t)bin << shift;
            pmask |= 15u << shift;
            if (krem == cnt_bin) {                        // the bin is taken whole
                t_strict = (unsigned long long)prefix + (1ull << shift);
                break;
            }
            if (pass == 7) {                              // the k-th key is tied: prefix is that key
                t_strict = prefix;
                ties = true;
            }
        }
    }

    // ---- take: keys below t_strict, and (ties) the krem lowest positions among keys == prefix ----
    bool take[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) take[e] = cand[e] && (unsigned long long)key[e] < t_strict;
    if (ties) {                                           // uniform; rare: a bitmap of the tied positions
        for (int w = tid; w < kMaxCap / 32; w += kThr) s_eqbits[w] = 0u;
        lds_barrier();
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int p = slot_pos<kPer, kThr>(tid, e);
            if (cand[e] && key[e] == prefix) atomicOr(&s_eqbits[p >> 5], 1u << (p & 31));
        }
        lds_barrier();
        if (wave == 0) {                                  // exclusive prefix of the word popcounts (128 words)
            const int c0 = __popc(s_eqbits[2 * lane]), c1 = __popc(s_eqbits[2 * lane + 1]);
            int x = c0 + c1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(x, off);
                if (lane >= off) x += t;
            }
            s_eqpre[2 * lane] = x - c0 - c1;
            s_eqpre[2 * lane + 1] = x - c1;
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int p = slot_pos<kPer, kThr>(tid, e);
            if (cand[e] && key[e] == prefix) {
                const int below = s_eqpre[p >> 5] + __popc(s_eqbits[p >> 5] & ((1u << (p & 31)) - 1u));
                take[e] = below < krem;
            }
        }
    }
    // compaction: one LDS atomic per wave; a lane's slots follow the set bits below it
    if (tid == 0) s_nsel = 0;
    const int kk8 = (kk + 7) & ~7;
    if (tid >= kk && tid < kk8) s_sel[tid] = ~0ull;       // padding past the kk taken entries
    lds_barrier();
    {
        unsigned long long m[kPer];
        int wave_total = 0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            m[e] = __ballot(take[e]);
            wave_total += __popcll(m[e]);
        }
        int base = 0;
        if (lane == 0 && wave_total > 0) base = atomicAdd(&s_nsel, wave_total);
        base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int slot = base + lanes_below(m[e]);
            base += __popcll(m[e]);
            if (take[e] && slot < kMaxK) {
                s_sel[slot] = ((unsigned long long)key[e] << 32) | (uint32_t)slot_pos<kPer, kThr>(tid, e);
                s_selv[slot] = sc[e];
            }
        }
    }
    lds_barrier();

    // ---- order: rank of each taken composite among the kk taken (eight per step) ----
    for (int j = tid; j < kk; j += kThr) {
        const unsigned long long cj = s_sel[j];
        int rank = 0;
        for (int i = 0; i < kk8; i += 8) {
            unsigned long long c[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(&s_sel[i + 2 * q]);
                c[2 * q] = ((unsigned long long)w[1] << 32) | w[0];
                c[2 * q + 1] = ((unsigned long long)w[3] << 32) | w[2];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += c[q] < cj ? 1 : 0;
        }
        idx[(int64_t)b * k + rank] = (int32_t)(uint32_t)(cj & 0xffffffffu);
        val[(int64_t)b * k + rank] = s_selv[j];
    }
    for (int j = kk + tid; j < k; j += kThr) {
        idx[(int64_t)b * k + j] = -1;
        val[(int64_t)b * k + j] = 0.f;
    }
    if (tid == 0) count[b] = kk;
}

}  // namespace

extern "C" int dllm_topk_tracked(int n_seq, int n_heads, int n_cap, int k, float* mass,
                                 const uint8_t* eligible, int32_t* idx, float* val, int32_t* count,
                                 int clear_mass, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq > 0 && n_heads > 0 && n_cap > 0 && k > 0);
    DLLM_CHECK_SUP(k <= kMaxK && n_cap <= kMaxCap);
    DLLM_CHECK_ARG(mass && eligible && idx && val && count);
    // positions per thread and threads: up to 1024 positions on 512 threads,
    // beyond that 1024 threads (measured: wide slots cost more than waves)
#define DLLM_TOPK_LAUNCH(P, T)                                                                         \
    hipLaunchKernelGGL((topk_kernel<P, T>), dim3(n_seq), dim3(T), 0, stream, n_heads, n_cap, k, mass, \
                       eligible, idx, val, count, clear_mass)
    if (n_cap <= 512) DLLM_TOPK_LAUNCH(1, 512);
    else if (n_cap <= 1024) DLLM_TOPK_LAUNCH(2, 512);
    else if (n_cap <= 2048) DLLM_TOPK_LAUNCH(2, 1024);
    else DLLM_TOPK_LAUNCH(4, 1024);
#undef DLLM_TOPK_LAUNCH
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
