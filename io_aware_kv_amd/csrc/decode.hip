// Decode-side reductions of a denoising step: per logits row the argmax token
// and its softmax probability (the confidence), then per sequence either the
// threshold rule or the Flash-Verify acceptance scan.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page), 方法步骤详情 step 2
// (confidence of each masked window position; positions at or above epsilon
// are decoded) and step 3 (draft tokens are accepted in position order while
// they equal the mask view's prediction and its confidence is at least gamma;
// the first failure ends acceptance).  [FST] = Fast-dLLM article (senqingzn.com),
// 并行解碼新策略 (confidence-aware parallel decoding):
// a sequence with no position above the threshold decodes its most confident
// one.
//
// The logits pass is a pure HBM stream (R x V values read once, a few bytes
// written), so the design is about keeping enough 16-byte loads in flight:
//   conf_partial_kernel  grid = rows x splits; each workgroup streams one
//                        contiguous chunk of one row with four 16-byte loads
//                        per lane in flight and keeps an online (max, first
//                        argmax, sum of exp(l - max)) per lane, merged over the
//                        workgroup into one partial.  Few rows get split
//                        across several workgroups so the chip fills.
//   decide_kernel        merges a row's partials in a fixed tree (so results
//                        do not depend on scheduling) into token and
//                        confidence = 1 / sum, and applies the per-sequence
//                        rule: one workgroup per sequence, 16 lanes per row.
// Ties: the lowest token id wins inside a row, the lowest row for the forced
// decode.  exp is the hardware base-2 exponential of a pre-scaled argument.
#include <math.h>

#include "common.h"

namespace {

using namespace dllm;

constexpr int kThr = 256;
constexpr int kWaves = kThr / 64;
constexpr int kUnroll = 4;
constexpr int kChunkQuantum = 2048;   // split boundaries are multiples of this many tokens
constexpr int kMinChunk = 8192;       // a split streams at least 16 KB of bf16 logits
constexpr int kTargetBlocks = 1024;   // four workgroups per compute unit
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;

enum Mode { kConfOnly = 0, kCommit = 1, kVerify = 2 };

struct Online {
    float m;   // running maximum (-inf before the first value)
    float s;   // sum of exp(l - m)
    int idx;   // first index holding m
};

__device__ __forceinline__ float exp_scaled(float x_log2) { return __builtin_amdgcn_exp2f(x_log2); }

// merge b into a; on equal maxima the lower index wins, and equal maxima scale
// by exactly 1 (also when both are -inf, so empty partials stay empty)
__device__ __forceinline__ void merge(Online& a, const Online& b) {
    const float M = fmaxf(a.m, b.m);
    const float sa = a.m == M ? a.s : a.s * exp_scaled((a.m - M) * kLog2e);
    const float sb = b.m == M ? b.s : b.s * exp_scaled((b.m - M) * kLog2e);
    a.idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : min(a.idx, b.idx));
    a.m = M;
    a.s = sa + sb;
}

template <int N>
__device__ __forceinline__ void consume(Online& st, const float* f, int base) {
    float vm = f[0];
#pragma unroll
    for (int e = 1; e < N; ++e) vm = fmaxf(vm, f[e]);
    if (vm > st.m) {
        int first = N - 1;
#pragma unroll
        for (int e = N - 2; e >= 0; --e) first = f[e] == vm ? e : first;
        st.s *= exp_scaled((st.m - vm) * kLog2e);
        st.m = vm;
        st.idx = base + first;
    }
    const float ml = st.m * kLog2e;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) acc += exp_scaled(fmaf(f[e], kLog2e, -ml));
    st.s += acc;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static float one(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    __device__ static void unpack(u32x4 v, float* f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(v[e] << 16);
            f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
        }
    }
};
template <> struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static float one(const float* p) { return *p; }
    __device__ static void unpack(u32x4 v, float* f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
    }
};

__device__ __forceinline__ Online shfl_xor(const Online& a, int mask) {
    return Online{__shfl_xor(a.m, mask), __shfl_xor(a.s, mask), __shfl_xor(a.idx, mask)};
}

// one partial per (row, split): part[row * n_split + split] = (m, s, idx, 0)
template <typename T, bool VEC>
__global__ __launch_bounds__(kThr) void conf_partial_kernel(int vocab, int64_t stride, const T* __restrict__ logits,
                                                            int chunk, int n_split, f32x4* __restrict__ part) {
    using E = Elem<T>;
    constexpr int kV = E::kVec;
    const int row = blockIdx.x / n_split, split = blockIdx.x % n_split;
    const int c0 = split * chunk, c1 = min(c0 + chunk, vocab);
    const T* p = logits + (int64_t)row * stride;
    const int t = threadIdx.x;
    Online st{-INFINITY, 0.f, 0x7fffffff};
    if (VEC) {
        const int v0 = c0 / kV, v1 = c1 / kV;   // whole vectors; c0 is a multiple of kV
        const u32x4* pv = (const u32x4*)p;
        int j = v0 + t;
        for (; j + (kUnroll - 1) * kThr < v1; j += kUnroll * kThr) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(pv + j + u * kThr);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float f[kV];
                E::unpack(v[u], f);
                consume<kV>(st, f, (j + u * kThr) * kV);
            }
        }
        for (; j < v1; j += kThr) {
            float f[kV];
            E::unpack(__builtin_nontemporal_load(pv + j), f);
            consume<kV>(st, f, j * kV);
        }
        const int tail = v1 * kV + t;           // fewer than kV tokens past the last whole vector
        if (tail < c1) {
            const float f = E::one(p + tail);
            consume<1>(st, &f, tail);
        }
    } else {
        for (int j = c0 + t; j < c1; j += kThr) {
            const float f = E::one(p + j);
            consume<1>(st, &f, j);
        }
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) merge(st, shfl_xor(st, mask));
    __shared__ Online s_w[kWaves];
    if ((t & 63) == 0) s_w[t >> 6] = st;
    __syncthreads();
    if (t == 0) {
        Online a = s_w[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) merge(a, s_w[w]);
        part[blockIdx.x] = f32x4{a.m, a.s, __int_as_float(a.idx), 0.f};
    }
}

// Rows are handled by groups of 16 lanes (16 groups per workgroup, kSlots
// rows per group in flight): lane l of a group merges the row's partials
// l, l+16, l+32, l+48 in that order, then the 16 lanes merge by xor-shuffles
// 8, 4, 2, 1.  Every partial of kSlots rows is loaded in one round, and the
// fixed merge tree keeps results independent of scheduling.
constexpr int kGroup = 16;
constexpr int kGroups = kThr / kGroup;
constexpr int kSlots = 4;
constexpr int kPerLane = kMaxSplits / kGroup;
constexpr int kRowsPerPass = kGroups * kSlots;

__device__ __forceinline__ void merge_rows(const f32x4* __restrict__ part, int n_split, const int* r, const bool* valid,
                                           Online* out) {
    const int sl = threadIdx.x & (kGroup - 1);
    f32x4 v[kSlots][kPerLane];
#pragma unroll
    for (int i = 0; i < kSlots; ++i)
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            const int sp = sl + u * kGroup;
            v[i][u] = valid[i] && sp < n_split ? part[(int64_t)r[i] * n_split + sp]
                                               : f32x4{-INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f};
        }
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        Online a{v[i][0][0], v[i][0][1], __float_as_int(v[i][0][2])};
#pragma unroll
        for (int u = 1; u < kPerLane; ++u) merge(a, Online{v[i][u][0], v[i][u][1], __float_as_int(v[i][u][2])});
#pragma unroll
        for (int mask = kGroup / 2; mask >= 1; mask >>= 1) merge(a, shfl_xor(a, mask));
        out[i] = a;
    }
}

// block-wide (count, best) reduction: sum of counts, the largest key with the
// lowest row among equal keys; every thread gets the result
struct Best {
    int cnt;
    float key;
    int row;
};
__device__ __forceinline__ void better(Best& a, const Best& b) {
    a.cnt += b.cnt;
    if (b.key > a.key || (b.key == a.key && b.row < a.row)) {
        a.key = b.key;
        a.row = b.row;
    }
}
__device__ Best block_reduce(Best v) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        Best o{__shfl_xor(v.cnt, mask), __shfl_xor(v.key, mask), __shfl_xor(v.row, mask)};
        better(v, o);
    }
    __shared__ Best s_b[kWaves];
    const int t = threadIdx.x;
    if ((t & 63) == 0) s_b[t >> 6] = v;
    lds_sync();
    Best a = s_b[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) better(a, s_b[w]);
    return a;
}

// MODE kConfOnly: kRowsPerPass rows per workgroup, token/conf from the partials.
// MODE kCommit / kVerify: one workgroup per sequence.  With FROM_PART the
// row's token and confidence come from the partials (and are written out);
// otherwise they are read from token/conf.
//   kCommit: flag[r] = conf >= thr, or, when no row of the sequence passes,
//            flag = 1 on its most confident row only; count[b] = flags set.
//   kVerify: flag[r] = 1 for the rows before the first row with
//            token != draft or conf < thr; count[b] = their number.
// A sequence whose row range is malformed (cu[b+1] < cu[b], or outside
// 0..n_rows) is clipped to 0..n_rows and, if still decreasing, is empty.
// Each flag is written once, after the sequence's rows are reduced: from
// registers when the sequence fits one pass (kRowsPerPass rows), else in a
// second pass that re-reads the confidences written in the first.
template <int MODE, bool FROM_PART>
__global__ __launch_bounds__(kThr) void decide_kernel(int n_rows, const int32_t* __restrict__ cu, const f32x4* __restrict__ part,
                                                      int n_split, int32_t* __restrict__ token, float* conf,
                                                      float thr, const int32_t* __restrict__ draft,
                                                      uint8_t* __restrict__ flag, int32_t* __restrict__ count) {
    const int t = threadIdx.x;
    const int g = t / kGroup, sl = t % kGroup;
    if (MODE == kConfOnly) {
        int r[kSlots];
        bool valid[kSlots];
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            r[i] = blockIdx.x * kRowsPerPass + i * kGroups + g;
            valid[i] = r[i] < n_rows;
        }
        Online a[kSlots];
        merge_rows(part, n_split, r, valid, a);
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if (valid[i] && sl == 0) {
                token[r[i]] = a[i].idx;
                conf[r[i]] = 1.f / a[i].s;
            }
        return;
    }
    const int b = blockIdx.x;
    int r0 = cu[b], r1 = cu[b + 1];
    r0 = max(r0, 0);
    r1 = min(r1, n_rows);
    if (r1 < r0) r1 = r0;
    Best loc{0, -INFINITY, 0x7fffffff};
    int r[kSlots] = {};
    bool valid[kSlots] = {}, ok[kSlots] = {};   // an empty sequence writes no flag
    for (int base = r0; base < r1; base += kRowsPerPass) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            r[i] = base + i * kGroups + g;
            valid[i] = r[i] < r1;
        }
        int tk[kSlots];
        float c[kSlots];
        if (FROM_PART) {
            Online a[kSlots];
            merge_rows(part, n_split, r, valid, a);
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                tk[i] = a[i].idx;
                c[i] = 1.f / a[i].s;
                if (valid[i] && sl == 0) {
                    token[r[i]] = tk[i];
                    conf[r[i]] = c[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                c[i] = valid[i] && sl == 0 ? conf[r[i]] : 0.f;
                tk[i] = MODE == kVerify && valid[i] && sl == 0 ? token[r[i]] : 0;
            }
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            ok[i] = false;
            if (!valid[i] || sl != 0) continue;
            if (MODE == kCommit) {
                ok[i] = c[i] >= thr;
                loc.cnt += ok[i];
                // rows of one lane come in increasing order: strict keeps the lowest
                if (c[i] > loc.key) {
                    loc.key = c[i];
                    loc.row = r[i];
                }
            } else if (!(tk[i] == draft[r[i]] && c[i] >= thr)) {
                loc.row = min(loc.row, r[i]);   // first failing row
            }
        }
    }
    if (MODE == kVerify) loc.key = 0.f;         // equal keys: the reduction keeps the lowest row
    const Best tot = block_reduce(loc);
    const bool one_pass = r1 - r0 <= kRowsPerPass;
    if (MODE == kCommit) {
        const bool forced = tot.cnt == 0;
        if (one_pass) {
#pragma unroll
            for (int i = 0; i < kSlots; ++i)
                if (valid[i] && sl == 0) flag[r[i]] = forced ? (r[i] == tot.row) : ok[i];
        } else {
            __syncthreads();                    // the first pass's conf stores are visible
            for (int q = r0 + t; q < r1; q += kThr) flag[q] = forced ? (q == tot.row) : (conf[q] >= thr);
        }
        if (t == 0) count[b] = forced ? (r1 > r0 ? 1 : 0) : tot.cnt;
    } else {
        const int first_fail = min(tot.row, r1);
        for (int q = r0 + t; q < r1; q += kThr) flag[q] = q < first_fail;
        if (t == 0) count[b] = first_fail - r0;
    }
}

struct Plan {
    int chunk, n_split;
};

Plan plan(int n_rows, int vocab) {
    int want = (kTargetBlocks + n_rows - 1) / max(n_rows, 1);
    int by_size = max(1, vocab / kMinChunk);
    int n = max(1, min(min(want, by_size), kMaxSplits));
    int chunk = (vocab + n - 1) / n;
    chunk = (chunk + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
    return Plan{chunk, (vocab + chunk - 1) / chunk};
}

template <typename T>
int launch_partials(int n_rows, int vocab, const void* logits, int64_t row_stride, const Plan& pl, f32x4* part,
                    hipStream_t stream) {
    const int64_t blocks = (int64_t)n_rows * pl.n_split;
    DLLM_CHECK_SUP(blocks < (1ll << 31));
    constexpr int kV = Elem<T>::kVec;
    const bool vec = row_stride % kV == 0 && ((uintptr_t)logits & 15) == 0;
    if (vec)
        hipLaunchKernelGGL((conf_partial_kernel<T, true>), dim3((unsigned)blocks), dim3(kThr), 0, stream, vocab,
                           row_stride, (const T*)logits, pl.chunk, pl.n_split, part);
    else
        hipLaunchKernelGGL((conf_partial_kernel<T, false>), dim3((unsigned)blocks), dim3(kThr), 0, stream, vocab,
                           row_stride, (const T*)logits, pl.chunk, pl.n_split, part);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

int check_logits(dllm_dtype dt, int n_rows, int vocab, const void* logits, int64_t row_stride) {
    DLLM_CHECK_ARG(n_rows >= 0 && vocab > 0 && row_stride >= vocab);
    DLLM_CHECK_ARG(dt == DLLM_BF16 || dt == DLLM_F32);
    DLLM_CHECK_ARG(n_rows == 0 || logits);
    return DLLM_OK;
}

int run_partials(dllm_dtype dt, int n_rows, int vocab, const void* logits, int64_t row_stride, const Plan& pl,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
    DLLM_CHECK_ARG(ws && ws_bytes >= (size_t)n_rows * pl.n_split * sizeof(f32x4));
    DLLM_CHECK_ARG(((uintptr_t)ws & 15) == 0);
    return dt == DLLM_BF16 ? launch_partials<uint16_t>(n_rows, vocab, logits, row_stride, pl, (f32x4*)ws, stream)
                           : launch_partials<float>(n_rows, vocab, logits, row_stride, pl, (f32x4*)ws, stream);
}

template <int MODE>
int launch_decide(bool from_part, int n_seq, int n_rows, const int32_t* cu, const f32x4* part, int n_split,
                  int32_t* token, float* conf, float thr, const int32_t* draft, uint8_t* flag, int32_t* count,
                  hipStream_t stream) {
    if (from_part)
        hipLaunchKernelGGL((decide_kernel<MODE, true>), dim3(n_seq), dim3(kThr), 0, stream, n_rows, cu, part, n_split,
                           token, conf, thr, draft, flag, count);
    else
        hipLaunchKernelGGL((decide_kernel<MODE, false>), dim3(n_seq), dim3(kThr), 0, stream, n_rows, cu, part,
                           n_split, token, conf, thr, draft, flag, count);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

}  // namespace

extern "C" size_t dllm_confidence_workspace(int n_rows, int vocab) {
    if (n_rows <= 0 || vocab <= 0) return 0;
    const Plan pl = plan(n_rows, vocab);
    return (size_t)n_rows * pl.n_split * sizeof(f32x4);
}

extern "C" int dllm_confidence_argmax(dllm_dtype dt, int n_rows, int vocab, const void* logits, int64_t row_stride,
                                      int32_t* token, float* conf, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_logits(dt, n_rows, vocab, logits, row_stride);
    if (rc) return rc;
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(token && conf);
    const Plan pl = plan(n_rows, vocab);
    if ((rc = run_partials(dt, n_rows, vocab, logits, row_stride, pl, ws, ws_bytes, stream))) return rc;
    hipLaunchKernelGGL((decide_kernel<kConfOnly, true>), dim3((n_rows + kRowsPerPass - 1) / kRowsPerPass), dim3(kThr), 0,
                       stream,
                       n_rows, (const int32_t*)nullptr, (const f32x4*)ws, pl.n_split, token, conf, 0.f,
                       (const int32_t*)nullptr, (uint8_t*)nullptr, (int32_t*)nullptr);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

extern "C" int dllm_confidence_commit(int n_seq, int n_rows, const int32_t* cu_rows, const float* conf, float eps,
                                      uint8_t* commit, int32_t* n_commit, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq >= 0 && n_rows >= 0);
    if (n_seq == 0) return DLLM_OK;
    DLLM_CHECK_ARG(cu_rows && n_commit && (n_rows == 0 || (conf && commit)));
    return launch_decide<kCommit>(false, n_seq, n_rows, cu_rows, nullptr, 1, nullptr, (float*)conf, eps, nullptr,
                                  commit, n_commit, stream);
}

extern "C" int dllm_verify_accept(int n_seq, int n_rows, const int32_t* cu_rows, const int32_t* draft,
                                  const int32_t* token, const float* conf, float gamma, uint8_t* accept,
                                  int32_t* n_accept, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq >= 0 && n_rows >= 0);
    if (n_seq == 0) return DLLM_OK;
    DLLM_CHECK_ARG(cu_rows && n_accept && (n_rows == 0 || (draft && token && conf && accept)));
    return launch_decide<kVerify>(false, n_seq, n_rows, cu_rows, nullptr, 1, (int32_t*)token, (float*)conf, gamma,
                                  draft, accept, n_accept, stream);
}

extern "C" int dllm_decode_commit(dllm_dtype dt, int n_seq, int n_rows, const int32_t* cu_rows, int vocab,
                                  const void* logits, int64_t row_stride, float eps, int32_t* token, float* conf,
                                  uint8_t* commit, int32_t* n_commit, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_logits(dt, n_rows, vocab, logits, row_stride);
    if (rc) return rc;
    DLLM_CHECK_ARG(n_seq >= 0);
    if (n_seq == 0) return DLLM_OK;
    DLLM_CHECK_ARG(cu_rows && n_commit && (n_rows == 0 || (token && conf && commit)));
    const Plan pl = plan(max(n_rows, 1), vocab);
    if (n_rows > 0 && (rc = run_partials(dt, n_rows, vocab, logits, row_stride, pl, ws, ws_bytes, stream))) return rc;
    return launch_decide<kCommit>(n_rows > 0, n_seq, n_rows, cu_rows, (const f32x4*)ws, pl.n_split, token, conf, eps,
                                  nullptr, commit, n_commit, stream);
}

extern "C" int dllm_decode_verify(dllm_dtype dt, int n_seq, int n_rows, const int32_t* cu_rows, int vocab,
                                  const void* logits, int64_t row_stride, const int32_t* draft, float gamma,
                                  int32_t* token, float* conf, uint8_t* accept, int32_t* n_accept, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    int rc = check_logits(dt, n_rows, vocab, logits, row_stride);
    if (rc) return rc;
    DLLM_CHECK_ARG(n_seq >= 0);
    if (n_seq == 0) return DLLM_OK;
    DLLM_CHECK_ARG(cu_rows && n_accept && (n_rows == 0 || (draft && token && conf && accept)));
    const Plan pl = plan(max(n_rows, 1), vocab);
    if (n_rows > 0 && (rc = run_partials(dt, n_rows, vocab, logits, row_stride, pl, ws, ws_bytes, stream))) return rc;
    return launch_decide<kVerify>(n_rows > 0, n_seq, n_rows, cu_rows, (const f32x4*)ws, pl.n_split, token, conf,
                                  gamma, draft, accept, n_accept, stream);
}
