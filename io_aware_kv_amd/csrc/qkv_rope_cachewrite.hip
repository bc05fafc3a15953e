// a1-a3: fused QKV projection, rotate-half rotary embedding and KV-cache write.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page).  核心方法: the
// projection, the rotary embedding and the cache write run as one kernel, K/V
// are formed on chip and stored straight into the preallocated flat cache, so
// no q/k/v intermediate crosses HBM; 研究动机: the unfused four-kernel chain
// is bound by memory traffic.
//
// bf16 kernel (gfx950): C = x W^T on v_mfma_f32_16x16x32_bf16.  A workgroup
// owns a BM x 128 output tile, i.e. one whole head of Q, K or V for D = 128
// (two heads for D = 64), so every rotate-half pair (i, i + D/2) lies in the
// tile.  Both operands have the contraction dimension contiguous in memory
// (x rows, W rows), so 16-byte loads feed the MFMA fragments directly from
// LDS.  When there are too few output tiles to fill 256 CUs (a cache-phase
// step has R ~ 72 rows: 96 tiles), the K dimension is split across
// workgroups; each writes an fp32 partial and the last one to finish a tile
// sums the partials in split order (deterministic) and runs the epilogue.
// The epilogue stages the tile in LDS, applies the rotation in fp32 with an
// fp64-reduced angle, rounds once to bf16 and writes whole 16-byte row
// segments of q_out or of the slot's cache row.
#include <math.h>
#include <stdlib.h>

#include "common.h"

namespace {

using namespace dllm;

constexpr int kBN = 128;          // output columns per tile
constexpr int kBK = 64;           // contraction step
constexpr int kLDA = kBK + 8;     // LDS row stride in halfwords (144 B: conflict-free b128 reads)
constexpr int kThreads = 256;     // 4 waves, 2 x 2 over the tile
constexpr double kTwoPi = 6.283185307179586476925286766559;

struct QkvArgs {
    int R, d_model, head_dim, n_out, splits, kt_per_split, n_ktiles, n_ntiles;
    float rope_base;
    const uint16_t* x;
    const uint16_t* w;
    const int32_t* pos;
    const int32_t* slot;
    uint16_t* q_out;
    uint16_t* k_cache;
    uint16_t* v_cache;
    int64_t cache_rows;
    float* partial;
    int32_t* counters;
};

template <int BM>
__global__ __launch_bounds__(kThreads) void qkv_bf16_kernel(QkvArgs a) {
    constexpr int kStage = (BM + kBN) * kLDA;          // halfwords per pipeline stage
    constexpr int kLDC = kBN + 4;                      // fp32 epilogue row stride
    static_assert(BM * kLDC * 4 <= 2 * kStage * 2, "epilogue tile must fit the stages");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
    __shared__ double s_theta[64];
    __shared__ int s_last;

    const int nt = blockIdx.x, mt = blockIdx.y, sp = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int row0 = mt * BM, col0 = nt * kBN;
    const int kt0 = sp * a.kt_per_split;
    const int kt1 = min(kt0 + a.kt_per_split, a.n_ktiles);
    const int half = a.head_dim >> 1;

    if (tid < half) s_theta[tid] = pow((double)a.rope_base, -2.0 * tid / a.head_dim);

    constexpr int kACh = BM * 8 / kThreads;           // 16-byte chunks per thread
    constexpr int kBCh = kBN * 8 / kThreads;
    constexpr int kMT = BM / 32;                        // 16-row tiles per wave
    u32x4 ra[kACh], rb[kBCh];
    f32x4 acc[kMT][4];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < kACh; ++i) {
            int c = tid + i * kThreads, r = c >> 3, kc = c & 7;
            int grow = row0 + r;
            if (grow < a.R)
                ra[i] = *(const u32x4*)(a.x + (int64_t)grow * a.d_model + kt * kBK + kc * 8);
            else
                ra[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kBCh; ++i) {
            int c = tid + i * kThreads, r = c >> 3, kc = c & 7;
            rb[i] = *(const u32x4*)(a.w + (int64_t)(col0 + r) * a.d_model + kt * kBK + kc * 8);
        }
    };
    auto lstore = [&](int stage) {
        uint16_t* As = smem + stage * kStage;
        uint16_t* Bs = As + BM * kLDA;
#pragma unroll
        for (int i = 0; i < kACh; ++i) {
            int c = tid + i * kThreads, r = c >> 3, kc = c & 7;
            *(u32x4*)(As + r * kLDA + kc * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < kBCh; ++i) {
            int c = tid + i * kThreads, r = c >> 3, kc = c & 7;
            *(u32x4*)(Bs + r * kLDA + kc * 8) = rb[i];
        }
    };

    if (kt0 < kt1) {
        gload(kt0);
        lstore(0);
    }
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        if (kt + 1 < kt1) gload(kt + 1);
        const uint16_t* As = smem + cur * kStage;
        const uint16_t* Bs = As + BM * kLDA;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k = ks * 32 + (lane >> 4) * 8;
            bf16x8 af[kMT], bfr[4];
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                af[i] = *(const bf16x8*)(As + (wm * (BM / 2) + i * 16 + (lane & 15)) * kLDA + k);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *(const bf16x8*)(Bs + (wn * 64 + j * 16 + (lane & 15)) * kLDA + k);
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < kt1) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---- stage the fp32 tile in LDS ----
    float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int r = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + e;
                int c = wn * 64 + j * 16 + (lane & 15);
                Cs[r * kLDC + c] = acc[i][j][e];
            }
    __syncthreads();

    const int rows_valid = min(BM, a.R - row0);
    if (a.splits > 1) {
        // publish this split's partial, then let the last split finish the tile
        const int tile = mt * a.n_ntiles + nt;
        float* mine = a.partial + ((int64_t)tile * a.splits + sp) * BM * kBN;
        for (int idx = tid; idx < rows_valid * (kBN / 4); idx += kThreads) {
            int r = idx / (kBN / 4), c4 = idx % (kBN / 4);
            *(f32x4*)(mine + r * kBN + c4 * 4) = *(const f32x4*)(Cs + r * kLDC + c4 * 4);
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = (atomicAdd(&a.counters[tile], 1) == a.splits - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const float* base = a.partial + (int64_t)tile * a.splits * BM * kBN;
        for (int idx = tid; idx < rows_valid * (kBN / 4); idx += kThreads) {
            int r = idx / (kBN / 4), c4 = idx % (kBN / 4);
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int q = 0; q < a.splits; ++q) s += *(const f32x4*)(base + (int64_t)q * BM * kBN + r * kBN + c4 * 4);
            *(f32x4*)(Cs + r * kLDC + c4 * 4) = s;
        }
        if (tid == 0) a.counters[tile] = 0;
        __syncthreads();
    }

    // ---- epilogue: rotate, round, write ----
    const int part = col0 / a.n_out;            // 0 = Q, 1 = K, 2 = V
    const int cpart = col0 % a.n_out;
    const int chunks_per_head = half / 8;
    for (int idx = tid; idx < rows_valid * (kBN / 16); idx += kThreads) {
        const int r = idx / (kBN / 16), j = idx % (kBN / 16);
        const int grow = row0 + r;
        const int hh = j / chunks_per_head, jj = j % chunks_per_head;
        const int c_lo = hh * a.head_dim + jj * 8, c_hi = c_lo + half;
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = Cs[r * kLDC + c_lo + e];
            hi[e] = Cs[r * kLDC + c_hi + e];
        }
        uint16_t* dst;
        if (part == 0) {
            dst = a.q_out + (int64_t)grow * a.n_out + cpart;
        } else {
            int s = a.slot[grow];
            if (s < 0 || (int64_t)s >= a.cache_rows) continue;
            dst = (part == 1 ? a.k_cache : a.v_cache) + (int64_t)s * a.n_out + cpart;
        }
        if (part < 2) {
            const double p = (double)a.pos[grow];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double ang = p * s_theta[jj * 8 + e];
                ang -= rint(ang * (1.0 / kTwoPi)) * kTwoPi;
                float sn, cs;
                sincosf((float)ang, &sn, &cs);
                float x0 = lo[e], x1 = hi[e];
                lo[e] = x0 * cs - x1 * sn;
                hi[e] = x1 * cs + x0 * sn;
            }
        }
        u32x4 plo, phi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            plo[e] = pack_bf16x2(lo[2 * e], lo[2 * e + 1]);
            phi[e] = pack_bf16x2(hi[2 * e], hi[2 * e + 1]);
        }
        *(u32x4*)(dst + c_lo) = plo;
        *(u32x4*)(dst + c_hi) = phi;
    }
}

// fp32 path (parity-sized shapes): one thread per (row, Q/K/V part, head,
// rotation pair) forms both columns of the pair, rotates and stores them.
__global__ void qkv_f32_kernel(int R, int d_model, int n_heads, int head_dim, float rope_base,
                               const float* __restrict__ x, const float* __restrict__ w,
                               const int32_t* __restrict__ pos, const int32_t* __restrict__ slot,
                               float* __restrict__ q_out, float* __restrict__ k_cache,
                               float* __restrict__ v_cache, int64_t cache_rows) {
    const int half = head_dim / 2;
    const int n_out = n_heads * head_dim;
    const int64_t total = (int64_t)R * 3 * n_heads * half;
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int i = idx % half;
    const int h = (idx / half) % n_heads;
    const int part = (idx / ((int64_t)half * n_heads)) % 3;
    const int r = idx / ((int64_t)half * n_heads * 3);
    const int c_lo = h * head_dim + i, c_hi = c_lo + half;
    const float* xr = x + (int64_t)r * d_model;
    const float* w_lo = w + (int64_t)(part * n_out + c_lo) * d_model;
    const float* w_hi = w + (int64_t)(part * n_out + c_hi) * d_model;
    float lo = 0.f, hi = 0.f;
    for (int k = 0; k < d_model; ++k) {
        lo = fmaf(xr[k], w_lo[k], lo);
        hi = fmaf(xr[k], w_hi[k], hi);
    }
    if (part < 2) {
        double theta = pow((double)rope_base, -2.0 * i / head_dim);
        double ang = (double)pos[r] * theta;
        ang -= rint(ang * (1.0 / kTwoPi)) * kTwoPi;
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        float x0 = lo, x1 = hi;
        lo = x0 * cs - x1 * sn;
        hi = x1 * cs + x0 * sn;
    }
    float* dst;
    if (part == 0) {
        dst = q_out + (int64_t)r * n_out;
    } else {
        int s = slot[r];
        if (s < 0 || (int64_t)s >= cache_rows) return;
        dst = (part == 1 ? k_cache : v_cache) + (int64_t)s * n_out;
    }
    dst[c_lo] = lo;
    dst[c_hi] = hi;
}

struct QkvPlan {
    int bm, n_mtiles, n_ntiles, n_ktiles, splits, kt_per_split;
    size_t partial_bytes, counter_bytes;
};

// Split-K only when the output tiles cannot fill the chip.  DLLM_QKV_SPLITK
// overrides the split count (a tuning knob; both the size query and the call
// read it, so they agree).
QkvPlan plan_bf16(int R, int d_model, int n_out) {
    QkvPlan p{};
    p.bm = R <= 64 ? 64 : 128;
    p.n_mtiles = (R + p.bm - 1) / p.bm;
    p.n_ntiles = 3 * n_out / kBN;
    p.n_ktiles = d_model / kBK;
    int tiles = p.n_mtiles * p.n_ntiles;
    int want = 1;
    if (tiles < 2 * kNumCu) want = (2 * kNumCu + tiles - 1) / tiles;
    const char* env = getenv("DLLM_QKV_SPLITK");
    if (env && atoi(env) > 0) want = atoi(env);
    if (want > p.n_ktiles) want = p.n_ktiles;
    if (want < 1) want = 1;
    p.kt_per_split = (p.n_ktiles + want - 1) / want;
    p.splits = (p.n_ktiles + p.kt_per_split - 1) / p.kt_per_split;
    if (p.splits > 1) {
        p.partial_bytes = (size_t)tiles * p.splits * p.bm * kBN * sizeof(float);
        p.counter_bytes = ((size_t)tiles * sizeof(int32_t) + 255) / 256 * 256;
    }
    return p;
}

int check_shape(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim) {
    DLLM_CHECK_ARG(n_rows >= 0 && d_model > 0 && n_heads > 0 && head_dim > 0);
    DLLM_CHECK_SUP(dt == DLLM_BF16 || dt == DLLM_F32);
    DLLM_CHECK_SUP(head_dim == 64 || head_dim == 128);
    if (dt == DLLM_BF16) {
        DLLM_CHECK_SUP((n_heads * head_dim) % kBN == 0);
        DLLM_CHECK_SUP(d_model % kBK == 0);
    }
    return DLLM_OK;
}

}  // namespace

extern "C" size_t dllm_qkv_rope_cachewrite_workspace(dllm_dtype dt, int n_rows, int d_model,
                                                     int n_heads, int head_dim) {
    if (check_shape(dt, n_rows, d_model, n_heads, head_dim) != DLLM_OK) return 0;
    if (dt != DLLM_BF16 || n_rows == 0) return 0;
    QkvPlan p = plan_bf16(n_rows, d_model, n_heads * head_dim);
    return p.counter_bytes + p.partial_bytes;
}

extern "C" int dllm_qkv_rope_cachewrite(dllm_dtype dt, int n_rows, int d_model, int n_heads,
                                        int head_dim, float rope_base, const void* x,
                                        const void* w_qkv, const int32_t* pos, const int32_t* slot,
                                        void* q_out, void* k_cache, void* v_cache,
                                        int64_t cache_rows, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    int st = check_shape(dt, n_rows, d_model, n_heads, head_dim);
    if (st != DLLM_OK) return st;
    DLLM_CHECK_ARG(rope_base > 0.f && cache_rows >= 0);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(x && w_qkv && pos && slot && q_out && k_cache && v_cache);
    const int n_out = n_heads * head_dim;
    if (dt == DLLM_F32) {
        int64_t total = (int64_t)n_rows * 3 * n_heads * (head_dim / 2);
        int threads = 256;
        int64_t blocks = (total + threads - 1) / threads;
        DLLM_CHECK_SUP(blocks < (1ll << 31));
        hipLaunchKernelGGL(qkv_f32_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           n_rows, d_model, n_heads, head_dim, rope_base, (const float*)x,
                           (const float*)w_qkv, pos, slot, (float*)q_out, (float*)k_cache,
                           (float*)v_cache, cache_rows);
        DLLM_CHECK_LAUNCH();
        return DLLM_OK;
    }
    QkvPlan p = plan_bf16(n_rows, d_model, n_out);
    DLLM_CHECK_ARG(workspace_bytes >= p.counter_bytes + p.partial_bytes);
    if (p.splits > 1) DLLM_CHECK_ARG(workspace != nullptr);
    DLLM_CHECK_SUP(p.n_mtiles < 65536);
    QkvArgs a;
    a.R = n_rows;
    a.d_model = d_model;
    a.head_dim = head_dim;
    a.n_out = n_out;
    a.splits = p.splits;
    a.kt_per_split = p.kt_per_split;
    a.n_ktiles = p.n_ktiles;
    a.n_ntiles = p.n_ntiles;
    a.rope_base = rope_base;
    a.x = (const uint16_t*)x;
    a.w = (const uint16_t*)w_qkv;
    a.pos = pos;
    a.slot = slot;
    a.q_out = (uint16_t*)q_out;
    a.k_cache = (uint16_t*)k_cache;
    a.v_cache = (uint16_t*)v_cache;
    a.cache_rows = cache_rows;
    a.counters = (int32_t*)workspace;
    a.partial = p.splits > 1 ? (float*)((char*)workspace + p.counter_bytes) : nullptr;
    dim3 grid(p.n_ntiles, p.n_mtiles, p.splits);
    if (p.bm == 64)
        hipLaunchKernelGGL(qkv_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(qkv_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
