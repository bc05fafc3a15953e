// a1-a3: fused QKV projection, rotate-half rotary embedding and KV-cache write.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page).  核心方法: the
// projection, the rotary embedding and the cache write run as one kernel, K/V
// are formed on chip and stored straight into the preallocated flat cache, so
// no q/k/v intermediate crosses HBM; 研究动机: the unfused four-kernel chain
// is bound by memory traffic.
//
// bf16 kernels (gfx950), C = x W^T on v_mfma_f32_16x16x32_bf16.  Both
// operands have the contraction dimension contiguous in memory (x rows, W
// rows), so 16-byte loads give MFMA fragments directly.  Every workgroup owns
// whole rotate-half pairs (i, i + D/2) of one head, so the rotation happens in
// the epilogue without leaving the workgroup: the fp32 tile is staged in LDS,
// rotated with an fp64-reduced angle, rounded once to bf16 and written as
// 16-byte row segments of q_out or of the slot's cache row.
//   * R <= 128 (cache phase): qkv_skinny_kernel streams W once at HBM rate.
//   * larger R (full refresh): qkv_bf16_kernel, LDS-tiled 128 x 128 tiles.
#include <math.h>
#include <stdlib.h>

#include <utility>

#include "common.h"

namespace {

using namespace dllm;

constexpr int kBN = 128;          // output columns per tile
constexpr int kBK = 64;           // contraction step
constexpr int kLDA = kBK + 8;     // LDS row stride in halfwords (144 B: conflict-free b128 reads)
constexpr int kThreads = 256;     // 4 waves, 2 x 2 over the tile
constexpr double kTwoPi = 6.283185307179586476925286766559;

struct QkvArgs {
    int R, d_model, head_dim, n_out, n_ktiles;
    float rope_base;
    const uint16_t* x;
    const uint16_t* w;
    const int32_t* pos;
    const int32_t* slot;
    uint16_t* q_out;
    uint16_t* k_cache;
    uint16_t* v_cache;
    int64_t cache_rows;
};

template <int BM>
__global__ __launch_bounds__(kThreads) void qkv_bf16_kernel(QkvArgs a) {
    constexpr int kStage = (BM + kBN) * kLDA;          // halfwords per pipeline stage
    constexpr int kLDC = kBN + 4;                      // fp32 epilogue row stride
    static_assert(BM * kLDC * 4 <= 2 * kStage * 2, "epilogue tile must fit the stages");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
    __shared__ double s_theta[64];

    const int nt = blockIdx.x, mt = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int row0 = mt * BM, col0 = nt * kBN;
    const int kt0 = 0, kt1 = a.n_ktiles;
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

    auto gload = [&](int kt) __attribute__((always_inline)) {
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
    auto lstore = [&](int stage) __attribute__((always_inline)) {
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

// Skinny projection (R <= 128 rows: the cache phase).  Streaming W at full
// HBM bandwidth is the whole game: W is 3*H*D x d_model and is read exactly
// once.  Each workgroup owns 64 output columns of one (Q/K/V part, head): 32
// "low" columns [j*32, j*32+32) and their rotation partners D/2 higher, so the
// rotation stays inside the workgroup; each of its 4 waves owns one 16-column
// strip.  Both operands are read with coalesced 16-byte loads (16 lanes cover
// one 256-byte row piece), DEPTH-1 K chunks ahead in a register ring, and
// staged through a double-buffered LDS tile whose 16-byte slots are
// XOR-swizzled by row, so the MFMA fragment reads are conflict-free.  A
// sched_barrier pins the issue order so the in-order wait counter never waits
// for a younger prefetch.  No split-K, so no cross-workgroup synchronisation.
constexpr int kSkKC = 128;                 // K chunk (4 MFMA k-steps)

template <int J>
struct Ic { static constexpr int value = J; };

template <int MT, int kDepth>   // 16-row tiles covering R; K chunks in flight + 1
__global__ __launch_bounds__(256, 1) void qkv_skinny_kernel(QkvArgs a) {
    constexpr int kRows = MT * 16;
    constexpr int kXPer = kRows * (kSkKC / 8) / 256;      // x 16-byte pieces per thread
    constexpr int kWPer = 64 * (kSkKC / 8) / 256;         // W pieces per thread (4)
    constexpr int kLDC = 64 + 4;
    static_assert(kRows * (kSkKC / 8) % 256 == 0, "x chunk must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kRows * kSkKC];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][64 * kSkKC];
    __shared__ double s_theta[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, ln = lane & 15;
    const int D = a.head_dim, half = D >> 1;
    const int groups_per_head = D / 64;
    const int grp = blockIdx.x;                          // (part, head, j)
    const int j = grp % groups_per_head;
    const int ph = grp / groups_per_head;                // part * H + head
    const int part = ph / (a.n_out / D);
    const int head = ph % (a.n_out / D);
    const int col_base = part * a.n_out + head * D;      // first W row of this head
    const int R = a.R;
    const int n_chunks = a.d_model / kSkKC;
    if (tid < half) s_theta[tid] = pow((double)a.rope_base, -2.0 * tid / D);

    // global pointers of this thread's pieces (row, 16-byte slot kc)
    const uint16_t* xg[kXPer];
    const uint16_t* wg[kWPer];
    int xl[kXPer], wl[kWPer];                            // swizzled LDS offsets (halfwords)
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
        int c = tid + i * 256, row = c >> 4, kc = c & 15;
        int grow = row < R ? row : R - 1;                 // padding rows repeat a real row
        xg[i] = a.x + (int64_t)grow * a.d_model + kc * 8;
        xl[i] = row * kSkKC + ((kc ^ row) & 15) * 8;
    }
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
        int c = tid + i * 256, r = c >> 4, kc = c & 15;   // r: tile column 0..63
        int wrow = col_base + (r >= 32 ? half : 0) + j * 32 + (r & 31);
        wg[i] = a.w + (int64_t)wrow * a.d_model + kc * 8;
        wl[i] = r * kSkKC + ((kc ^ r) & 15) * 8;
    }
    u32x4 rx[kDepth][kXPer], rw[kDepth][kWPer];
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](auto S, int c) __attribute__((always_inline)) {
        constexpr int sl = decltype(S)::value;
        const int cc = c < n_chunks ? c : n_chunks - 1;   // past the end: re-read the last chunk
#pragma unroll
        for (int i = 0; i < kWPer; ++i) rw[sl][i] = *(const u32x4*)(wg[i] + cc * kSkKC);
#pragma unroll
        for (int i = 0; i < kXPer; ++i) rx[sl][i] = *(const u32x4*)(xg[i] + cc * kSkKC);
    };
    auto store = [&](auto S, int buf) __attribute__((always_inline)) {
        constexpr int sl = decltype(S)::value;
#pragma unroll
        for (int i = 0; i < kWPer; ++i) *(u32x4*)(&ws[buf][wl[i]]) = rw[sl][i];
#pragma unroll
        for (int i = 0; i < kXPer; ++i) *(u32x4*)(&xs[buf][xl[i]]) = rx[sl][i];
    };
    // this wave's 16 output columns: tile columns wave*16 .. wave*16+15
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < kSkKC / 32; ++ks) {
            const int kc = ks * 4 + g;
            const int wr = wave * 16 + ln;
            bf16x8 bw = *(const bf16x8*)(&ws[buf][wr * kSkKC + ((kc ^ wr) & 15) * 8]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int row = m * 16 + ln;
                bf16x8 ax = *(const bf16x8*)(&xs[buf][row * kSkKC + ((kc ^ row) & 15) * 8]);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc[m], 0, 0, 0);
            }
        }
    };

    // prologue: chunks 0 .. DEPTH-2 in flight, chunk 0 staged in LDS
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((load(Ic<I>{}, I), __builtin_amdgcn_sched_barrier(0)), ...);
    }(std::make_integer_sequence<int, kDepth - 1>{});
    store(Ic<0>{}, 0);
    __syncthreads();
    // iteration c: issue chunk c+DEPTH-1, compute chunk c, stage chunk c+1.
    // Loads, stores and barriers are unconditional (exact wait counts); only
    // the LDS-only compute is skipped on the padded trip past the last chunk.
    auto iter = [&](auto S, int c) __attribute__((always_inline)) {
        constexpr int sl = decltype(S)::value;       // c % kDepth
        load(Ic<(sl + kDepth - 1) % kDepth>{}, c + kDepth - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (c < n_chunks) compute(c & 1);
        __builtin_amdgcn_sched_barrier(0);
        store(Ic<(sl + 1) % kDepth>{}, (c + 1) & 1);
        __syncthreads();
    };
    const int n_pad = (n_chunks + kDepth - 1) / kDepth * kDepth;
    for (int c0 = 0; c0 < n_pad; c0 += kDepth) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (iter(Ic<I>{}, c0 + I), ...);
        }(std::make_integer_sequence<int, kDepth>{});
    }

    // ---- epilogue: fp32 tile [R_pad][64] in LDS, rotate pairs, write ----
    float* Cs = reinterpret_cast<float*>(&xs[0][0]);
    static_assert(kRows * kLDC * 4 <= (int)sizeof(xs), "epilogue tile must fit");
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Cs[(m * 16 + g * 4 + e) * kLDC + wave * 16 + ln] = acc[m][e];
    __syncthreads();
    const int cpart = head * D + j * 32;                // low column within the part
    for (int idx = tid; idx < R * 4; idx += 256) {
        const int r = idx >> 2, q = idx & 3;             // 8-column piece q of the 32 low columns
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = Cs[r * kLDC + q * 8 + e];
            hi[e] = Cs[r * kLDC + 32 + q * 8 + e];
        }
        uint16_t* dst;
        if (part == 0) {
            dst = a.q_out + (int64_t)r * a.n_out;
        } else {
            int sl = a.slot[r];
            if (sl < 0 || (int64_t)sl >= a.cache_rows) continue;
            dst = (part == 1 ? a.k_cache : a.v_cache) + (int64_t)sl * a.n_out;
        }
        if (part < 2) {
            const double p = (double)a.pos[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double ang = p * s_theta[j * 32 + q * 8 + e];
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
        *(u32x4*)(dst + cpart + q * 8) = plo;
        *(u32x4*)(dst + cpart + half + q * 8) = phi;
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
    bool skinny;
    int bm, n_mtiles, n_ntiles, n_ktiles;
};

// Cache-phase row counts (R <= 128) take the weight-streaming kernel; larger
// R takes the LDS-tiled kernel.  Neither splits K, so no workspace is needed.
QkvPlan plan_bf16(int R, int d_model, int n_out) {
    QkvPlan p{};
    p.skinny = R <= 128 && d_model % 128 == 0;
    p.bm = R <= 64 ? 64 : 128;
    p.n_mtiles = (R + p.bm - 1) / p.bm;
    p.n_ntiles = 3 * n_out / kBN;
    p.n_ktiles = d_model / kBK;
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
    return 0;      // no kernel of this entry point needs scratch memory
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
    (void)workspace;
    (void)workspace_bytes;
    DLLM_CHECK_SUP(p.n_mtiles < 65536);
    QkvArgs a;
    a.R = n_rows;
    a.d_model = d_model;
    a.head_dim = head_dim;
    a.n_out = n_out;
    a.n_ktiles = p.n_ktiles;
    a.rope_base = rope_base;
    a.x = (const uint16_t*)x;
    a.w = (const uint16_t*)w_qkv;
    a.pos = pos;
    a.slot = slot;
    a.q_out = (uint16_t*)q_out;
    a.k_cache = (uint16_t*)k_cache;
    a.v_cache = (uint16_t*)v_cache;
    a.cache_rows = cache_rows;
    if (p.skinny) {
        dim3 grid(3 * n_out / 64);
        switch ((n_rows + 15) / 16) {
            case 1: hipLaunchKernelGGL((qkv_skinny_kernel<1, 8>), grid, dim3(256), 0, stream, a); break;
            case 2: hipLaunchKernelGGL((qkv_skinny_kernel<2, 8>), grid, dim3(256), 0, stream, a); break;
            case 3: hipLaunchKernelGGL((qkv_skinny_kernel<3, 6>), grid, dim3(256), 0, stream, a); break;
            case 4: hipLaunchKernelGGL((qkv_skinny_kernel<4, 6>), grid, dim3(256), 0, stream, a); break;
            case 5: hipLaunchKernelGGL((qkv_skinny_kernel<5, 6>), grid, dim3(256), 0, stream, a); break;
            case 6: hipLaunchKernelGGL((qkv_skinny_kernel<6, 5>), grid, dim3(256), 0, stream, a); break;
            case 7: hipLaunchKernelGGL((qkv_skinny_kernel<7, 5>), grid, dim3(256), 0, stream, a); break;
            default: hipLaunchKernelGGL((qkv_skinny_kernel<8, 4>), grid, dim3(256), 0, stream, a); break;
        }
    } else {
        dim3 grid(p.n_ntiles, p.n_mtiles, 1);
        if (p.bm == 64)
            hipLaunchKernelGGL(qkv_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(qkv_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    }
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
