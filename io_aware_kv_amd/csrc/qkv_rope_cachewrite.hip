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
//   * R <= 128 (cache phase): qkv_stream2_kernel streams W once through one
//     ring of direct-to-LDS copies shared by the workgroup's four waves.
//   * a few hundred rows: qkv_mid_kernel, the same streaming design on a
//     grid of row groups by pair groups.
//   * large R (full refresh): qkv_gemm_kernel, 256 x 256 (or smaller) tiles
//     fed by direct-to-LDS copies.
//   * shapes the others cannot take: qkv_bf16_kernel, LDS-tiled 128 x 128.
#include <math.h>
#include <stdlib.h>
#include <string.h>

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
    // paged mode (cache-phase kernel only): slots formed on the device from the
    // block table; slot above is then unused
    const int32_t* cu_q;
    const int32_t* logical;
    const int32_t* page_table;
    int32_t* slot_out;
    int n_seq, max_pages, page_size, pool_pages;
    // unfused comparison arm: unrotated q|k|v rows to raw_out [R, 3 n_out]; no
    // rotation and no cache write (nullptr otherwise)
    uint16_t* raw_out;
    int kv_fp8;             // K/V caches hold E4M3 codes (one byte per element)
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
        int64_t cache_off = 0;                           // element offset of a cache row's piece
        if (a.raw_out) {
            dst = a.raw_out + (int64_t)grow * 3 * a.n_out + part * a.n_out + cpart;
        } else if (part == 0) {
            dst = a.q_out + (int64_t)grow * a.n_out + cpart;
        } else {
            int s = a.slot[grow];
            if (s < 0 || (int64_t)s >= a.cache_rows) continue;
            cache_off = (int64_t)s * a.n_out + cpart;
            dst = (part == 1 ? a.k_cache : a.v_cache) + cache_off;
        }
        if (part < 2 && !a.raw_out) {
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
        if (part > 0 && a.kv_fp8 && !a.raw_out) {
            uint8_t* d8 = (uint8_t*)(part == 1 ? a.k_cache : a.v_cache) + cache_off;
            *(uint2*)(d8 + c_lo) = make_uint2(e4m3x4(lo[0], lo[1], lo[2], lo[3]), e4m3x4(lo[4], lo[5], lo[6], lo[7]));
            *(uint2*)(d8 + c_hi) = make_uint2(e4m3x4(hi[0], hi[1], hi[2], hi[3]), e4m3x4(hi[4], hi[5], hi[6], hi[7]));
            continue;
        }
        *(u32x4*)(dst + c_lo) = plo;
        *(u32x4*)(dst + c_hi) = phi;
    }
}

// Projection for R > 128 rows: BM x BN output tiles, four waves each owning
// WM = 16 WMF rows by one whole head of 128 columns (WGM waves along the rows,
// 4 / WGM along the columns).  The MFMA computes the transposed tile (W rows
// as its A operand), so a lane's four accumulator values are four consecutive
// output columns of one row: they pack into one 8-byte LDS write, and the
// rotate-half partner (column c + 64) of each sits in the same lane four
// n-tiles further on.
//
// Tile shapes (GemmCfg): 256 x 256 (one workgroup per compute unit, four
// 32 KiB stages) for large R; 128 x 256, 64 x 256, 256 x 128 and 128 x 128 so
// that mid-size R still spreads over every compute unit, each either alone on
// its compute unit with a deep ring (OCC 1: up to 150 KiB of stages, so the
// copies run 5 to 7 stages ahead of the MFMAs: a smaller tile has less MFMA
// work per stage to hide a copy's latency behind) or two per compute unit
// (OCC 2: at most 78 KiB each).  A wave's fragment reuse falls with its row
// count (LDS bytes per MFMA grow as 1/WM + 1/128).
//
// Operands reach LDS through 16-byte direct-to-LDS loads (no register
// staging), NS stages of BK = 32 deep.  A direct-to-LDS load writes lane i's
// 16 bytes to LDS offset base + 16 i, so the XOR swizzle that keeps the
// fragment reads free of bank conflicts is applied on the source side: lane i
// fetches the logical 16-byte slot that belongs at its physical place.
//
// Pipeline: the fragments of stage kt+1 are read from LDS while the MFMAs of
// stage kt run, and the wave's copy instructions for stage kt+NS are spread
// over its groups of 8 MFMAs rather than issued at once, which would fill the
// address queue and hold up the wave.  One barrier per stage both publishes
// stage kt+1 and frees stage kt's buffer for the copy of kt+NS.
//
// Tiles are ordered in groups of 4 row tiles x all column tiles, column
// major inside a group, so the workgroups one XCD runs at a time share their
// x and W slices in that XCD's L2.
constexpr int kGBK = 32;
constexpr int kGroupM = 4;
constexpr int kGemmLdsPair = 78 * 1024;   // per workgroup when two share a compute unit
constexpr int kGemmLdsOne = 150 * 1024;   // ring of a workgroup alone on its compute unit
constexpr int kGemmMaxStages = 8;
constexpr int kGemmKB = 2;                // stages (of BK) per barrier

template <int WMF, int WGM, int OCC>
struct GemmCfg {
    static constexpr int WM = 16 * WMF;               // rows per wave
    static constexpr int BM = WGM * WM;
    static constexpr int BN = (4 / WGM) * 128;
    static constexpr int BK = kGBK;
    static constexpr int kStage = (BM + BN) * BK;      // halfwords per stage
    static constexpr int kInst = (BM + BN) / 16 / 4;   // 1 KiB copy instructions per wave per stage
    static constexpr bool kBig = BM == 256 && BN == 256;
    static constexpr int kOcc = OCC;
    static constexpr int kRing = (OCC == 2 ? kGemmLdsPair : kGemmLdsOne) / (2 * kStage);
    static constexpr int NS = kBig ? 4 : (kRing < kGemmMaxStages ? kRing : kGemmMaxStages);
    static constexpr int kCopyPerGroup = (kInst + WMF - 1) / WMF;
    static constexpr int kWPerGroup = 8 / WMF > 2 ? 8 / WMF : 2;
    static_assert(WGM == 1 || WGM == 2 || WGM == 4, "four waves");
    static_assert(NS * kStage >= 4 * WM * 128, "the epilogue reuses the stages as one WM x 128 tile per wave");
    // stages per barrier: kGemmKB for the deep-ring small tiles (fewer
    // barriers per MFMA); one for the 256 x 256 tile, whose copies need the
    // latency hiding of a new stage every barrier (two per barrier measured
    // 15% slower), and for the two-per-unit tiles (three-stage rings)
    static constexpr int KB = (!kBig && NS >= 2 * kGemmKB) ? kGemmKB : 1;
    static_assert(NS >= 2 * KB && NS >= 3, "two iterations of stages in the ring");
    static_assert(OCC == 1 || NS * kStage * 2 + 8 * BM + 512 <= kGemmLdsPair, "two workgroups per compute unit");
    static_assert(!kBig || OCC == 1, "one 256 x 256 workgroup per compute unit");
    static_assert((NS - KB) * kInst < 64 && (NS - 1) * kInst < 64, "wait counts");
};

// Physical 16-byte slot of logical slot 0 in a 64-byte staged row: any 16
// consecutive rows read at one logical slot hit 16 distinct bank groups (and
// every 8 consecutive rows 8 distinct ones), so the fragment reads are free
// of bank conflicts.
__device__ __forceinline__ int gemm_swz(int row) { return ((row >> 2) ^ (row >> 1)) & 3; }

// wait until at most `ahead` (<= MAXA) stages of this wave's copies are still
// in flight (s_waitcnt takes an immediate: one branch per count)
template <int KI, int MAXA>
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
    if (MAXA >= 6 && ahead >= 6) __builtin_amdgcn_s_waitcnt(waitcnt_imm(6 * KI, 0));
    else if (MAXA >= 5 && ahead == 5) __builtin_amdgcn_s_waitcnt(waitcnt_imm(5 * KI, 0));
    else if (MAXA >= 4 && ahead == 4) __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * KI, 0));
    else if (MAXA >= 3 && ahead == 3) __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * KI, 0));
    else if (ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * KI, 0));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_imm(KI, 0));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
}

// EPI (compile-time, so the rotating instantiation keeps its registers):
// kEpiRot rotates q and k and writes bf16 rows; kEpiRaw is the unfused arm's
// plain row store; kEpiRotE4M3 rotates and writes the K/V rows as E4M3 codes.
enum { kEpiRot = 0, kEpiRaw = 1, kEpiRotE4M3 = 2 };
template <int WMF, int WGM, int OCC, int EPI>
__global__ __launch_bounds__(256, OCC) void qkv_gemm_kernel(QkvArgs a, int n_mtiles, int n_ntiles) {
    using C = GemmCfg<WMF, WGM, OCC>;
    constexpr bool RAW = EPI == kEpiRaw;
    constexpr int BM = C::BM, BK = C::BK, NS = C::NS, WM = C::WM, kInst = C::kInst, kStage = C::kStage;
    constexpr int kSlots = BK / 8;                      // 16-byte slots per staged row
    constexpr int kRowsPerInst = 64 / kSlots;           // rows one 1 KiB copy instruction covers
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * kStage];
    __shared__ double s_theta[64];
    __shared__ int s_pos[BM], s_slot[BM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, ln = lane & 15;
    const int wm = wave % WGM, wn = wave / WGM;
    // ---- tile order: XCD-contiguous items, grouped 4 row tiles x all column tiles ----
    const int item = xcd_remap(blockIdx.x, n_mtiles * n_ntiles);
    const int per_group = kGroupM * n_ntiles;
    const int first_m = (item / per_group) * kGroupM;
    const int gm_sz = min(kGroupM, n_mtiles - first_m);
    const int local = item % per_group;
    const int mt = first_m + local % gm_sz, nt = local / gm_sz;
    const int row0 = mt * BM, col0 = nt * C::BN;
    // rotation frequencies in revolutions per position (theta / 2 pi)
    if (tid < a.head_dim / 2) s_theta[tid] = pow((double)a.rope_base, -2.0 * tid / a.head_dim) * (1.0 / kTwoPi);
    if (!RAW && tid < BM) {
        const int grow = min(row0 + tid, a.R - 1);
        s_pos[tid] = a.pos[grow];
        s_slot[tid] = a.slot[grow];
    }

    // ---- copy sources: instruction j of a stage covers rows kRowsPerInst*j ..; x first, then W ----
    const uint16_t* src[kInst];
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
        const int j = wave * kInst + i;
        const int r = (j * kRowsPerInst) % BM + lane / kSlots;
        if (j * kRowsPerInst < BM) {
            int grow = row0 + r;
            grow = grow < a.R ? grow : a.R - 1;         // ragged tail: re-read a real row, never stored
            src[i] = a.x + (int64_t)grow * a.d_model + ((lane % kSlots) ^ gemm_swz(r)) * 8;
        } else {
            const int c = j * kRowsPerInst - BM + lane / kSlots;
            src[i] = a.w + (int64_t)(col0 + c) * a.d_model + ((lane % kSlots) ^ gemm_swz(c)) * 8;
        }
    }
    // Copies are issued from inline assembly: the compiler cannot tell that a
    // copy into one stage and a fragment read of another do not overlap, and
    // with the builtin it waits for every copy before the next read.  The
    // stage barrier below waits for exactly the copies a stage needs.
    const uint32_t lds0 = lds_addr(smem);
    auto issue_one = [&](int stage, int kt, int i) __attribute__((always_inline)) {
        const int j = wave * kInst + i;
        copy16_to_lds(src[i] + kt * BK, lds0 + (uint32_t)(stage * kStage + j * 512) * 2u);
    };
    // fragments: x rows (MFMA B operand, 16 tokens) and W rows (MFMA A operand, 16 features)
    auto read_x = [&](int kt, int i) __attribute__((always_inline)) {
        const int r = wm * WM + i * 16 + ln;
        return *(const bf16x8*)(smem + (kt % NS) * kStage + r * BK + ((g ^ gemm_swz(r)) % kSlots) * 8);
    };
    auto read_w = [&](int kt, int t) __attribute__((always_inline)) {
        const int c = wn * 128 + t * 16 + ln;
        return *(const bf16x8*)(smem + (kt % NS) * kStage + BM * BK + c * BK + ((g ^ gemm_swz(c)) % kSlots) * 8);
    };
    // This thread's copies of stage `next` have landed (later stages may stay
    // in flight) and its fragment reads have returned; then meet the other
    // waves.  A plain barrier: the fence of __syncthreads would also wait for
    // the stages in flight.
    // Barriers come every KB stages.  At the barrier before stages kt .. kt+KB-1
    // every wave has read stages up to kt (stage s's fragments are read while
    // stage s-1 computes), so their buffers take the copies of this iteration;
    // stages kt+1 .. kt+KB (read in this iteration) must have landed, while the
    // copies issued after them may stay in flight.
    constexpr int KB = C::KB;
    const int n_kt = a.d_model / BK;                    // a multiple of KB
    auto stage_barrier = [&](int kt) __attribute__((always_inline)) {
        const int issued = min(n_kt - 1, max(NS - 1, kt - KB + NS));
        wait_stages_ahead<kInst, NS - KB>(max(0, issued - min(kt + KB, n_kt - 1)));
        __builtin_amdgcn_s_barrier();
    };

    // acc[i][t]: tokens wm*WM + 16 i + (lane % 16), features wn*128 + 16 t + 4 (lane / 16) + e
    f32x4 acc[WMF][8];
#pragma unroll
    for (int i = 0; i < WMF; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 cx[WMF], cw[8];
    if constexpr (KB == 1) {
        // One stage per barrier: the copies for stage kt + NS go out during
        // stage kt, into the buffer stage kt was read from before the barrier.
        // Every iteration (and the prologue) issues one whole stage: past the
        // last stage, copies of one cached 16-byte line into the buffer just
        // freed, never read.  So each wait is one constant count and no branch
        // surrounds a copy.
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < kInst; ++i) issue_one(s, min(s, n_kt - 1), i);
        // stage `next` has landed; the NS - 2 stages issued after it may
        // still be in flight; this wave's fragment reads have returned
        auto stage_barrier1 = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * kInst, 0));
            __builtin_amdgcn_s_barrier();
        };
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 1) * kInst, 0));   // stage 0
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int t = 0; t < 8; ++t) cw[t] = read_w(0, t);
#pragma unroll
        for (int i = 0; i < WMF; ++i) cx[i] = read_x(0, i);
        for (int kt = 0; kt < n_kt; ++kt) {
            // After the last stage the reads below are of a stale buffer and go
            // unused: kept unconditional so the fragment registers need no merge.
            stage_barrier1();                           // stage kt + 1
            const bool more = kt + NS < n_kt;
            const int kc = more ? kt + NS : 0;
            bf16x8 nx[WMF], nw[8];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < WMF; ++i) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cw[t], cx[i], acc[i][t], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < C::kCopyPerGroup; ++c)
                    if (i * C::kCopyPerGroup + c < kInst) {
                        const int ci = i * C::kCopyPerGroup + c;
                        const int j = wave * kInst + ci;
                        // past the last stage every lane reads W's first 16
                        // bytes (one cached line) into the freed buffer
                        copy16_to_lds(more ? src[ci] + kc * BK : (const uint16_t*)a.w,
                                      lds0 + (uint32_t)((kt % NS) * kStage + j * 512) * 2u);
                    }
                // the next step's W fragments early (its first group needs all
                // eight), x fragment i once this group has used its register
#pragma unroll
                for (int c = 0; c < C::kWPerGroup; ++c)
                    if (i * C::kWPerGroup + c < 8) nw[i * C::kWPerGroup + c] = read_w(kt + 1, i * C::kWPerGroup + c);
                nx[i] = read_x(kt + 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < WMF; ++i) cx[i] = nx[i];
#pragma unroll
            for (int t = 0; t < 8; ++t) cw[t] = nw[t];
        }
        // the copies of the last iterations land before the epilogue reuses
        // the ring
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    } else {
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < n_kt)
#pragma unroll
            for (int i = 0; i < kInst; ++i) issue_one(s, s, i);
    wait_stages_ahead<kInst, NS - KB>(min(NS - KB, n_kt - 1));   // stage 0 (and maybe more) landed
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int t = 0; t < 8; ++t) cw[t] = read_w(0, t);
#pragma unroll
    for (int i = 0; i < WMF; ++i) cx[i] = read_x(0, i);
    for (int kt = 0; kt < n_kt; kt += KB) {
        stage_barrier(kt);
#pragma unroll
        for (int sub = 0; sub < KB; ++sub) {
            const int s = kt + sub;
            // the stage whose buffer (read before this barrier) takes copies now
            const int refill = s - KB + 1 + NS;
            const bool more = refill >= NS && refill < n_kt;
            bf16x8 nx[WMF], nw[8];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < WMF; ++i) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cw[t], cx[i], acc[i][t], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < C::kCopyPerGroup; ++c)
                    if (more && i * C::kCopyPerGroup + c < kInst)
                        issue_one(refill % NS, refill, i * C::kCopyPerGroup + c);
                // the next stage's W fragments early (its first group needs all
                // eight), x fragment i once this group has used its register.
                // After the last stage these read a stale buffer and go unused:
                // kept unconditional so the fragment registers need no merge.
#pragma unroll
                for (int c = 0; c < C::kWPerGroup; ++c)
                    if (i * C::kWPerGroup + c < 8) nw[i * C::kWPerGroup + c] = read_w(s + 1, i * C::kWPerGroup + c);
                nx[i] = read_x(s + 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < WMF; ++i) cx[i] = nx[i];
#pragma unroll
            for (int t = 0; t < 8; ++t) cw[t] = nw[t];
        }
    }
    }

    // ---- epilogue: rotate in registers (pairs are n-tiles t and t+4), bf16, via LDS to rows ----
    const int part = col0 / a.n_out;                    // 0 = Q, 1 = K, 2 = V (tiles never straddle parts)
    const int cpart = col0 % a.n_out + wn * 128;        // first column of this wave's head within the part
    if (part < 2 && !RAW) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double fr = s_theta[t * 16 + g * 4 + e];
#pragma unroll
                for (int i = 0; i < WMF; ++i) {
                    // the angle in revolutions, reduced in fp64 to |rev| <= 1/2;
                    // hardware sin/cos take revolutions (library sincosf here
                    // would push the accumulators out of registers)
                    double rv = (double)s_pos[wm * WM + i * 16 + ln] * fr;
                    rv -= rint(rv);
                    const float rev = (float)rv;
                    const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
                    const float x0 = acc[i][t][e], x1 = acc[i][t + 4][e];
                    acc[i][t][e] = x0 * cs - x1 * sn;
                    acc[i][t + 4][e] = x1 * cs + x0 * sn;
                }
            }
    }
    __syncthreads();                                    // every wave is done reading the stages
    if (EPI == kEpiRotE4M3 && part > 0) {
        // this wave's WM x 128 tile of codes, rows of 8 pieces of 16 bytes,
        // piece p of row r stored at piece p ^ (r % 8)
        uint8_t* t8 = reinterpret_cast<uint8_t*>(smem) + wave * (WM * 128);
#pragma unroll
        for (int i = 0; i < WMF; ++i)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int r = i * 16 + ln, c = t * 16 + g * 4;
                *(uint32_t*)(&t8[r * 128 + (((c >> 4) ^ (r & 7)) << 4) + (c & 15)]) =
                    e4m3x4(acc[i][t][0], acc[i][t][1], acc[i][t][2], acc[i][t][3]);
            }
        __syncthreads();
        // WM rows x 8 pieces of 16 B; a pass covers 8 rows
        for (int pass = 0; pass < WM / 8; ++pass) {
            const int r = pass * 8 + (lane >> 3), pc = lane & 7;
            const int grow = row0 + wm * WM + r;
            if (grow >= a.R) break;
            const int sl = s_slot[wm * WM + r];
            if (sl < 0 || (int64_t)sl >= a.cache_rows) continue;
            const u32x4 v = *(const u32x4*)(&t8[r * 128 + ((pc ^ (r & 7)) << 4)]);
            uint8_t* d8 = (uint8_t*)(part == 1 ? a.k_cache : a.v_cache) + (int64_t)sl * a.n_out;
            *(u32x4*)(d8 + cpart + pc * 16) = v;
        }
        return;
    }
    // this wave's WM x 128 bf16 tile, rows of 16 pieces of 16 bytes, piece p
    // of row r stored at piece p ^ (r % 16)
    uint16_t* tile = smem + wave * (WM * 128);
#pragma unroll
    for (int i = 0; i < WMF; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int r = i * 16 + ln, c = t * 16 + g * 4;
            uint2 v;
            v.x = pack_bf16x2(acc[i][t][0], acc[i][t][1]);
            v.y = pack_bf16x2(acc[i][t][2], acc[i][t][3]);
            *(uint2*)(&tile[r * 128 + (((c >> 3) ^ (r & 15)) << 3) + (c & 7)]) = v;
        }
    __syncthreads();
    // WM rows x 16 pieces of 16 B; a pass covers 4 rows
    for (int pass = 0; pass < WM / 4; ++pass) {
        const int r = pass * 4 + (lane >> 4), pc = lane & 15;
        const int grow = row0 + wm * WM + r;
        if (grow >= a.R) break;
        const u32x4 v = *(const u32x4*)(&tile[r * 128 + ((pc ^ (r & 15)) << 3)]);
        uint16_t* dst;
        if (RAW) {
            dst = a.raw_out + (int64_t)grow * 3 * a.n_out + part * a.n_out;
        } else if (part == 0) {
            dst = a.q_out + (int64_t)grow * a.n_out;
        } else {
            const int sl = s_slot[wm * WM + r];
            if (sl < 0 || (int64_t)sl >= a.cache_rows) continue;
            dst = (part == 1 ? a.k_cache : a.v_cache) + (int64_t)sl * a.n_out;
        }
        *(u32x4*)(dst + cpart + pc * 8) = v;
    }
}


// Cache-phase projection (R <= 128 rows).  Streaming W from HBM is the whole
// HBM cost (W is read exactly once); every workgroup also re-reads all of x
// from L2.  Each of 256-odd workgroups owns PP = 8 NT rotation pairs (columns
// c and c + D/2 of one head, over the flattened Q/K/V pair list), i.e. 2 PP
// rows of W, and all R rows of x (padded to 16 MT).  Measured on MI355X: a
// compute unit keeps a bounded amount of memory traffic in flight, and the
// L2-hit x copies share it with the HBM-miss W copies, so neither a deeper
// ring nor larger copies moves the kernel; staggering the workgroups' K order
// (so the compute units of one L2 do not read the same x lines at once) does
// a little.
constexpr int kStreamMaxRows = 128;
constexpr int kMaxSeqPaged = 1024;        // paged mode: cu_q entries staged (n_seq + 1 <= this + 1)

// Cache-phase projection with a shared ring: the four waves fill one ring of
// 128-wide K stages together (256-byte row pieces, two whole L2 lines per row
// per copy; each wave issues a quarter of a stage's copies) and each wave
// takes one 32-wide k-step of every stage for all rows and pairs.  One
// LDS-only barrier per stage publishes it (every wave's copies have landed)
// and frees the oldest slot (every wave has read it).  With all 160 KiB of LDS
// in one ring, five 32 KiB stages at 72 rows: four in flight per compute unit.
constexpr int kStream2Lds = 160 * 1024;

template <int MT, int NT>
struct Stream2Cfg {
    static constexpr int kKC = 128;                               // K elements per stage
    static constexpr int kRows = 16 * (MT + NT);                  // x (padded), then W lo, W hi
    static constexpr int kStageBytes = kRows * kKC * 2;
    static constexpr int kInst = kStageBytes / 1024 / 4;          // 1 KiB copies per wave per stage
    static constexpr int kNS0 = kStream2Lds / kStageBytes;
    static constexpr int kNS = kNS0 < 6 ? kNS0 : 6;
    static constexpr int kPP = NT * 8;                            // pairs per workgroup
    static constexpr int kLdc = 2 * kPP + 4;                      // partial-sum row stride (floats)
    static constexpr int kCsBytes = 4 * MT * 16 * kLdc * 4 + kPP * 8;
    static constexpr int kSmem = kNS * kStageBytes > kCsBytes ? kNS * kStageBytes : kCsBytes;
};

template <int MT, int NT, bool PAGED>
__global__ __launch_bounds__(256, 1) void qkv_stream2_kernel(QkvArgs a, int n_pairs) {
    using C = Stream2Cfg<MT, NT>;
    constexpr int KC = C::kKC, NS = C::kNS, kInst = C::kInst, kPP = C::kPP;
    constexpr int kStageBytes = C::kStageBytes;
    static_assert(NS >= 2 && (NS - 1) * kInst < 64, "ring depth / wait count");
    static_assert(C::kSmem <= kStream2Lds, "LDS budget");
    static_assert(kStageBytes >= (kMaxSeqPaged + 1 + kStreamMaxRows) * 4, "cu_q and positions fit a ring slot");
    constexpr int kPieces = kPP / 8;                       // 8-pair output pieces per row
    constexpr int kItems = (kStreamMaxRows * kPieces + 255) / 256;   // epilogue items per thread
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, ln = lane & 15;
    const int D = a.head_dim, half = D >> 1, H = a.n_out / D;
    const int p0 = blockIdx.x * kPP;
    const int n_st = a.d_model / KC;
    // rotation frequency of this thread's pair (threads < kPP), formed before
    // the main loop so the fp64 pow's latency is hidden behind it (at the end
    // of the kernel it cost ~1 us of the batch-1 launch); staged to LDS in
    // the epilogue
    double theta_own = 0.0;
    if (tid < kPP) {
        const int p = min(p0 + tid, n_pairs - 1);
        theta_own = pow((double)a.rope_base, -2.0 * (p % half) / D) * (1.0 / kTwoPi);   // revolutions per position
    }

    // epilogue items (row, 8-pair piece) of this thread: idx = tid + 256 k;
    // their positions and slots are first used after the ring has drained.
    // Paged mode: cu_q and the rows' logical positions are copied straight
    // into the ring's last slot (which no copy fills before the first barrier
    // of the main loop), ahead of every other copy; the slot lookups follow
    // once the ring is running.
    int it_pos[kItems], it_slot[kItems], it_log[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int idx = tid + 256 * k;
        const int r = min(idx / kPieces, a.R - 1);
        it_log[k] = 0;
        if constexpr (PAGED) {
            it_pos[k] = a.pos[r];
        } else if (!a.raw_out) {
            it_pos[k] = a.pos[r];
            it_slot[k] = a.slot[r];
        } else {
            it_pos[k] = 0;
            it_slot[k] = -1;
        }
    }
    // [0, kMaxSeqPaged] cu_q, then [kMaxSeqPaged + 1, + kStreamMaxRows) logical positions
    constexpr int kMetaCopies = (kMaxSeqPaged + 1 + kStreamMaxRows + 255) / 256;   // 4-byte copies per wave
    const uint32_t meta0 = lds_addr(smem + (NS - 1) * kStageBytes);
    if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < kMetaCopies; ++i) {
            const int e = 256 * i + 64 * wave + lane;
            const int32_t* src = e <= kMaxSeqPaged ? a.cu_q + min(e, a.n_seq)
                                                   : a.logical + min(e - (kMaxSeqPaged + 1), a.R - 1);
            copy4_to_lds(src, __builtin_amdgcn_readfirstlane(meta0 + (uint32_t)(256 * i + 64 * wave) * 4));
        }
    }

    // copy sources: copy i of this wave covers staged rows 4 (4 i + wave) ..
    // +3 (so copy i of the four waves is one 16-row tile: x for i < MT, W
    // rows after), lane -> row + lane / 16 and the 16-byte slot lane % 16 of
    // its place; the logical slot stored there is XOR-swizzled by the row, so
    // the 16 rows a fragment read touches sit in 16 distinct bank groups
    const uint16_t* src[kInst];
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
        const int r = 4 * (4 * i + wave) + (lane >> 4);
        const int ls = (lane & 15) ^ (r & 15);
        const uint16_t* row_ptr;
        if (r < MT * 16) {
            row_ptr = a.x + (int64_t)min(r, a.R - 1) * a.d_model;          // padding rows repeat a real row
        } else {
            const int wr = r - MT * 16;                                      // 0 .. 2 PP - 1
            const int p = min(p0 + (wr % kPP), n_pairs - 1);                 // past the last pair: repeat it
            const int hp = p / half, i_pair = p % half;
            const int part = hp / H, head = hp % H;
            const int64_t wrow = (int64_t)part * a.n_out + head * D + i_pair + (wr >= kPP ? half : 0);
            row_ptr = a.w + wrow * a.d_model;
        }
        src[i] = row_ptr + ls * 8;
    }
    const uint32_t ring0 = lds_addr(smem);
    // workgroups start at different K stages (and wrap), so the compute units
    // sharing an L2 do not all read the same x lines at the same moment
    const int k_off = (int)((blockIdx.x * 7u) % (unsigned)n_st);
    auto issue = [&](int slot, int j) __attribute__((always_inline)) {
        int c = min(j, n_st - 1) + k_off;                  // past the end: re-read the last stage
        c -= c >= n_st ? n_st : 0;
        const uint32_t base = __builtin_amdgcn_readfirstlane(ring0 + slot * kStageBytes + wave * 1024);
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            // W rows are read once: non-temporal, so they do not push x (which
            // every workgroup re-reads) out of L2 (the choice is per copy index,
            // the same for every wave: no branch)
            if (i >= MT) copy16_to_lds_nt(src[i] + c * KC, base + i * 4096);
            else copy16_to_lds(src[i] + c * KC, base + i * 4096);
        }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);

    if constexpr (PAGED) {
        // sequence of each item row from cu_q, then its page entry
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 1) * kInst, 15));   // the metadata, not the stages
        lds_sync();                                        // every wave's metadata copies
        const int* s_cuq = reinterpret_cast<const int*>(smem + (NS - 1) * kStageBytes);
        const int* s_log = s_cuq + kMaxSeqPaged + 1;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int r = min((tid + 256 * k) / kPieces, a.R - 1);
            int lo = 0, hi = a.n_seq - 1;                  // last b with cu_q[b] <= r
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_cuq[mid] <= r) lo = mid; else hi = mid - 1;
            }
            const int l = s_log[r];
            it_log[k] = l;
            const bool in_seq = r >= s_cuq[lo] && r < s_cuq[lo + 1];
            const int j = l >= 0 ? l / a.page_size : -1;
            const bool ok = in_seq && j >= 0 && j < a.max_pages;
            // the page entry (-1: no slot), resolved after the ring drains
            it_slot[k] = ok ? a.page_table[(int64_t)lo * a.max_pages + j] : -1;
        }
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ls = 4 * wave + g;                           // this lane's logical slot: k-step = wave
    for (int j = 0; j < n_st; ++j) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * kInst, 15));   // this wave's copies of stage j
        lds_sync();                                        // everyone's copies; everyone is done with j - 1
        // fragment reads ahead of the next stage's copies
        const uint16_t* st = reinterpret_cast<const uint16_t*>(smem + (j % NS) * kStageBytes);
        bf16x8 xf[MT], wf[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int r = MT * 16 + t * 16 + ln;
            wf[t] = *(const bf16x8*)(st + r * KC + ((ls ^ (r & 15)) * 8));
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int r = m * 16 + ln;
            xf[m] = *(const bf16x8*)(st + r * KC + ((ls ^ (r & 15)) * 8));
        }
        issue((j + NS - 1) % NS, j + NS - 1);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[m], wf[t], acc[m][t], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));        // drain the re-read stages
    __syncthreads();
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int idx = tid + 256 * k;
            const int r = idx / kPieces;
            const int page = it_slot[k];
            const int l = it_log[k];
            it_slot[k] = (page >= 0 && page < a.pool_pages) ? page * a.page_size + l % a.page_size : -1;
            if (blockIdx.x == 0 && a.slot_out && idx % kPieces == 0 && r < a.R) a.slot_out[r] = it_slot[k];
        }
    }

    // ---- epilogue: per-wave fp32 partials [row][2 PP] in LDS, summed, rotated, stored ----
    float* Cs = reinterpret_cast<float*>(smem);
    constexpr int kLdc = C::kLdc, kRowsPad = MT * 16;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Cs[(wave * kRowsPad + m * 16 + g * 4 + e) * kLdc + t * 16 + ln] = acc[m][t][e];
    double* s_theta = reinterpret_cast<double*>(Cs + 4 * kRowsPad * kLdc);
    if (tid < kPP) s_theta[tid] = theta_own;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int idx = tid + 256 * k;
        const int r = idx / kPieces, q = idx % kPieces;
        const int p = p0 + q * 8;
        if (r >= a.R || p >= n_pairs) continue;
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sl = 0.f, sh = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                sl += Cs[(w * kRowsPad + r) * kLdc + q * 8 + e];
                sh += Cs[(w * kRowsPad + r) * kLdc + kPP + q * 8 + e];
            }
            lo[e] = sl;
            hi[e] = sh;
        }
        const int hp = p / half, i0 = p % half;            // a piece never straddles a head (half % 8 == 0)
        const int part = hp / H, head = hp % H;
        uint16_t* dst;
        int64_t cache_off = 0;                           // element offset of the cache row
        if (!PAGED && a.raw_out) {
            dst = a.raw_out + (int64_t)r * 3 * a.n_out + part * a.n_out;
        } else if (part == 0) {
            dst = a.q_out + (int64_t)r * a.n_out;
        } else {
            const int sl = it_slot[k];
            if (sl < 0 || (int64_t)sl >= a.cache_rows) continue;
            cache_off = (int64_t)sl * a.n_out;
            dst = (part == 1 ? a.k_cache : a.v_cache) + cache_off;
        }
        if (part < 2 && (PAGED || !a.raw_out)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // the angle in revolutions, reduced in fp64 to |rev| <= 1/2 (the
                // hardware sin/cos take revolutions)
                double rv = (double)it_pos[k] * s_theta[q * 8 + e];
                rv -= rint(rv);
                const float rev = (float)rv;
                const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                const float x0 = lo[e], x1 = hi[e];
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
        if (part > 0 && a.kv_fp8) {
            uint8_t* d8 = (uint8_t*)(part == 1 ? a.k_cache : a.v_cache) + cache_off + head * D + i0;
            *(uint2*)d8 = make_uint2(e4m3x4(lo[0], lo[1], lo[2], lo[3]), e4m3x4(lo[4], lo[5], lo[6], lo[7]));
            *(uint2*)(d8 + half) = make_uint2(e4m3x4(hi[0], hi[1], hi[2], hi[3]), e4m3x4(hi[4], hi[5], hi[6], hi[7]));
            continue;
        }
        *(u32x4*)(dst + head * D + i0) = plo;
        *(u32x4*)(dst + head * D + i0 + half) = phi;
    }
}

// Mid-size projection (a few hundred rows): the streaming design above on a
// two-dimensional grid.  A workgroup owns PP = 8 NT rotation pairs (2 PP rows
// of W) and one group of 16 MT rows of x.  Its four waves split each 64-wide
// K stage into its two 32-wide k-steps (wave & 1) and the row tiles into two
// halves (wave >> 1), so a wave reads MT / 2 + NT fragments for MT / 2 x NT
// MFMAs per stage; stages of 64 keep four or five of them in LDS at tiles of
// 160 x 96 or 128 x 192.  A workgroup moves (16 MT + 2 PP) rows of 2 d_model
// bytes through its compute unit instead of all R rows of x, and the row
// groups of one pair group run on one XCD (dispatch order) with the same K
// order, so they can share their W lines in L2 (at 288 rows the counters
// show W fetched about 1.5 times).
constexpr int kMidLds = 160 * 1024;

template <int MT, int NT>
struct MidCfg {
    static constexpr int kKC = 64;                                // K elements per stage
    static constexpr int kRows = 16 * (MT + NT);                  // x rows of the group, then W lo, W hi
    static constexpr int kStageBytes = kRows * kKC * 2;
    static constexpr int kInst = kRows / 32;                      // 1 KiB copies (8 rows) per wave per stage
    static constexpr int kPP = NT * 8;                            // pairs per workgroup
    static constexpr int kMW = MT / 2;                            // row tiles per wave
    static constexpr int kLdc = 2 * kPP + 4;                      // summed tile row stride (floats)
    static constexpr int kPartBytes = MT * NT * 1024;             // the odd k-step waves' partial sums
    static constexpr int kSumBytes = MT * 16 * kLdc * 4 + kPP * 8;   // summed tile, then frequencies
    static constexpr int kNS0 = kMidLds / kStageBytes;
    static constexpr int kNS = kNS0 < 6 ? kNS0 : 6;
    static constexpr int kEpi = kPartBytes > kSumBytes ? kPartBytes : kSumBytes;
    static constexpr int kSmem = kNS * kStageBytes > kEpi ? kNS * kStageBytes : kEpi;
};

// Physical 16-byte slot of a logical slot in a 128-byte staged row: rows r
// and r + 1 share a 256-byte bank window, so the slot is XOR-ed with r / 2;
// any 16 consecutive rows read at one logical slot then touch 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int mid_swz(int row) { return (row >> 1) & 7; }

template <int MT, int NT, bool PAGED>
__global__ __launch_bounds__(256, 1) void qkv_mid_kernel(QkvArgs a, int n_pairs, int n_cg, int n_rg) {
    using C = MidCfg<MT, NT>;
    constexpr int KC = C::kKC, NS = C::kNS, kInst = C::kInst, kPP = C::kPP, MW = C::kMW;
    constexpr int kStageBytes = C::kStageBytes;
    constexpr int kRowsG = 16 * MT;                       // x rows per workgroup
    static_assert(MT % 2 == 0 && (MT + NT) % 2 == 0 && NT % 2 == 0, "wave split and whole copies");
    static_assert(NS >= 3 && (NS - 1) * kInst < 64, "ring depth / wait count");
    static_assert(C::kSmem <= kMidLds, "LDS budget");
    static_assert(kStageBytes >= (kMaxSeqPaged + 1 + kRowsG) * 4, "cu_q and positions fit a ring slot");
    constexpr int kPieces = kPP / 8;                       // 8-pair output pieces per row
    constexpr int kItems = (kRowsG * kPieces + 255) / 256; // epilogue items per thread
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ks = wave & 1, mh = wave >> 1;               // k-step of each stage, half of the row tiles
    const int g = lane >> 4, ln = lane & 15;
    const int D = a.head_dim, half = D >> 1, H = a.n_out / D;
    // pair group and row group: the n_rg row groups of a pair group are
    // dispatched to one XCD (workgroup b runs on XCD b % 8)
    int cg, rg;
    {
        const int b = blockIdx.x;
        if (n_cg % kNumXcd == 0) {
            const int i = b / kNumXcd;
            cg = b % kNumXcd + kNumXcd * (i / n_rg);
            rg = i % n_rg;
        } else {
            cg = b / n_rg;
            rg = b % n_rg;
        }
    }
    const int p0 = cg * kPP;
    const int row0 = rg * kRowsG;
    const int n_st = a.d_model / KC;
    double theta_own = 0.0;
    if (tid < kPP) {
        const int p = min(p0 + tid, n_pairs - 1);
        theta_own = pow((double)a.rope_base, -2.0 * (p % half) / D) * (1.0 / kTwoPi);   // revolutions per position
    }

    // epilogue items (local row, 8-pair piece): idx = tid + 256 k
    int it_pos[kItems], it_slot[kItems], it_log[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int idx = tid + 256 * k;
        const int r = min(row0 + idx / kPieces, a.R - 1);
        it_log[k] = 0;
        if constexpr (PAGED) {
            it_pos[k] = a.pos[r];
        } else if (!a.raw_out) {
            it_pos[k] = a.pos[r];
            it_slot[k] = a.slot[r];
        } else {
            it_pos[k] = 0;
            it_slot[k] = -1;
        }
    }
    // paged mode: cu_q, then the group's logical positions, copied into the
    // ring's last slot (no stage copy fills it before the main loop's first
    // barrier) ahead of every other copy
    constexpr int kMetaCopies = (kMaxSeqPaged + 1 + kRowsG + 255) / 256;   // 4-byte copies per wave
    const uint32_t meta0 = lds_addr(smem + (NS - 1) * kStageBytes);
    if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < kMetaCopies; ++i) {
            const int e = 256 * i + 64 * wave + lane;
            const int32_t* src = e <= kMaxSeqPaged ? a.cu_q + min(e, a.n_seq)
                                                   : a.logical + min(row0 + e - (kMaxSeqPaged + 1), a.R - 1);
            copy4_to_lds(src, __builtin_amdgcn_readfirstlane(meta0 + (uint32_t)(256 * i + 64 * wave) * 4));
        }
    }

    // copy sources: copy i of this wave covers staged rows 8 (4 i + wave) ..
    // +7 (x for i < MT / 2, W rows after), lane -> row + lane / 8 and the
    // 16-byte place lane % 8 of that row; the logical slot stored there is
    // swizzled by the row
    const uint16_t* src[kInst];
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
        const int r = 8 * (4 * i + wave) + (lane >> 3);
        const int ls = (lane & 7) ^ mid_swz(r);
        const uint16_t* row_ptr;
        if (r < kRowsG) {
            row_ptr = a.x + (int64_t)min(row0 + r, a.R - 1) * a.d_model;   // rows past R repeat a real row
        } else {
            const int wr = r - kRowsG;                                       // 0 .. 2 PP - 1
            const int p = min(p0 + (wr % kPP), n_pairs - 1);                 // past the last pair: repeat it
            const int hp = p / half, i_pair = p % half;
            const int part = hp / H, head = hp % H;
            const int64_t wrow = (int64_t)part * a.n_out + head * D + i_pair + (wr >= kPP ? half : 0);
            row_ptr = a.w + wrow * a.d_model;
        }
        src[i] = row_ptr + ls * 8;
    }
    const uint32_t ring0 = lds_addr(smem);
    // the row groups of a pair group walk K in the same order (shared W
    // lines); pair groups start at different stages
    const int k_off = (int)((cg * 7u) % (unsigned)n_st);
    auto issue = [&](int slot, int j) __attribute__((always_inline)) {
        int c = min(j, n_st - 1) + k_off;                  // past the end: re-read the last stage
        c -= c >= n_st ? n_st : 0;
        const uint32_t base = __builtin_amdgcn_readfirstlane(ring0 + slot * kStageBytes + wave * 1024);
#pragma unroll
        for (int i = 0; i < kInst; ++i) copy16_to_lds(src[i] + c * KC, base + i * 4096);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);

    if constexpr (PAGED) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 1) * kInst, 15));   // the metadata, not the stages
        lds_sync();
        const int* s_cuq = reinterpret_cast<const int*>(smem + (NS - 1) * kStageBytes);
        const int* s_log = s_cuq + kMaxSeqPaged + 1;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int rl = min((tid + 256 * k) / kPieces, kRowsG - 1);
            const int r = min(row0 + rl, a.R - 1);
            int lo = 0, hi = a.n_seq - 1;                  // last b with cu_q[b] <= r
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_cuq[mid] <= r) lo = mid; else hi = mid - 1;
            }
            const int l = s_log[r - row0];
            it_log[k] = l;
            const bool in_seq = r >= s_cuq[lo] && r < s_cuq[lo + 1];
            const int j = l >= 0 ? l / a.page_size : -1;
            const bool ok = in_seq && j >= 0 && j < a.max_pages;
            it_slot[k] = ok ? a.page_table[(int64_t)lo * a.max_pages + j] : -1;
        }
    }

    f32x4 acc[MW][NT];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ls = 4 * ks + g;                             // this lane's logical slot
    for (int j = 0; j < n_st; ++j) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * kInst, 15));   // this wave's copies of stage j
        lds_sync();                                        // everyone's copies; everyone is done with j - 1
        // the stage's fragment reads go out ahead of the next stage's copies
        // (issued after them, the copies delayed the reads the MFMAs wait for:
        // 288 rows 57.7 -> 50.3 us)
        const uint16_t* st = reinterpret_cast<const uint16_t*>(smem + (j % NS) * kStageBytes);
        bf16x8 xf[MW], wf[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int r = kRowsG + t * 16 + ln;
            wf[t] = *(const bf16x8*)(st + r * KC + ((ls ^ mid_swz(r)) * 8));
        }
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int r = (mh * MW + m) * 16 + ln;
            xf[m] = *(const bf16x8*)(st + r * KC + ((ls ^ mid_swz(r)) * 8));
        }
        issue((j + NS - 1) % NS, j + NS - 1);
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[m], wf[t], acc[m][t], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));        // drain the re-read stages
    __syncthreads();
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int idx = tid + 256 * k;
            const int r = row0 + idx / kPieces;
            const int page = it_slot[k];
            const int l = it_log[k];
            it_slot[k] = (page >= 0 && page < a.pool_pages) ? page * a.page_size + l % a.page_size : -1;
            if (cg == 0 && a.slot_out && idx % kPieces == 0 && idx / kPieces < kRowsG && r < a.R)
                a.slot_out[r] = it_slot[k];
        }
    }

    // ---- epilogue: the odd k-step waves hand their sums to the even ones
    // (same fragment layout), which store the [row][2 PP] fp32 tile; then
    // every thread rotates and stores 8-pair pieces ----
    f32x4* part = reinterpret_cast<f32x4*>(smem);
    if (ks == 1) {
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) part[((mh * MW + m) * NT + t) * 64 + lane] = acc[m][t];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 o = part[((mh * MW + m) * NT + t) * 64 + lane];
                acc[m][t] += o;
            }
    }
    __syncthreads();
    float* Cs = reinterpret_cast<float*>(smem);
    constexpr int kLdc = C::kLdc;
    if (ks == 0) {
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Cs[((mh * MW + m) * 16 + g * 4 + e) * kLdc + t * 16 + ln] = acc[m][t][e];
    }
    double* s_theta = reinterpret_cast<double*>(Cs + kRowsG * kLdc);
    if (tid < kPP) s_theta[tid] = theta_own;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int idx = tid + 256 * k;
        const int rl = idx / kPieces, q = idx % kPieces;
        const int r = row0 + rl;
        const int p = p0 + q * 8;
        if (rl >= kRowsG || r >= a.R || p >= n_pairs) continue;
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = Cs[rl * kLdc + q * 8 + e];
            hi[e] = Cs[rl * kLdc + kPP + q * 8 + e];
        }
        const int hp = p / half, i0 = p % half;            // a piece never straddles a head (half % 8 == 0)
        const int prt = hp / H, head = hp % H;
        uint16_t* dst;
        int64_t cache_off = 0;
        if (!PAGED && a.raw_out) {
            dst = a.raw_out + (int64_t)r * 3 * a.n_out + prt * a.n_out;
        } else if (prt == 0) {
            dst = a.q_out + (int64_t)r * a.n_out;
        } else {
            const int sl = it_slot[k];
            if (sl < 0 || (int64_t)sl >= a.cache_rows) continue;
            cache_off = (int64_t)sl * a.n_out;
            dst = (prt == 1 ? a.k_cache : a.v_cache) + cache_off;
        }
        if (prt < 2 && (PAGED || !a.raw_out)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double rv = (double)it_pos[k] * s_theta[q * 8 + e];
                rv -= rint(rv);
                const float rev = (float)rv;
                const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                const float x0 = lo[e], x1 = hi[e];
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
        if (prt > 0 && a.kv_fp8) {
            uint8_t* d8 = (uint8_t*)(prt == 1 ? a.k_cache : a.v_cache) + cache_off + head * D + i0;
            *(uint2*)d8 = make_uint2(e4m3x4(lo[0], lo[1], lo[2], lo[3]), e4m3x4(lo[4], lo[5], lo[6], lo[7]));
            *(uint2*)(d8 + half) = make_uint2(e4m3x4(hi[0], hi[1], hi[2], hi[3]), e4m3x4(hi[4], hi[5], hi[6], hi[7]));
            continue;
        }
        *(u32x4*)(dst + head * D + i0) = plo;
        *(u32x4*)(dst + head * D + i0 + half) = phi;
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

enum QkvKind { kSkinny, kTiled128, kGemm, kMid };
// tile shapes of qkv_gemm_kernel (rows x columns, workgroups per compute unit)
enum GemmShape {
    kG256x256, kG128x256, kG128x256o2, kG64x256, kG64x256o2, kG256x128, kG256x128o2, kG128x128, kG128x128o2,
    kNumShapes
};
constexpr int kShapeBM[kNumShapes] = {256, 128, 128, 64, 64, 256, 256, 128, 128};
constexpr int kShapeBN[kNumShapes] = {256, 256, 256, 256, 256, 128, 128, 128, 128};
constexpr int kShapeOcc[kNumShapes] = {1, 1, 2, 1, 2, 1, 2, 1, 2};
// Time of one workgroup alone on a compute unit (T1) and of two sharing one
// (T2), measured on MI355X for the LLaDA-8B-shaped projection (d_model 4096,
// 12288 columns; microseconds, used only to rank the shapes)
constexpr double kShapeT1[kNumShapes] = {119, 85, 91, 69, 74, 83, 73, 55, 55};
constexpr double kShapeT2[kNumShapes] = {0, 0, 125, 0, 110, 0, 133, 0, 85};
constexpr const char* kShapeName[kNumShapes] = {"g256x256", "g128x256", "g128x256o2", "g64x256", "g64x256o2",
                                                "g256x128", "g256x128o2", "g128x128", "g128x128o2"};

// tile shapes of qkv_mid_kernel (16 MT rows of x by 16 NT rows of W) and the
// time of one workgroup alone on a compute unit (microseconds, measured on
// MI355X for the LLaDA-8B-shaped projection; used only to rank the shapes)
enum MidShape { kM6x6, kM10x6, kM12x6, kM16x6, kM4x12, kM8x12, kNumMid };
constexpr int kMidMT[kNumMid] = {6, 10, 12, 16, 4, 8};
constexpr int kMidNT[kNumMid] = {6, 6, 6, 6, 12, 12};
constexpr double kMidT1[kNumMid] = {37, 47, 57, 68, 43, 63};
constexpr const char* kMidName[kNumMid] = {"mid6x6", "mid10x6", "mid12x6", "mid16x6", "mid4x12", "mid8x12"};

struct QkvPlan {
    QkvKind kind;
    GemmShape shape;
    MidShape mid;
    int bm, n_mtiles, n_ntiles, n_ktiles;
    int n_cg, n_rg;          // kMid: pair groups and row groups
};

// Cache-phase row counts (R <= 128) take the weight-streaming kernel
// (d_model a multiple of 128).  Larger R takes qkv_gemm_kernel (head_dim 128,
// whole heads per wave) or qkv_mid_kernel in the shape with the least
// estimated time: the workgroups the busiest compute unit runs (spread over
// 256 units), alone or in pairs, at the measured time of each.  None splits K
// across workgroups, so no workspace is needed.  Shapes the GEMM cannot take
// fall back to the 128 x 128 LDS-tiled kernel.
// The qkv_kernel tuning override (DLLM_QKV_KERNEL, read once per process, or
// dllm_set_tuning: tiled|gemm|g128x256|...) forces the choice where the shape
// allows it.
QkvPlan plan_bf16(int R, int d_model, int n_out, int head_dim) {
    QkvPlan p{};
    const bool gemm_ok = head_dim == 128 && n_out % 256 == 0 && d_model % (kGBK * kGemmKB) == 0;
    if (R <= 128 && d_model % 128 == 0) p.kind = kSkinny;
    else p.kind = gemm_ok ? kGemm : kTiled128;
    p.shape = kG256x256;
    const int n_pairs = 3 * n_out / 2;
    const bool mid_ok = R > 128 && d_model % 64 == 0 && head_dim % 16 == 0;
    double best = 0.0;
    if (p.kind == kGemm) {
        for (int sh = 0; sh < kNumShapes; ++sh) {
            const int64_t tiles = (int64_t)((R + kShapeBM[sh] - 1) / kShapeBM[sh]) * (3 * n_out / kShapeBN[sh]);
            // workgroups the busiest compute unit runs, in pairs where two fit
            const int64_t load = (tiles + kNumCu - 1) / kNumCu;
            const double t = kShapeOcc[sh] == 2 ? (double)(load / 2) * kShapeT2[sh] + (double)(load % 2) * kShapeT1[sh]
                                                : (double)load * kShapeT1[sh];
            if (sh == 0 || t < best) {
                best = t;
                p.shape = (GemmShape)sh;
            }
        }
    }
    // the mid-size kernel where its workgroups, spread over the compute
    // units, finish before the best GEMM tiling (or where the GEMM cannot run)
    auto mid_time = [&](int m) {
        const int64_t wgs = (int64_t)((R + 16 * kMidMT[m] - 1) / (16 * kMidMT[m])) *
                            ((n_pairs + 8 * kMidNT[m] - 1) / (8 * kMidNT[m]));
        return (double)((wgs + kNumCu - 1) / kNumCu) * kMidT1[m];
    };
    if (mid_ok) {
        for (int m = 0; m < kNumMid; ++m) {
            const double t = mid_time(m);
            if (p.kind != kMid && p.kind != kGemm) p.kind = kMid, p.mid = (MidShape)m, best = t;
            else if (t < best) p.kind = kMid, p.mid = (MidShape)m, best = t;
        }
    }
    if (const char* e = tuning_qkv_kernel()) {
        if (!strcmp(e, "tiled")) p.kind = kTiled128;
        else if (!strcmp(e, "gemm") && gemm_ok) p.kind = kGemm, p.shape = kG256x256;
        else {
            for (int sh = 0; sh < kNumShapes; ++sh)
                if (!strcmp(e, kShapeName[sh]) && gemm_ok) p.kind = kGemm, p.shape = (GemmShape)sh;
            for (int m = 0; m < kNumMid; ++m)
                if (!strcmp(e, kMidName[m]) && mid_ok) p.kind = kMid, p.mid = (MidShape)m;
        }
    }
    if (p.kind == kGemm) {
        p.bm = kShapeBM[p.shape];
        p.n_mtiles = (R + p.bm - 1) / p.bm;
        p.n_ntiles = 3 * n_out / kShapeBN[p.shape];
    } else if (p.kind == kMid) {
        p.bm = 16 * kMidMT[p.mid];
        p.n_rg = (R + p.bm - 1) / p.bm;
        p.n_cg = (n_pairs + 8 * kMidNT[p.mid] - 1) / (8 * kMidNT[p.mid]);
        p.n_mtiles = p.n_rg;
        p.n_ntiles = p.n_cg;
    } else {
        p.bm = R <= 64 ? 64 : 128;
        p.n_mtiles = (R + p.bm - 1) / p.bm;
        p.n_ntiles = 3 * n_out / kBN;
    }
    p.n_ktiles = d_model / kBK;
    return p;
}

template <int WMF, int WGM, int OCC>
void launch_gemm(const QkvArgs& a, const QkvPlan& p, hipStream_t stream) {
    const unsigned tiles = (unsigned)((int64_t)p.n_mtiles * p.n_ntiles);
    if (a.raw_out)
        hipLaunchKernelGGL((qkv_gemm_kernel<WMF, WGM, OCC, kEpiRaw>), dim3(tiles), dim3(256), 0, stream, a,
                           p.n_mtiles, p.n_ntiles);
    else if (a.kv_fp8)
        hipLaunchKernelGGL((qkv_gemm_kernel<WMF, WGM, OCC, kEpiRotE4M3>), dim3(tiles), dim3(256), 0, stream, a,
                           p.n_mtiles, p.n_ntiles);
    else
        hipLaunchKernelGGL((qkv_gemm_kernel<WMF, WGM, OCC, kEpiRot>), dim3(tiles), dim3(256), 0, stream, a,
                           p.n_mtiles, p.n_ntiles);
}

int check_shape(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim) {
    DLLM_CHECK_ARG(n_rows >= 0 && d_model > 0 && n_heads > 0 && head_dim > 0);
    DLLM_CHECK_SUP(dt == DLLM_BF16 || dt == DLLM_F32 || dt == DLLM_BF16_E4M3KV);
    DLLM_CHECK_SUP(head_dim == 64 || head_dim == 128);
    DLLM_CHECK_SUP(dt != DLLM_BF16_E4M3KV || head_dim == 128);
    if (dt != DLLM_F32) {
        DLLM_CHECK_SUP((n_heads * head_dim) % kBN == 0);
        DLLM_CHECK_SUP(d_model % kBK == 0);
    }
    return DLLM_OK;
}

template <int NT, bool PAGED>
void launch_stream2_nt(int mt, dim3 grid, hipStream_t stream, const QkvArgs& a, int n_pairs) {
    switch (mt) {
        case 1: hipLaunchKernelGGL((qkv_stream2_kernel<1, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 2: hipLaunchKernelGGL((qkv_stream2_kernel<2, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 3: hipLaunchKernelGGL((qkv_stream2_kernel<3, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 4: hipLaunchKernelGGL((qkv_stream2_kernel<4, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 5: hipLaunchKernelGGL((qkv_stream2_kernel<5, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 6: hipLaunchKernelGGL((qkv_stream2_kernel<6, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        case 7: hipLaunchKernelGGL((qkv_stream2_kernel<7, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
        default: hipLaunchKernelGGL((qkv_stream2_kernel<8, NT, PAGED>), grid, dim3(256), 0, stream, a, n_pairs); break;
    }
}

template <bool PAGED>
void launch_stream(int mt, int nt, dim3 grid, hipStream_t stream, const QkvArgs& a, int n_pairs) {
    if (nt == 3) launch_stream2_nt<3, PAGED>(mt, grid, stream, a, n_pairs);
    else if (nt == 2) launch_stream2_nt<2, PAGED>(mt, grid, stream, a, n_pairs);
    else launch_stream2_nt<1, PAGED>(mt, grid, stream, a, n_pairs);
}

template <int MT, int NT>
void launch_mid_mt(bool paged, const QkvArgs& a, const QkvPlan& p, int n_pairs, hipStream_t stream) {
    const dim3 grid((unsigned)(p.n_cg * p.n_rg));
    if (paged)
        hipLaunchKernelGGL((qkv_mid_kernel<MT, NT, true>), grid, dim3(256), 0, stream, a, n_pairs, p.n_cg, p.n_rg);
    else
        hipLaunchKernelGGL((qkv_mid_kernel<MT, NT, false>), grid, dim3(256), 0, stream, a, n_pairs, p.n_cg, p.n_rg);
}

void launch_mid(bool paged, const QkvArgs& a, const QkvPlan& p, int n_pairs, hipStream_t stream) {
    switch (p.mid) {
        case kM6x6: launch_mid_mt<6, 6>(paged, a, p, n_pairs, stream); break;
        case kM10x6: launch_mid_mt<10, 6>(paged, a, p, n_pairs, stream); break;
        case kM12x6: launch_mid_mt<12, 6>(paged, a, p, n_pairs, stream); break;
        case kM16x6: launch_mid_mt<16, 6>(paged, a, p, n_pairs, stream); break;
        case kM4x12: launch_mid_mt<4, 12>(paged, a, p, n_pairs, stream); break;
        default: launch_mid_mt<8, 12>(paged, a, p, n_pairs, stream); break;
    }
}

}  // namespace

extern "C" size_t dllm_qkv_rope_cachewrite_workspace(dllm_dtype dt, int n_rows, int d_model,
                                                     int n_heads, int head_dim) {
    if (check_shape(dt, n_rows, d_model, n_heads, head_dim) != DLLM_OK) return 0;
    return 0;      // no kernel of this entry point needs scratch memory
}

namespace {

// paged: the slot mapping's arguments (nullptr page_table: slots given)
struct PagedArgs {
    int n_seq, max_pages, page_size;
    const int32_t* cu_q;
    const int32_t* logical;
    const int32_t* page_table;
    int32_t* slot_out;
};

int qkv_launch(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim, float rope_base,
               const void* x, const void* w_qkv, const int32_t* pos, const int32_t* slot, void* q_out,
               void* k_cache, void* v_cache, int64_t cache_rows, const PagedArgs* pg,
               hipStream_t stream, void* raw_out = nullptr) {
    const int n_out = n_heads * head_dim;
    const int pool_pages = pg ? (int)(cache_rows / pg->page_size < (1ll << 30) ? cache_rows / pg->page_size
                                                                               : (1ll << 30))
                              : 0;
    const bool e4m3 = dt == DLLM_BF16_E4M3KV;           // bf16 compute, one-byte caches
    if (e4m3) dt = DLLM_BF16;
    // the cache-phase and mid-size kernels form the slots from the block table
    // themselves; the others take them from a launch of their own
    const QkvKind kind0 = plan_bf16(n_rows, d_model, n_out, head_dim).kind;
    const bool slots_inside = dt == DLLM_BF16 && (kind0 == kSkinny || kind0 == kMid);
    if (pg && !slots_inside) {
        // slots first (the same rule, its own launch), then the slot-taking kernels
        int st = dllm_map_slots(pg->n_seq, n_rows, pg->page_size, pg->max_pages, pool_pages, pg->cu_q,
                                pg->logical, pg->page_table, pg->slot_out, stream);
        if (st != DLLM_OK) return st;
        slot = pg->slot_out;
    }
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
    QkvPlan p = plan_bf16(n_rows, d_model, n_out, head_dim);
    DLLM_CHECK_SUP(p.n_mtiles < 65536);
    QkvArgs a{};
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
    a.raw_out = (uint16_t*)raw_out;
    a.kv_fp8 = e4m3 ? 1 : 0;
    if (p.kind == kGemm) {
        DLLM_CHECK_SUP((int64_t)p.n_mtiles * p.n_ntiles < (1ll << 31));
        switch (p.shape) {
            case kG256x256: launch_gemm<8, 2, 1>(a, p, stream); break;
            case kG128x256: launch_gemm<4, 2, 1>(a, p, stream); break;
            case kG128x256o2: launch_gemm<4, 2, 2>(a, p, stream); break;
            case kG64x256: launch_gemm<2, 2, 1>(a, p, stream); break;
            case kG64x256o2: launch_gemm<2, 2, 2>(a, p, stream); break;
            case kG256x128: launch_gemm<4, 4, 1>(a, p, stream); break;
            case kG256x128o2: launch_gemm<4, 4, 2>(a, p, stream); break;
            case kG128x128: launch_gemm<2, 4, 1>(a, p, stream); break;
            default: launch_gemm<2, 4, 2>(a, p, stream); break;
        }
    } else if (p.kind == kMid) {
        DLLM_CHECK_SUP((int64_t)p.n_cg * p.n_rg < (1ll << 31));
        const int n_pairs = 3 * n_out / 2;
        if (pg) {
            a.cu_q = pg->cu_q;
            a.logical = pg->logical;
            a.page_table = pg->page_table;
            a.slot_out = pg->slot_out;
            a.n_seq = pg->n_seq;
            a.max_pages = pg->max_pages;
            a.page_size = pg->page_size;
            a.pool_pages = pool_pages;
        }
        launch_mid(pg != nullptr, a, p, n_pairs, stream);
    } else if (p.kind == kSkinny) {
        // pairs per workgroup: the most (up to 24) that still leaves >= 256 workgroups
        const int n_pairs = 3 * n_out / 2;
        const int nt = n_pairs >= 3 * 8 * kNumCu ? 3 : n_pairs >= 2 * 8 * kNumCu ? 2 : 1;
        const dim3 grid((n_pairs + 8 * nt - 1) / (8 * nt));
        if (pg) {
            a.cu_q = pg->cu_q;
            a.logical = pg->logical;
            a.page_table = pg->page_table;
            a.slot_out = pg->slot_out;
            a.n_seq = pg->n_seq;
            a.max_pages = pg->max_pages;
            a.page_size = pg->page_size;
            a.pool_pages = pool_pages;
            launch_stream<true>((n_rows + 15) / 16, nt, grid, stream, a, n_pairs);
        } else {
            launch_stream<false>((n_rows + 15) / 16, nt, grid, stream, a, n_pairs);
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

}  // namespace

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
    (void)workspace;
    (void)workspace_bytes;
    return qkv_launch(dt, n_rows, d_model, n_heads, head_dim, rope_base, x, w_qkv, pos, slot, q_out,
                      k_cache, v_cache, cache_rows, nullptr, stream);
}

extern "C" int dllm_qkv_rope_cachewrite_paged(dllm_dtype dt, int n_seq, int n_rows, int d_model,
                                              int n_heads, int head_dim, float rope_base,
                                              const void* x, const void* w_qkv, const int32_t* pos,
                                              const int32_t* cu_q, const int32_t* q_logical,
                                              const int32_t* page_table, int max_pages,
                                              int page_size, int32_t* slot, void* q_out,
                                              void* k_cache, void* v_cache, int64_t cache_rows,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
    int st = check_shape(dt, n_rows, d_model, n_heads, head_dim);
    if (st != DLLM_OK) return st;
    DLLM_CHECK_ARG(rope_base > 0.f && cache_rows >= 0);
    DLLM_CHECK_ARG(n_seq > 0 && max_pages > 0 && page_size > 0);
    DLLM_CHECK_SUP(n_seq <= kMaxSeqPaged);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(x && w_qkv && pos && cu_q && q_logical && page_table && slot && q_out && k_cache &&
                   v_cache);
    (void)workspace;
    (void)workspace_bytes;
    const PagedArgs pg{n_seq, max_pages, page_size, cu_q, q_logical, page_table, slot};
    return qkv_launch(dt, n_rows, d_model, n_heads, head_dim, rope_base, x, w_qkv, pos, nullptr, q_out,
                      k_cache, v_cache, cache_rows, &pg, stream);
}

extern "C" int dllm_qkv_project(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim,
                                const void* x, const void* w_qkv, void* qkv_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    int st = check_shape(dt, n_rows, d_model, n_heads, head_dim);
    if (st != DLLM_OK) return st;
    DLLM_CHECK_SUP(dt == DLLM_BF16);                    // no cache: plain bf16 only
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(x && w_qkv && qkv_out);
    (void)workspace;
    (void)workspace_bytes;
    return qkv_launch(dt, n_rows, d_model, n_heads, head_dim, 1.f, x, w_qkv, nullptr, nullptr, nullptr,
                      nullptr, nullptr, 0, nullptr, stream, qkv_out);
}
