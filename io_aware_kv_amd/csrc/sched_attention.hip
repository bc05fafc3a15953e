// a4-a5: block-table scheduled bidirectional attention over the paged KV cache,
// and one layer's term of the tracked-set score (formula (2)).
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page).  核心方法 and
// 技术新颖性: a block-table scheduled attention aligns variable-length query
// blocks with their KV blocks, without padding or synchronisation, and mixes
// sequences in the cache phase (a small window) with sequences in a full
// refresh inside one batch.  方法步骤详情 step 2: the queries attend
// bidirectionally over the full cache; step 4, formula (2): a_i sums, over
// layers, the attention key i receives from the masked-window queries,
// averaged over heads and window rows.
//
// bf16 kernel (gfx950).  One launch covers every (sequence, head, 128-row
// query tile[, key split]) item.  Items are decoded on the device from cu_q
// and kv_len: each workgroup scans the per-sequence item counts (no host
// round trip), and consecutive items (same head, next query tile) are placed
// on the same XCD so they share its L2 copy of the head's keys.  Four waves
// own 32 query rows each (two 16-row MFMA tiles, which share every K and V
// fragment read) and walk the item's keys in 64-key tiles gathered through the
// block table by direct-to-LDS copies, a two-stage ring so that two
// workgroups share a compute unit.  S^T = K Q^T and O^T = V^T P^T run on
// v_mfma_f32_16x16x32_bf16; the K rows fed to the first product are permuted
// so that the P^T fragment a lane holds covers 8 consecutive keys, and the
// matching V^T fragment is read from the row-major V tile with the gfx950 LDS
// transpose read.  Softmax is online in fp32 (base 2).
//
// Formula (2) needs the masked-window rows' final log-sum-exp.  When keys are
// not split, the workgroup of the sequence's first query tile keeps those
// rows' bf16 probabilities of every key tile (the values its P V product
// uses) and their exponent references in a workspace, and after the main pass
// rescales them with the final log-sum-exp and sums the columns: the keys are
// read once.  When keys are split, the merge launch recomputes the rows'
// scores from the merged statistics.  Either way each (sequence, head, key)
// term is added to mass_accum[b][h][key] by exactly one workgroup, in a fixed
// order: no atomics, no cross-workgroup synchronisation, deterministic
// results.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "common.h"

namespace {

using namespace dllm;

constexpr int kQT = 128;             // query rows per item
constexpr int kKT = 64;              // keys per tile
constexpr int kHD = 128;             // head dim of the bf16 kernel
constexpr int kLDK = kHD + 8;        // K tile row stride, halfwords (272 B)
constexpr int kLDV = kKT + 8;        // V^T tile row stride, halfwords (144 B)
constexpr int kMaxSeq = 1024;
constexpr int kMaxPages = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.f;      // base-2 headroom of the online-softmax reference
constexpr int kMassChunk = 16;            // key tiles per round of the score pass (256 threads x 4 keys)

struct AttnArgs {
    int n_seq, n_rows, H, n_out, max_kv, max_pages, n_cap, max_mass, pool_pages;
    int head_dim;
    float scale_log2;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* cu_q;
    const int32_t* page_table;
    const int32_t* kv_len;
    const uint32_t* mask;
    const int64_t* mask_off;
    int64_t mask_words;
    const int32_t* mass_count;
    float* mass_accum;      // [n_seq, H, n_cap], this head's term added per layer
    int mass_overwrite;     // store the term instead of adding it (first scoring layer)
    // unsplit path: the window rows' probabilities of every key tile (bf16,
    // [b*H + h][tile][max_mass][64 keys]) and each row's exponent reference
    // after that tile ([b*H + h][tile][max_mass]), for the score pass
    uint16_t* mass_p;
    float* mass_ref;
    int mass_tiles;
    uint16_t* o;
    int splits;             // key splits per (sequence, head, query tile); 1 = fused path
    uint16_t* part_o;       // split mode: [item][kQT][kHD] unnormalised outputs, bf16
    float* part_ml;         // split mode: [item][kQT][2] running max (base 2) and sum
    int qt_rows;            // split mode: query rows per first-launch item (64 or 128)
};

// split partial outputs, fragment-major: element offset of lane `lane`'s four
// values of (item, wave, row tile rt, 16-column tile dt).  They are stored in
// bf16 (the merged output is rounded to bf16 anyway): half the bytes the
// merge moves, which at batch 1 is most of the split path's cost.  Row wave*32 +
// rt*16 + lane%16, columns dt*16 + (lane/16)*4 .. +3.
__host__ __device__ __forceinline__ int64_t part_frag(int64_t item, int wave, int rt, int dt, int lane) {
    return ((((item * 4 + wave) * 2 + rt) * 8 + dt) * 64 + lane) * 4;
}

struct SeqInfo {
    int r0, rows, kv, nqt;
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b) {
    SeqInfo s;
    int r0 = a.cu_q[b], r1 = a.cu_q[b + 1];
    r0 = max(0, min(r0, a.n_rows));
    r1 = max(r0, min(r1, a.n_rows));
    s.r0 = r0;
    s.rows = r1 - r0;
    int kv = a.kv_len[b];
    kv = max(0, min(kv, min(a.max_kv, a.max_pages * 16)));
    s.kv = kv;
    s.nqt = (s.rows + kQT - 1) / kQT;
    return s;
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 lane swaps: a swap of a value with itself leaves each lane holding its
// own value in one result and its partner's in the other, so combining the
// two results reduces without selecting (and without an LDS round trip).
// A plain v_max_f32: fmaxf on values the compiler cannot prove canonical
// (a lane swap's results) first quiets each operand with an extra maximum;
// the scores are never NaN, so that step is dropped.
__device__ __forceinline__ float max_raw(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float wave_max16(float v) {
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = max_raw(__uint_as_float(t[0]), __uint_as_float(t[1]));
    t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_raw(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float wave_sum16(float v) {
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(t[0]) + __uint_as_float(t[1]);
    t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Key (within a 64-key tile) that A-row m of sub-tile t feeds to S^T.
__device__ __forceinline__ int perm_key(int t, int m) {
    return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}
// Key of S^T register e of sub-tile t held by lane group g.
__device__ __forceinline__ int reg_key(int t, int g, int e) {
    return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
}

template <int J>
struct Ic { static constexpr int value = J; };

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 LDS transpose read: inside each 16-lane group, output lane j, element e
// is element (j & 3) of the 8-byte piece addressed by lane 4e + (j >> 2).  With
// lane s pointing at row (key) kbase + (s >> 2), column d0 + 4 (s & 3) of a
// row-major [key][d] tile, lane j receives V[kbase + e][d0 + j], e = 0..3: the
// V^T operand (d = lane, four consecutive keys) without a transposed copy.
__device__ __forceinline__ s16x4 ds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// K/V (and the query tile, and mask words) reach LDS through direct-to-LDS
// copies, NS key tiles deep.  A copy writes lane i's bytes at base + size*i,
// so K and V rows (256 B: one key, one head) are stored with their 16-byte
// slots permuted by an XOR swizzle applied on the source side.  swz_k keeps
// the 16 keys a K-fragment read touches in 16 distinct bank groups; swz_v
// keeps the 8 keys x 32 bytes of a 32-lane V transpose read in 16 distinct
// bank groups.
//
// The copies are issued from inline assembly.  A copy the compiler can see
// makes it wait for every copy in flight before any LDS read it cannot prove
// disjoint, and it cannot for the transpose read; the ring's ordering is
// instead explicit: each step waits for its own stage with s_waitcnt and
// publishes it with a barrier, and the assembly's memory clobber keeps LDS
// reads from moving across a copy.
constexpr int kTileH = kKT * kHD;       // halfwords of one K (or V) tile: 16 KiB
constexpr int kDmaPerWave = 8;          // 1 KiB copies per wave per stage (16 for K, 16 for V)
constexpr int kAttnThreads = 256;       // 4 waves
constexpr int kMaskStageBytes = 2048;   // up to 256 rows x 2 mask words per stage
constexpr int kStageBytes = 2 * kTileH * 2 + kMaskStageBytes;
constexpr int kMaxSplits = 16;          // key splits per (sequence, head, query tile)
constexpr int kMassQOffset = 1024;      // after the main pass: the score pass's factors at this LDS offset
static_assert(kQT * 4 <= kMassQOffset && kMassQOffset + kMassChunk * kQT * 4 <= 2 * kStageBytes, "tail LDS layout");

__device__ __forceinline__ int swz_k(int key) { return (key + 4 * (key >> 4)) & 15; }
__device__ __forceinline__ int swz_v(int key) { return 2 * ((key & 3) + 4 * ((key >> 3) & 1)); }

// One workgroup per (sequence, head, QT-row query tile, key split); wave w
// owns query rows 16 RT w .. 16 RT w + 16 RT - 1 (RT row tiles of 16), so the
// K and V fragments a wave reads from LDS serve RT row tiles.
// s_waitcnt until at most `younger` ring stages (of PER copies each) are in
// flight: the count is only known at run time, the immediate must be a constant
// X more vector-memory operations (stores issued after the stage's copies)
// may also stay in flight
template <int NS, int PER, int X = 0>
__device__ __forceinline__ void wait_stages(int younger) {
    static_assert(NS <= 4 && 4 * PER + X < 64, "wait_stages cases");
    if (younger <= 0) __builtin_amdgcn_s_waitcnt(waitcnt_imm(X, 15));
    else if (younger == 1) __builtin_amdgcn_s_waitcnt(waitcnt_imm(PER + X, 15));
    else if (younger == 2) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * PER + X, 15));
    else if (younger == 3) __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * PER + X, 15));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * PER + X, 15));
}
// the same with `stores` (0, 3 or 6) younger stores: a smaller count than the
// stores in flight only waits longer, so larger values are clamped to 6
template <int NS, int PER>
__device__ __forceinline__ void wait_stages_st(int younger, int stores) {
    if (stores >= 6) wait_stages<NS, PER, 6>(younger);
    else if (stores >= 3) wait_stages<NS, PER, 3>(younger);
    else wait_stages<NS, PER, 0>(younger);
}

// NS: ring stages.  Two are launched (two workgroups per compute unit); four
// stages with one workgroup per unit measured slower even on small grids.
// KV8: the caches hold E4M3 codes.  Their tiles cannot use the
// direct-to-LDS copies (the MFMA needs bf16): a wave loads its pieces of the
// next tile into registers after the barrier, and before the following
// barrier decodes them and writes the bf16 values to exactly the LDS places
// the copies would fill, so every fragment read is the same as for bf16
// caches.  One tile is in flight, as with the two-stage ring.
template <int RT, int NS, bool HAS_MASK, bool KV8>
__global__ __launch_bounds__(kAttnThreads, NS == 2 ? 2 : 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int kRing = NS * kStageBytes;
    constexpr int QT = 64 * RT;
    constexpr int kMaskPerWave = HAS_MASK ? QT * 2 / 64 / 4 : 0;      // 4-byte copies per wave per stage
    constexpr int kPerStage = kDmaPerWave + kMaskPerWave;              // copies per wave per stage
    static_assert(QT * 8 <= kMaskStageBytes, "layout");
    static_assert(NS * kPerStage + 4 * RT < 64, "wait counts");
    static_assert(kRing >= (4 * kMaxSeq + 1) * 4, "the schedule scan borrows the ring");
    // one LDS allocation: the ring (which the schedule scan borrows first), then the page tables
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRing + (kMaxPages + 1) * 4 + kMaxPages / 4];
    int* s_pref = reinterpret_cast<int*>(lds);                                    // [kMaxSeq + 1], scheduling only
    int* s_seq = s_pref + (kMaxSeq + 1);                                          // [kMaxSeq][3], scheduling only
    int* s_pages = reinterpret_cast<int*>(lds + kRing);                      // [kMaxPages]
    int* s_total = s_pages + kMaxPages;
    // per key tile: bit q (q < 4) = page 4t + q exists and is valid, bit 4 = every key valid
    uint8_t* s_tile_full = reinterpret_cast<uint8_t*>(s_total + 1);               // [kMaxPages / 4]
    auto k_tile = [&](int sl) { return reinterpret_cast<uint16_t*>(lds + sl * kStageBytes); };
    auto v_tile = [&](int sl) { return reinterpret_cast<uint16_t*>(lds + sl * kStageBytes) + kTileH; };
    auto m_words = [&](int sl) { return reinterpret_cast<uint32_t*>(lds + sl * kStageBytes + 4 * kTileH); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, ln = lane & 15;

    // A single sequence's page-table row does not depend on the schedule: it is
    // fetched together with the schedule's loads (one round trip fewer).
    constexpr int kPrePages = kMaxPages / kAttnThreads;
    static_assert(kPrePages * kAttnThreads == kMaxPages, "every page entry has a thread");
    const bool one_seq = a.n_seq == 1;
    int pre_pages[kPrePages];
    if (one_seq) {
#pragma unroll
        for (int i = 0; i < kPrePages; ++i) {
            const int j = tid + i * kAttnThreads;
            pre_pages[i] = j < a.max_pages ? a.page_table[j] : -1;
        }
    }

    // ---- schedule: per-sequence item counts (query tiles x heads x splits), prefix-summed by wave 0 ----
    if (wave == 0) {
        int base = 0;
        for (int c = 0; c < a.n_seq; c += 64) {
            int b = c + lane;
            int items = 0;
            if (b < a.n_seq) {
                SeqInfo s = seq_info(a, b);
                items = (s.rows + QT - 1) / QT * a.H * a.splits;
                s_seq[3 * b] = s.r0;
                s_seq[3 * b + 1] = s.rows;
                s_seq[3 * b + 2] = s.kv;
            }
            int scan = items;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int t = __shfl_up(scan, off);
                if (lane >= off) scan += t;
            }
            if (b < a.n_seq) s_pref[b + 1] = base + scan;
            base += __shfl(scan, 63);
        }
        if (lane == 0) {
            s_pref[0] = 0;
            *s_total = base;
        }
    }
    __syncthreads();
    // a malformed cu_q (not non-decreasing) can claim more items than were
    // launched: then nothing runs (outputs unspecified, nothing out of bounds)
    const int total = *s_total;
    if (total > (int)gridDim.x || (int)blockIdx.x >= total) return;
    const int item = xcd_remap(blockIdx.x, total);
    int lo = 0, hi = a.n_seq - 1;                       // last b with s_pref[b] <= item
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    SeqInfo si;                                          // from the scan: no second round trip
    si.r0 = s_seq[3 * b];
    si.rows = s_seq[3 * b + 1];
    si.kv = s_seq[3 * b + 2];
    si.nqt = (si.rows + kQT - 1) / kQT;
    const int nqt = (si.rows + QT - 1) / QT;
    const int local = item - s_pref[b];
    const int seq_first = s_pref[b];                    // the ring overwrites s_pref below
    const int qt = local % nqt;                         // consecutive items: next query tile, same head
    const int hs = local / nqt;
    const int sp = hs % a.splits;                       // key split
    const int h = hs / a.splits;
    const int seq_r0 = si.r0;
    const int r0 = seq_r0 + qt * QT;
    const int nr = min(QT, si.rows - qt * QT);
    const int ntiles = (si.kv + kKT - 1) / kKT;
    const int tiles_per = (ntiles + a.splits - 1) / a.splits;
    const int t_begin = min(sp * tiles_per, ntiles);    // this item's key tiles
    const int t_end = min(t_begin + tiles_per, ntiles);
    const int npages = (si.kv + 15) / 16;
    if (one_seq) {
#pragma unroll
        for (int i = 0; i < kPrePages; ++i) {
            const int j = tid + i * kAttnThreads, p = pre_pages[i];
            if (j < npages) s_pages[j] = (p >= 0 && p < a.pool_pages) ? p : -1;
        }
    } else {
        for (int j = tid; j < npages; j += kAttnThreads) {
            int p = a.page_table[(int64_t)b * a.max_pages + j];
            s_pages[j] = (p >= 0 && p < a.pool_pages) ? p : -1;
        }
    }
    __syncthreads();
    for (int t = tid; t < kMaxPages / 4; t += kAttnThreads) {
        uint32_t pg = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) pg |= (t * 4 + q < npages && s_pages[t * 4 + q] >= 0 ? 1u : 0u) << q;
        const bool full = t < ntiles && (t + 1) * kKT <= si.kv && pg == 15u;
        s_tile_full[t] = (uint8_t)(pg | (full ? 16u : 0u));
    }
    __syncthreads();

    const int last_page = max(npages - 1, 0);
    // Items whose key tiles are all full (every key valid, no mask) and number
    // at most 64 take their copy bases from registers: lane 2j + e of vpg<k>
    // holds page 4(t_begin + 32k + j) + 2(wave & 1) + e, the page of half e of
    // this wave's keys in the item's tile 32k + j, read once here; then no
    // step of the main pass waits on an LDS read of a page entry or a tile
    // flag (those round trips cost 6% of a full-refresh launch).
    // (two named registers, not an array: a select between array elements
    // became an indexed scratch array that the compiler placed in LDS)
    bool fast = !HAS_MASK && !KV8 && t_end - t_begin <= 64;
    auto page_lane = [&](int k) __attribute__((always_inline)) {
        const int t = t_begin + 32 * k + (lane >> 1);
        fast &= __builtin_amdgcn_ballot_w64(t < t_end && !(s_tile_full[min(t, kMaxPages / 4 - 1)] & 16)) == 0;
        return s_pages[min(4 * t + 2 * (wave & 1) + (lane & 1), kMaxPages - 1)];
    };
    const int vpg0 = page_lane(0), vpg1 = page_lane(1);
    // keys past kv_len or on a bad page read the sequence's key 0 (a row the
    // item reads anyway); the visibility bits zero them
    const int key0_page = npages > 0 ? s_pages[0] : -1;
    const int64_t safe_row = key0_page >= 0 ? (int64_t)key0_page * 16 : 0;
    const int64_t mwords = (si.kv + 31) / 32;
    const int64_t mask_row0 = HAS_MASK ? a.mask_off[b] + (int64_t)(qt * QT) * mwords : 0;
    // window rows of formula (2) (query tile 0 only); loaded before any copy is issued
    const bool want_mass = qt == 0 && a.mass_accum != nullptr && a.mass_count != nullptr;
    const int mb_in = want_mass ? a.mass_count[b] : 0;
    // unsplit: window rows whose probabilities the main pass keeps
    const int mbp = a.splits == 1 ? max(0, min(mb_in, min(a.max_mass, min(si.rows, QT)))) : 0;
    // this (sequence, head)'s probability rows and references (wave-uniform bases)
    const int64_t mass_item0 = (int64_t)(b * a.H + h) * a.mass_tiles * a.max_mass;
    uint16_t* const mp_item = mbp > 0 ? a.mass_p + mass_item0 * kKT : nullptr;
    float* const mr_item = mbp > 0 ? a.mass_ref + mass_item0 : nullptr;

    // ---- copies: K groups (waves 0, 1) or V groups (waves 2, 3) of 4 keys; mask words; query tile ----
    const bool is_v = wave >= 2;
    const uint16_t* kv_src = (is_v ? a.v : a.k) + h * kHD;
    const uint8_t* kv_src8 = reinterpret_cast<const uint8_t*>(is_v ? a.v : a.k) + h * kHD;
    // KV8: this wave's codes of the tile in flight.  Ordinary loads, which the
    // compiler tracks: it waits before any use or register copy of them (with
    // a load it cannot see, the register allocator once copied a code pair
    // ahead of the wait and staged stale codes).
    u32x2 kv8[KV8 ? kDmaPerWave : 1];
    int lslot[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int kk = 4 * ((wave & 1) * kDmaPerWave + i) + (lane >> 4);
        lslot[i] = (lane & 15) ^ (is_v ? swz_v(kk) : swz_k(kk));
    }
    // A sequence whose rows fit one query tile reads each key once (per head
    // and split): its K and V lines are fetched non-temporally, which leaves the
    // caches to the lines that are read again (the window rows' probabilities,
    // other sequences' tiles).  Full refreshes read every key once per query
    // tile and keep the default policy, so the tiles after the first hit in L2.
    // (The choice is made once per issued tile: a branch per copy measured 3%
    // slower on full refreshes.)  Split launches (few sequences, latency-bound)
    // keep the default policy: measured 0.4 us faster at batch 1.
    const bool kv_once = si.nqt == 1 && a.splits == 1;
    auto issue_p = [&](auto NTC, auto FULLC, int sl, int t) __attribute__((always_inline)) {
        constexpr bool kNt = decltype(NTC)::value != 0;
        constexpr bool kFullPath = decltype(FULLC)::value != 0;
        auto copy_kv = [&](const uint16_t* src, uint32_t dst) __attribute__((always_inline)) {
            if constexpr (kNt) copy16_to_lds_nt(src, dst);
            else copy16_to_lds(src, dst);
        };
        auto load_kv8 = [&](const uint8_t* src) __attribute__((always_inline)) -> u32x2 {
            if constexpr (kNt) return __builtin_nontemporal_load((const u32x2*)src);
            else return *(const u32x2*)src;
        };
        const uint32_t dst = lds_addr(is_v ? v_tile(sl) : k_tile(sl));
        // (the masked and E4M3 kernels keep only the general path: their
        // register budget has no room for both)
        if (kFullPath && !HAS_MASK && !KV8 && t < t_end &&
            (fast || (__builtin_amdgcn_readfirstlane(s_tile_full[t]) & 16))) {
            // every key valid: a wave's copies touch two pages (wave-uniform), so
            // a copy's source is a page base plus a fixed 32-bit lane offset
            int p0, p1;
            if (fast) {
                const int j = t - t_begin, l0 = 2 * (j & 31);
                const int a0 = __builtin_amdgcn_readlane(vpg0, l0), a1 = __builtin_amdgcn_readlane(vpg0, l0 + 1);
                const int c0 = __builtin_amdgcn_readlane(vpg1, l0), c1 = __builtin_amdgcn_readlane(vpg1, l0 + 1);
                p0 = (j & 32) ? c0 : a0;
                p1 = (j & 32) ? c1 : a1;
            } else {
                p0 = __builtin_amdgcn_readfirstlane(s_pages[t * 4 + 2 * (wave & 1)]);
                p1 = __builtin_amdgcn_readfirstlane(s_pages[t * 4 + 2 * (wave & 1) + 1]);
            }
            const int64_t b0 = (int64_t)p0 * 16 * a.n_out, b1 = (int64_t)p1 * 16 * a.n_out;
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) {
                const int q = (wave & 1) * kDmaPerWave + i;        // 4-key group of the tile
                const uint32_t off = (uint32_t)((4 * (q & 3) + (lane >> 4)) * a.n_out + lslot[i] * 8);
                const int64_t base = i < kDmaPerWave / 2 ? b0 : b1;
                if constexpr (KV8)
                    kv8[i] = load_kv8(kv_src8 + base + off);
                else
                    copy_kv(kv_src + base + off, __builtin_amdgcn_readfirstlane(dst + q * 1024));
            }
        } else {
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) {
                const int q = (wave & 1) * kDmaPerWave + i;        // 4-key group of the tile
                const int kg = t * kKT + 4 * q + (lane >> 4);
                const int page = s_pages[min(kg >> 4, last_page)];
                const bool ok = (t < t_end) & (kg < si.kv) & (page >= 0);
                const int64_t row = ok ? (int64_t)page * 16 + (kg & 15) : safe_row;
                if constexpr (KV8)
                    kv8[i] = load_kv8(kv_src8 + row * a.n_out + lslot[i] * 8);
                else
                    copy_kv(kv_src + row * a.n_out + lslot[i] * 8, __builtin_amdgcn_readfirstlane(dst + q * 1024));
            }
        }
        if constexpr (HAS_MASK) {
            // words 2t, 2t+1 of every query row of the tile: [row][2]
            const uint32_t mdst = lds_addr(m_words(sl));
#pragma unroll
            for (int i = 0; i < kMaskPerWave; ++i) {
                const int m = wave * kMaskPerWave + i;
                const int idx = m * 64 + lane;
                const int row = min(idx >> 1, max(nr - 1, 0));
                int64_t wi = mask_row0 + (int64_t)row * mwords + 2 * (int64_t)t + (idx & 1);
                wi = min(max(wi, (int64_t)0), a.mask_words - 1);
                copy4_to_lds(a.mask + wi, __builtin_amdgcn_readfirstlane(mdst + m * 256));
            }
        }
    };
    auto issue = [&](int sl, int t) __attribute__((always_inline)) {
        if (kv_once) issue_p(Ic<1>{}, Ic<1>{}, sl, t);
        else issue_p(Ic<0>{}, Ic<1>{}, sl, t);
    };
    // the ring's first fill: one straight-line form (the general path, cached
    // copies) so that every path through it issues the same copies, which the
    // query fragments' wait counts; the streaming hint is lost on these NS tiles
    auto issue_first = [&](int sl, int t) __attribute__((always_inline)) {
        issue_p(Ic<0>{}, Ic<0>{}, sl, t);
    };

    // KV8: decode the codes loaded by issue() (their wait is the caller's) into
    // the bf16 places of stage sl
    auto commit8 = [&](int sl) __attribute__((always_inline)) {
        if constexpr (KV8) {
            uint8_t* dst = reinterpret_cast<uint8_t*>(is_v ? v_tile(sl) : k_tile(sl));
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) {
                const int q = (wave & 1) * kDmaPerWave + i;
                *(bf16x8*)(dst + q * 1024 + 16 * lane) = e4m3x8_to_bf16(kv8[i][0], kv8[i][1]);
            }
        }
    };

    // ---- query fragments (B operand of S^T = K Q^T), rows of this wave, straight
    // into registers; then every ring stage is issued at once (the fragments
    // are older than every copy, so one explicit wait covers them) ----
    const int wrow = wave * 16 * RT;
    bool rt_active[RT], row_ok[RT];
    u32x4 qraw[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = wrow + rt * 16 + ln;
        rt_active[rt] = wrow + rt * 16 < nr;
        row_ok[rt] = row < nr;
        const int qrow = r0 + min(row, max(nr - 1, 0));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qraw[rt][ks] = load_untracked_x4(a.q + (int64_t)qrow * a.n_out + h * kHD + ks * 32 + g * 8);
    }
    const int n_main = t_end - t_begin;
    if constexpr (KV8) {
        // tile 0 always (an item without tiles loads rows it would read, and
        // never reads the stage back), so the wait is unconditional
        issue_first(0, t_begin);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));   // the query fragments and tile 0's codes
        commit8(0);
    } else {
        // the whole ring, always (a stage past the item's last tile copies rows
        // it reads anyway and is never read back), so one constant wait covers
        // the query fragments: they are older than every copy
#pragma unroll
        for (int s = 0; s < NS; ++s) issue_first(s, t_begin + s);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(NS * kPerStage, 15));
    }
    bf16x8 qf[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[rt][ks] = __builtin_bit_cast(bf16x8, fence_value(qraw[rt][ks]));
    __builtin_amdgcn_sched_barrier(0);

    // ---- per-tile math ----
    // visibility of this lane's 16 scores in tile t (row validity and mask applied)
    auto vis_bits = [&](int t, bool rok, uint32_t w0, uint32_t w1) __attribute__((always_inline)) -> uint32_t {
        uint32_t bits = 0;
        const int kbase = t * kKT;
        const uint32_t pg = s_tile_full[t];                  // the tile's valid pages, one read
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kk = reg_key(t4, g, e);
                const int kg = kbase + kk;
                const uint32_t w = (kk < 32) ? w0 : w1;
                const bool ok = (kg < si.kv) & (((pg >> (kk >> 4)) & 1u) != 0) &
                                (((w >> (kk & 31)) & 1u) != 0);
                bits |= (ok ? 1u : 0u) << (t4 * 4 + e);
            }
        return rok ? bits : 0u;
    };
    // mask words of query row `row` (tile-relative) for tile t, from the stage's copy
    auto mask_pair = [&](int sl, int row, int t, uint32_t& w0, uint32_t& w1) __attribute__((always_inline)) {
        if constexpr (!HAS_MASK) {
            w0 = w1 = 0xffffffffu;
        } else {
            const uint32_t* mw = m_words(sl);
            const int64_t i0 = mask_row0 + (int64_t)min(row, max(nr - 1, 0)) * mwords + 2 * (int64_t)t;
            w0 = (i0 >= 0 && i0 < a.mask_words) ? mw[2 * row] : 0u;
            w1 = (i0 + 1 >= 0 && i0 + 1 < a.mask_words) ? mw[2 * row + 1] : 0u;
        }
    };

    // Row sums of the probabilities come from the matrix cores: a tile of
    // ones in place of V^T gives, in every element of a lane's accumulator,
    // the sum over the tile's keys of that lane's query row (of the bf16
    // probabilities the P.V product uses, so numerator and denominator see
    // the same values); two more MFMAs per row tile replace 16 adds per lane.
    // The masked kernel keeps the adds (its visibility code needs the
    // registers): each lane sums its own keys, the lane groups meet at the end.
    constexpr bool kMfmaSum = !HAS_MASK;
    float m_run[RT], l_run[RT];
    f32x4 acc[RT][8], acc_l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_run[rt] = kNegBig;
        acc_l[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    // Every row tile of the wave is computed, also one past the item's last
    // row (its rows repeat the last query row and are never stored): the loop
    // is straight-line code with no per-row-tile tests, which the compiler
    // schedules far better; the extra tiles occur only in an item's last
    // query tile and run on other SIMDs in parallel.  The masked kernels keep
    // the tests (their visibility code needs the registers).
    constexpr bool kSkipIdle = HAS_MASK;
    // S^T for the active row tiles (K fragments shared across them)
    auto scores = [&](const uint16_t* kt_lds, f32x4 (&st)[RT][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int key = perm_key(t4, ln);
            bf16x8 kf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kf[ks] = *(const bf16x8*)(kt_lds + key * kHD + (((ks * 4 + g) ^ swz_k(key)) * 8));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                st[rt][t4] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kSkipIdle && !rt_active[rt]) continue;   // uniform per wave
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    st[rt][t4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[rt][ks], st[rt][t4], 0, 0, 0);
            }
        }
    };

    auto attend = [&](int sl, int t) __attribute__((always_inline)) {
        f32x4 st[RT][4];
        scores(k_tile(sl), st);
        bool full = !HAS_MASK;
        if (!HAS_MASK && !fast) full = (s_tile_full[t] & 16) != 0;
        // raw scores; the scale is folded into the exponent (c > 0 keeps the order).
        // Keys a row may not see get -inf: one branch for every row tile, with
        // a side effect the compiler may not speculate, so that a full tile
        // runs none of it (flattened into selects, or with its key indices
        // hoisted above the branch, it cost every full tile up to ~100 vector
        // instructions)
        if (!full) {
            asm volatile("");
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (kSkipIdle && !rt_active[rt]) continue;
                uint32_t w0, w1;
                mask_pair(sl, wrow + rt * 16 + ln, t, w0, w1);
                const uint32_t vis = vis_bits(t, row_ok[rt], w0, w1);
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        st[rt][t4][e] = ((vis >> (t4 * 4 + e)) & 1u) ? st[rt][t4][e] : -INFINITY;
            }
        }
        bf16x8 pf[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (kSkipIdle && !rt_active[rt]) continue;
            float mx = -INFINITY;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[rt][t4][e]);
            mx = wave_max16(mx);
            // The exponent reference moves only when the row maximum passes it by
            // more than kRescaleSlack (base 2): probabilities relative to it stay
            // below 2^kRescaleSlack, sums and outputs use the same reference, and
            // the rescale of the accumulators (most of this step's ALU work
            // while maxima still grow) is mostly skipped.
            const float mt = mx * a.scale_log2;
            const bool grow = mt > m_run[rt] + kRescaleSlack;
            const float m_new = grow ? mt : m_run[rt];
            float rs = 0.f;                               // the masked kernel's per-lane row sum
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(st[rt][t4][e], a.scale_log2, -m_new));
                    st[rt][t4][e] = p;
                    if constexpr (!kMfmaSum) rs += p;
                }
            if (grow) {                                   // the reference moved: rescale that row
                const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
                if constexpr (kMfmaSum) acc_l[rt] *= alpha;
                else acc_l[rt][0] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[rt][dt] *= alpha;
            }
            if constexpr (!kMfmaSum) acc_l[rt][0] += rs;  // after the rescale: p is relative to m_new
            m_run[rt] = m_new;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 u;
                u[0] = pack_bf16x2(st[rt][2 * c][0], st[rt][2 * c][1]);
                u[1] = pack_bf16x2(st[rt][2 * c][2], st[rt][2 * c][3]);
                u[2] = pack_bf16x2(st[rt][2 * c + 1][0], st[rt][2 * c + 1][1]);
                u[3] = pack_bf16x2(st[rt][2 * c + 1][2], st[rt][2 * c + 1][3]);
                pf[rt][c] = __builtin_bit_cast(bf16x8, u);
            }
            // the window rows keep this tile's probabilities for the score pass
            if (wrow + rt * 16 < mbp) {                   // uniform per wave
                const int my_row = wrow + rt * 16 + ln;
                if (my_row < mbp) {
                    const uint32_t pt = (uint32_t)(t * a.max_mass + my_row);   // < 2^15 rows per item
                    uint16_t* prow = mp_item + (pt * kKT + 8 * g);
                    *(bf16x8*)prow = pf[rt][0];
                    *(bf16x8*)(prow + 32) = pf[rt][1];
                    if (g == 0) mr_item[pt] = m_run[rt];
                }
            }
        }
        // O^T += V^T P^T.  V^T fragments: source lane ln of group g points at key
        // c*32 + 8g + 4*hf + (ln >> 2), column dt*16 + 4*(ln & 3)
        const uint16_t* vt_lds = v_tile(sl);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 vf[8];
            {
                // keys c*32 + 8g + (ln >> 2) (lo) and 4 further (hi); one 8-element
                // initializer per fragment (element-wise insertion is mis-lowered)
                const int key = c * 32 + 8 * g + (ln >> 2);
                const uint16_t* vlo = vt_lds + key * kHD + 4 * (ln & 1);
                const uint16_t* vhi = vlo + 4 * kHD;
                const int sw = swz_v(key);               // equal for key and key + 4
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const int lsl = 2 * dt + ((ln & 3) >> 1);
                    const s16x4 lo4 = ds_read_tr(vlo + ((lsl ^ sw) * 8));
                    const s16x4 hi4 = ds_read_tr(vhi + ((lsl ^ sw) * 8));
                    typedef short s16x8 __attribute__((ext_vector_type(8)));
                    const s16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    vf[dt] = __builtin_bit_cast(bf16x8, v8);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (kSkipIdle && !rt_active[rt]) continue;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[rt][c], acc[rt][dt], 0, 0, 0);
                if constexpr (kMfmaSum)
                    acc_l[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[rt][c], acc_l[rt], 0, 0, 0);
            }
        }
    };

    // ---- main pass: this item's key tiles through the ring ----
    // The prologue filled the ring; from the second step on, each step refills
    // the slot the previous step read, and nothing past t_end is ever fetched.
    // A step waits until its own tile has landed (the stages issued after it
    // may stay in flight), then an LDS-only barrier publishes it
    // (__syncthreads would also wait for the younger stages).
    // Vector-memory stores share the counter with the copies and complete in
    // issue order: a wave that keeps window rows' probabilities issues
    // st_attend stores per step (two 16-byte stores and a reference per row
    // tile of window rows), and every wait for a tile lets the stores issued
    // after that tile's copies stay in flight rather than waiting for them.
    int st_attend = 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) st_attend += (wrow + rt * 16 < mbp) ? 3 : 0;
    if constexpr (KV8) {
        // tile i's codes were loaded in step i - 1; its stage was last read in step i - 2
        for (int i = 0; i < n_main; ++i) {
            if (i > 0) {
                wait_stages_st<NS, 0>(0, st_attend);         // after the loads: step i - 1's stores
                commit8(i % NS);
            }
            lds_sync();
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < n_main) issue((i + 1) % NS, t_begin + i + 1);
            __builtin_amdgcn_sched_barrier(0);
            attend(i % NS, t_begin + i);
        }
    } else {
        for (int i = 0; i < n_main; ++i) {
            // stages issued before this step: the prologue's NS, then one per step
            const int issued = NS + max(0, min(n_main - NS, i - 1));
            // ... younger than tile i, and the stores of the steps since its copies
            wait_stages_st<NS, kPerStage>(issued - 1 - i, st_attend * min(i, NS - 1));
            lds_sync();
            __builtin_amdgcn_sched_barrier(0);
            if (i > 0 && i - 1 + NS < n_main) issue((i - 1) % NS, t_begin + i - 1 + NS);
            __builtin_amdgcn_sched_barrier(0);
            attend(i % NS, t_begin + i);
        }
    }
    __syncthreads();                                    // every copy has been waited for above
    // the MFMA row sums already cover every key of the row (all four lane
    // groups); the per-lane sums of the masked kernel meet here
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l_run[rt] = kMfmaSum ? acc_l[rt][0] : wave_sum16(acc_l[rt][0]);

    // LDS after the main pass (the ring is free): final log-sum-exp (base 2) of
    // the tile's rows, then the score pass's factors
    float* s_lse = reinterpret_cast<float*>(lds);                        // [kQT]

    if (a.splits > 1) {
        // ---- split mode: publish the unnormalised partial; attn_finish_kernel
        // merges the splits and forms the column mass ----
        // fragment-major: [item][wave][rt][dt][lane][4], so every store
        // instruction writes 512 B of whole lines (row-major stores would
        // scatter 32-byte pieces over 16 rows)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (!rt_active[rt]) continue;
            const int my_row = wrow + rt * 16 + ln;
            uint16_t* po = a.part_o + part_frag(item, wave, rt, 0, lane);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint2 u;
                u.x = pack_bf16x2(acc[rt][dt][0], acc[rt][dt][1]);
                u.y = pack_bf16x2(acc[rt][dt][2], acc[rt][dt][3]);
                *(uint2*)(po + dt * 256) = u;
            }
            if (g == 0) {
                a.part_ml[((int64_t)item * kQT + my_row) * 2] = m_run[rt];
                a.part_ml[((int64_t)item * kQT + my_row) * 2 + 1] = l_run[rt];
            }
        }
        return;
    } else {
        // ---- output ----
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (!row_ok[rt]) continue;
            const int my_row = wrow + rt * 16 + ln;
            const float inv = l_run[rt] > 0.f ? 1.f / l_run[rt] : 0.f;
            uint16_t* orow = a.o + (int64_t)(r0 + my_row) * a.n_out + h * kHD + g * 4;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint2 u;
                u.x = pack_bf16x2(acc[rt][dt][0] * inv, acc[rt][dt][1] * inv);
                u.y = pack_bf16x2(acc[rt][dt][2] * inv, acc[rt][dt][3] * inv);
                *(uint2*)(orow + dt * 16) = u;
            }
            if (g == 0 && my_row < kQT)
                s_lse[my_row] = l_run[rt] > 0.f ? m_run[rt] + __log2f(l_run[rt]) : INFINITY;
        }
    }

    // ---- formula (2): this head's column mass over every key of the sequence ----
    // The main pass kept the window rows' probabilities of every key tile
    // relative to the row's exponent reference at that tile; with the final
    // log-sum-exp each is rescaled by exp2(reference - lse).  Each thread owns
    // four consecutive keys of a tile and sums over the window rows in a fixed
    // order; each key's term is added to mass_accum once, by this workgroup
    // only.  No K re-read and no score recompute.
    if (!want_mass) return;
    const int mb = mbp;
    if (mb == 0 || si.kv == 0) return;
    __syncthreads();                                         // every wave's probabilities and s_lse
    const float norm = 1.f / ((float)a.H * (float)mb);
    float* macc = a.mass_accum + ((int64_t)b * a.H + h) * a.n_cap;
    const int kmax = min(si.kv, a.n_cap);
    const int ntiles_m = (kmax + kKT - 1) / kKT;
    float* s_fac = reinterpret_cast<float*>(lds + kMassQOffset);   // [kMassChunk][mb]
    for (int t0 = 0; t0 < ntiles_m; t0 += kMassChunk) {
        for (int j = tid; j < kMassChunk * mb; j += kAttnThreads) {
            const int tc = j / mb, i = j % mb;
            const int t = t0 + tc;
            s_fac[j] = t < ntiles_m ? exp2f(mr_item[t * a.max_mass + i] - s_lse[i]) : 0.f;
        }
        __syncthreads();
        const int tc = tid / (kKT / 4), kq = tid % (kKT / 4);
        const int t = t0 + tc;
        if (t < ntiles_m) {
            const uint16_t* pcol = mp_item + ((uint32_t)(t * a.max_mass) * kKT + 4 * kq);
            float cs[4] = {0.f, 0.f, 0.f, 0.f};
            for (int i0 = 0; i0 < mb; i0 += 8) {
                uint2 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    w[u] = i0 + u < mb ? *(const uint2*)(pcol + (i0 + u) * kKT) : make_uint2(0u, 0u);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (i0 + u >= mb) continue;
                    const float f = s_fac[tc * mb + i0 + u];
                    cs[0] += bf16_bits_to_f32(w[u].x & 0xffffu) * f;
                    cs[1] += bf16_bits_to_f32(w[u].x >> 16) * f;
                    cs[2] += bf16_bits_to_f32(w[u].y & 0xffffu) * f;
                    cs[3] += bf16_bits_to_f32(w[u].y >> 16) * f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kk = t * kKT + 4 * kq + e;
                if (kk < kmax) macc[kk] = (a.mass_overwrite ? 0.f : macc[kk]) + cs[e] * norm;
            }
        }
        __syncthreads();
    }
}

// Split mode, second launch.  Items per sequence b: H * ceil(rows_b / 16)
// merge items (b, h, 16-row chunk) and, when formula (2) is requested,
// H * ntiles mass items (b, h, key tile).  A merge item combines the key
// splits of its rows in split order (fixed, so the result is deterministic)
// and writes o: one thread per (row, 8 columns), every split's partials in
// flight together.  A mass item rebuilds the masked-window rows' final
// log-sum-exp from the split partials, recomputes those rows' scores against
// its 64 keys (S^T = K Q^T on MFMA) and adds the column sums to
// mass_accum[b][h][its keys], which no other item touches: no atomics and no
// cross-workgroup synchronisation.  Every load that does not depend on
// another is issued before the first wait.
constexpr int kFinThreads = 256;
constexpr int kMergeRows = kFinThreads / (kHD / 8);      // 16 rows per merge item

// MAXS: a power of two >= the split count.  Every loop over splits runs to
// MAXS with clamped indices (loads in flight together; a loop to the runtime
// count with a running maximum or sum would serialise them) and the values
// past the split count are ignored.  MAXRT: 16-row tiles of window rows a mass
// item holds query fragments for (max_mass <= 16 MAXRT): the fragments of
// every tile are loaded before the first wait, so MAXRT sets the registers,
// and with them how many workgroups share a compute unit (2 at 8 tiles, 4 at 2).
template <int MAXS, bool KV8, int MAXRT>
__global__ __launch_bounds__(kFinThreads) void attn_finish_kernel(AttnArgs a) {
    __shared__ int s_pref[kMaxSeq + 1];
    __shared__ int s_total;
    __shared__ float s_lse[kQT];
    __shared__ float s_csum[4][kKT];
    __shared__ int s_seq[kMaxSeq * 3];          // (r0, rows, kv) per sequence, from the scan
    __shared__ int s_first[kMaxSeq + 1];        // first-launch items before each sequence
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, ln = lane & 15;
    const bool want_mass = a.mass_accum != nullptr && a.mass_count != nullptr;
    if (wave == 0) {
        int base = 0, base1 = 0;
        for (int c = 0; c < a.n_seq; c += 64) {
            int b = c + lane;
            int items = 0, first = 0;
            if (b < a.n_seq) {
                SeqInfo s = seq_info(a, b);
                items = a.H * ((s.rows + kMergeRows - 1) / kMergeRows + (want_mass ? (s.kv + kKT - 1) / kKT : 0));
                first = (s.rows + a.qt_rows - 1) / a.qt_rows * a.H * a.splits;
                s_seq[3 * b] = s.r0;
                s_seq[3 * b + 1] = s.rows;
                s_seq[3 * b + 2] = s.kv;
            }
            int scan = items, scan1 = first;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int t = __shfl_up(scan, off), t1 = __shfl_up(scan1, off);
                if (lane >= off) {
                    scan += t;
                    scan1 += t1;
                }
            }
            if (b < a.n_seq) {
                s_pref[b + 1] = base + scan;
                s_first[b + 1] = base1 + scan1;
            }
            base += __shfl(scan, 63);
            base1 += __shfl(scan1, 63);
        }
        if (lane == 0) {
            s_pref[0] = 0;
            s_first[0] = 0;
            s_total = base;
        }
    }
    __syncthreads();
    const int total = s_total;
    if (total > (int)gridDim.x || (int)blockIdx.x >= total) return;
    const int item = xcd_remap(blockIdx.x, total);
    int lo = 0, hi = a.n_seq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    SeqInfo si;                                          // from the scan: no second round trip
    si.r0 = s_seq[3 * b];
    si.rows = s_seq[3 * b + 1];
    si.kv = s_seq[3 * b + 2];
    si.nqt = (si.rows + kQT - 1) / kQT;
    const int local = item - s_pref[b];
    const int seq_r0 = si.r0;
    const int nch = (si.rows + kMergeRows - 1) / kMergeRows;
    // split-mode item index of (b, h, split, qt) in the first launch
    const int first_items = s_first[b];
    const int nqt1 = (si.rows + a.qt_rows - 1) / a.qt_rows;   // first-launch query tiles
    auto split_item = [&](int h, int spl, int qt) { return first_items + (h * a.splits + spl) * nqt1 + qt; };
    const int rt_per_wave = a.qt_rows / 64;                      // row tiles a first-launch wave held

    if (local < a.H * nch) {
        // ---- merge item: rows ch*16 .. ch*16+15 of head h, thread = (row, 8 columns) ----
        const int ch = local % nch, h = local / nch;
        const int row = ch * kMergeRows + (tid >> 4), c8 = tid & 15;
        if (row >= si.rows) return;
        const int qt = row / a.qt_rows, r = row % a.qt_rows;
        float ms[MAXS], ls[MAXS];
        uint2 pw[MAXS][2];
#pragma unroll
        for (int spl = 0; spl < MAXS; ++spl) {
            const int64_t it = split_item(h, min(spl, a.splits - 1), qt);
            ms[spl] = a.part_ml[(it * kQT + r) * 2];
            ls[spl] = a.part_ml[(it * kQT + r) * 2 + 1];
            // columns c8*8 .. +7: tile dt = c8/2, lane groups 2 (c8 % 2) and +1
            const int w = r / (16 * rt_per_wave), rt = (r >> 4) % rt_per_wave, lr = r & 15, g0 = 2 * (c8 & 1);
            pw[spl][0] = *(const uint2*)(a.part_o + part_frag(it, w, rt, c8 >> 1, g0 * 16 + lr));
            pw[spl][1] = *(const uint2*)(a.part_o + part_frag(it, w, rt, c8 >> 1, (g0 + 1) * 16 + lr));
        }
        float m = -INFINITY;
#pragma unroll
        for (int spl = 0; spl < MAXS; ++spl)
            if (spl < a.splits) m = fmaxf(m, ms[spl]);
        float l = 0.f, o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int spl = 0; spl < MAXS; ++spl) {
            if (spl >= a.splits) continue;
            const float f = exp2f(ms[spl] - m);
            l += ls[spl] * f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                o8[4 * hf + 0] += bf16_bits_to_f32(pw[spl][hf].x & 0xffffu) * f;
                o8[4 * hf + 1] += bf16_bits_to_f32(pw[spl][hf].x >> 16) * f;
                o8[4 * hf + 2] += bf16_bits_to_f32(pw[spl][hf].y & 0xffffu) * f;
                o8[4 * hf + 3] += bf16_bits_to_f32(pw[spl][hf].y >> 16) * f;
            }
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(o8[2 * e] * inv, o8[2 * e + 1] * inv);
        *(u32x4*)(a.o + (int64_t)(seq_r0 + row) * a.n_out + h * kHD + c8 * 8) = u;
        return;
    }

    // ---- mass item: (h, key tile kt) of sequence b ----
    const int ml = local - a.H * nch;
    const int ntiles = (si.kv + kKT - 1) / kKT;
    const int kt = ml % ntiles, h = ml / ntiles;
    // wave w: keys kt*64 + 16w .. +15 (A operand, natural order) x window row tiles.
    // The wave's 16 keys share one page (16-key pages, 16-aligned), so one
    // page-table entry gives every key's validity; they also share one 32-bit
    // mask word per row.
    const int kw0 = kt * kKT + wave * 16;
    const int page = a.page_table[(int64_t)b * a.max_pages + (min(kw0, si.kv - 1) >> 4)];
    int mb = a.mass_count[b];
    // window rows' split statistics, queries and mask words, and the running
    // scores of this item's keys: all independent of the page entry above
    const int r_ml = min(tid, kQT - 1);
    float ms[MAXS], ls[MAXS];
#pragma unroll
    for (int spl = 0; spl < MAXS; ++spl) {
        const int64_t it = split_item(h, min(spl, a.splits - 1), 0);
        ms[spl] = a.part_ml[(it * kQT + r_ml) * 2];
        ls[spl] = a.part_ml[(it * kQT + r_ml) * 2 + 1];
    }
    const int mb_rows = max(1, min(si.rows, min(a.max_mass, 16 * MAXRT)));   // mb <= this (clamped below)
    bf16x8 qfr[MAXRT][4];
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt) {
        if (rt * 16 >= mb_rows) continue;                    // uniform: only the window's row tiles
        const int qrow = seq_r0 + min(rt * 16 + ln, mb_rows - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qfr[rt][ks] = *(const bf16x8*)(a.q + (int64_t)qrow * a.n_out + h * kHD + ks * 32 + g * 8);
    }
    const bool has_mask = a.mask != nullptr;
    const int64_t mwords = (si.kv + 31) / 32;
    uint32_t mword[MAXRT];
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt) {
        mword[rt] = 0xffffffffu;
        if (has_mask && rt * 16 < mb_rows) {
            const int64_t wi = a.mask_off[b] + (int64_t)min(rt * 16 + ln, mb_rows - 1) * mwords + kw0 / 32;
            mword[rt] = (wi >= 0 && wi < a.mask_words) ? a.mask[wi] : 0u;
        }
    }
    float* macc = a.mass_accum + ((int64_t)b * a.H + h) * a.n_cap;
    const int key_t = kt * kKT + tid;
    const float mold =
        (tid < kKT && key_t < si.kv && key_t < a.n_cap && !a.mass_overwrite) ? macc[key_t] : 0.f;
    // keys: need the page entry
    const bool page_ok = page >= 0 && page < a.pool_pages;
    const int kw = kw0 + ln;                                 // this lane's key row for the A operand
    const bool key_ok = kw < si.kv && page_ok;
    const int64_t krow = key_ok ? (int64_t)page * 16 + (kw & 15) : 0;
    bf16x8 kf[4];
    uint2 kf8[4];                                            // KV8: codes, decoded after the waits
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if constexpr (KV8)
            kf8[ks] = *(const uint2*)(reinterpret_cast<const uint8_t*>(a.k) + krow * a.n_out + h * kHD + ks * 32 +
                                      g * 8);
        else
            kf[ks] = *(const bf16x8*)(a.k + krow * a.n_out + h * kHD + ks * 32 + g * 8);
    }

    mb = max(0, min(mb, min(a.max_mass, min(si.rows, 16 * MAXRT))));
    if (mb == 0) return;                                     // uniform: nothing to add
    // final log-sum-exp (base 2) of each window row, merged over the splits
    if (tid < mb) {
        float m = -INFINITY;
#pragma unroll
        for (int spl = 0; spl < MAXS; ++spl)
            if (spl < a.splits) m = fmaxf(m, ms[spl]);
        float l = 0.f;
#pragma unroll
        for (int spl = 0; spl < MAXS; ++spl)
            if (spl < a.splits) l += ls[spl] * exp2f(ms[spl] - m);
        s_lse[tid] = l > 0.f ? m + __log2f(l) : INFINITY;      // a row that sees nothing adds 0
    }
    __syncthreads();
    if constexpr (KV8) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = e4m3x8_to_bf16(kf8[ks].x, kf8[ks].y);
    }
    // C layout: register e of lane group g is key kw0 + 4g + e
    uint32_t kvalid = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) kvalid |= (page_ok && kw0 + 4 * g + e < si.kv ? 1u : 0u) << e;
    const int rtiles = (mb + 15) / 16;
    float csum[4] = {0.f, 0.f, 0.f, 0.f};                    // keys 16w + 4g + e
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt) {
        if (rt >= rtiles) continue;
        const int row = rt * 16 + ln;                        // this lane's window row (B operand / C column)
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qfr[rt][ks], st, 0, 0, 0);
        const float lse = row < mb ? s_lse[row] : INFINITY;
        uint32_t vis = row < mb ? kvalid : 0u;
        vis &= (mword[rt] >> ((kw0 + 4 * g) & 31)) & 0xfu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = ((vis >> e) & 1u) ? exp2f(fmaf(st[e], a.scale_log2, -lse)) : 0.f;
            csum[e] += row16_sum(p);
        }
    }
    if (ln == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s_csum[wave][g * 4 + e] = csum[e];
    }
    __syncthreads();
    if (tid < kKT && key_t < si.kv && key_t < a.n_cap) {
        const float norm = 1.f / ((float)a.H * (float)mb);
        macc[key_t] = mold + s_csum[tid >> 4][tid & 15] * norm;
    }
}

// fp32 path (parity-sized shapes): one workgroup per (sequence, head) walks the
// sequence's rows in order; exact two-pass softmax per row in LDS.
constexpr int kF32Threads = 256;
constexpr int kF32MaxKv = 4096;

__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(AttnArgs a, const float* q,
                                                               const float* kc, const float* vc,
                                                               float* o) {
    __shared__ float s_p[kF32MaxKv];
    __shared__ float s_colsum[kF32MaxKv];
    __shared__ float s_q[128];
    __shared__ float s_red[kF32Threads / 64];
    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int D = a.head_dim;
    const SeqInfo si = seq_info(a, b);
    const int r0 = max(0, min(a.cu_q[b], a.n_rows));
    const float scale = 1.f / sqrtf((float)D);
    int mb = (a.mass_count && a.mass_accum) ? a.mass_count[b] : 0;
    mb = max(0, min(mb, min(a.max_mass, si.rows)));
    for (int j = tid; j < si.kv; j += kF32Threads) s_colsum[j] = 0.f;
    const int64_t words = (si.kv + 31) / 32;
    for (int ri = 0; ri < si.rows; ++ri) {
        __syncthreads();
        for (int d = tid; d < D; d += kF32Threads) s_q[d] = q[(int64_t)(r0 + ri) * a.n_out + h * D + d];
        __syncthreads();
        float mx = -INFINITY;
        for (int j = tid; j < si.kv; j += kF32Threads) {
            int p = a.page_table[(int64_t)b * a.max_pages + (j >> 4)];
            bool ok = p >= 0 && p < a.pool_pages;
            if (ok && a.mask) {
                int64_t wi = a.mask_off[b] + ri * words + j / 32;
                ok = wi >= 0 && wi < a.mask_words && ((a.mask[wi] >> (j & 31)) & 1u);
            }
            float s = -INFINITY;
            if (ok) {
                const float* kr = kc + ((int64_t)p * 16 + (j & 15)) * a.n_out + h * D;
                float acc = 0.f;
                for (int d = 0; d < D; ++d) acc = fmaf(s_q[d], kr[d], acc);
                s = acc * scale;
            }
            s_p[j] = s;
            mx = fmaxf(mx, s);
        }
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if ((tid & 63) == 0) s_red[tid >> 6] = mx;
        __syncthreads();
        mx = s_red[0];
        for (int w = 1; w < kF32Threads / 64; ++w) mx = fmaxf(mx, s_red[w]);
        __syncthreads();
        float sum = 0.f;
        for (int j = tid; j < si.kv; j += kF32Threads) {
            float e = (mx == -INFINITY || s_p[j] == -INFINITY) ? 0.f : expf(s_p[j] - mx);
            s_p[j] = e;
            sum += e;
        }
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if ((tid & 63) == 0) s_red[tid >> 6] = sum;
        __syncthreads();
        sum = 0.f;
        for (int w = 0; w < kF32Threads / 64; ++w) sum += s_red[w];
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
        for (int j = tid; j < si.kv; j += kF32Threads) {
            float p = s_p[j] * inv;
            s_p[j] = p;
            if (ri < mb) s_colsum[j] += p;
        }
        __syncthreads();
        for (int d = tid; d < D; d += kF32Threads) {
            float acc = 0.f;
            for (int j = 0; j < si.kv; ++j) {
                float p = s_p[j];
                if (p != 0.f) {
                    int pg = a.page_table[(int64_t)b * a.max_pages + (j >> 4)];
                    acc = fmaf(p, vc[((int64_t)pg * 16 + (j & 15)) * a.n_out + h * D + d], acc);
                }
            }
            o[(int64_t)(r0 + ri) * a.n_out + h * D + d] = acc;
        }
    }
    if (mb == 0 || si.kv == 0) return;
    __syncthreads();
    const float norm = 1.f / ((float)a.H * (float)mb);
    float* macc = a.mass_accum + ((int64_t)b * a.H + h) * a.n_cap;
    for (int j = tid; j < si.kv && j < a.n_cap; j += kF32Threads)
        macc[j] = (a.mass_overwrite ? 0.f : macc[j]) + s_colsum[j] * norm;
}

// Items = (sequence, head, 128-row query tile[, key split]); the launch is
// sized for the worst case sum_b ceil(rows_b / 128) <= n_rows / 128 + n_seq,
// and surplus workgroups exit after the schedule scan.
//
// When batch x heads cannot fill the chip (one workgroup streams at most
// ~50 GB/s), keys are split so that roughly 512 workgroups stream them, and a
// second launch merges the splits and forms the column mass.
// The attn_splits tuning override (DLLM_ATTN_SPLITS, read once per process,
// or dllm_set_tuning) forces the split count; the workspace query reads the
// same stored value, so the two agree.
int choose_splits(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int max_kv) {
    if (dt != DLLM_BF16 && dt != DLLM_BF16_E4M3KV) return 1;
    const int ktiles = (max_kv + kKT - 1) / kKT;
    int s = 1;
    const int qtiles = (n_rows + kQT - 1) / kQT;
    const int est = n_heads * (n_seq > qtiles ? n_seq : qtiles);
    if (est < kNumCu) {
        s = (2 * kNumCu + est - 1) / est;
        const int cap = ktiles / 2 > 1 ? ktiles / 2 : 1;     // at least two tiles per split
        if (s > cap) s = cap;
    }
    if (const int forced = tuning_attn_splits(); forced > 0) s = forced;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s > ktiles) s = ktiles > 0 ? ktiles : 1;
    return s < 1 ? 1 : s;
}

int64_t first_items(int n_seq, int n_rows, int n_heads, int splits, int qt_rows) {
    return (int64_t)n_heads * (n_rows / qt_rows + n_seq) * splits;
}

// Split launches without a mask, with at most 64 score rows and with fewer
// 128-row items than compute units use 64-row query tiles (each wave one
// 16-row MFMA tile): twice the workgroups and half the dependent MFMA and
// softmax work per wave per key tile, which is what such a launch (latency-
// bound) waits on.  Where the 128-row items already fill the compute units
// the doubled grid measured slower (the verify step: 58 -> 65 us).
constexpr int kSplitQT = 64;
bool split_rt1(int n_seq, int n_rows, int n_heads, int splits, bool mask, int mass_rows) {
    return splits > 1 && !mask && mass_rows <= kSplitQT &&
           first_items(n_seq, n_rows, n_heads, splits, kQT) <= kNumCu;
}

// the workspace query does not see the mask: it sizes for 64-row tiles, the
// larger item count
size_t split_workspace(int n_seq, int n_rows, int n_heads, int splits) {
    if (splits <= 1) return 0;
    const int64_t items = first_items(n_seq, n_rows, n_heads, splits, kSplitQT);
    return (size_t)items * kQT * (kHD * sizeof(uint16_t) + 2 * sizeof(float));
}

int mass_tiles(int max_kv) { return (max_kv + kKT - 1) / kKT; }

// fused path with a score: the window rows' bf16 probabilities of every key
// tile and their exponent references, per (sequence, head)
size_t mass_workspace(int n_seq, int n_heads, int max_kv, int max_mass, int splits) {
    if (splits > 1 || max_mass <= 0) return 0;
    return (size_t)n_seq * n_heads * mass_tiles(max_kv) * max_mass * (kKT * sizeof(uint16_t) + sizeof(float));
}

size_t bf16_workspace(int n_seq, int n_rows, int n_heads, int max_kv, int max_mass, int splits) {
    return split_workspace(n_seq, n_rows, n_heads, splits) +
           mass_workspace(n_seq, n_heads, max_kv, max_mass, splits);
}

template <bool KV8>
void launch_attn(const AttnArgs& a, dim3 grid, dim3 block, bool mask, bool rt1, hipStream_t stream) {
    if (rt1) hipLaunchKernelGGL((attn_bf16_kernel<1, 2, false, KV8>), grid, block, 0, stream, a);
    else if (mask) hipLaunchKernelGGL((attn_bf16_kernel<2, 2, true, KV8>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<2, 2, false, KV8>), grid, block, 0, stream, a);
}

template <bool KV8, int MAXRT>
void launch_finish_rt(const AttnArgs& a, int splits, unsigned fin, hipStream_t stream) {
    if (splits <= 2) hipLaunchKernelGGL((attn_finish_kernel<2, KV8, MAXRT>), dim3(fin), dim3(kFinThreads), 0, stream, a);
    else if (splits <= 4) hipLaunchKernelGGL((attn_finish_kernel<4, KV8, MAXRT>), dim3(fin), dim3(kFinThreads), 0, stream, a);
    else if (splits <= 8) hipLaunchKernelGGL((attn_finish_kernel<8, KV8, MAXRT>), dim3(fin), dim3(kFinThreads), 0, stream, a);
    else hipLaunchKernelGGL((attn_finish_kernel<16, KV8, MAXRT>), dim3(fin), dim3(kFinThreads), 0, stream, a);
}

// the window rows' tile count (a.max_mass <= kQT) picks the instantiation
template <bool KV8>
void launch_finish(const AttnArgs& a, int splits, unsigned fin, hipStream_t stream) {
    if (a.max_mass <= 32) launch_finish_rt<KV8, 2>(a, splits, fin, stream);
    else if (a.max_mass <= 64) launch_finish_rt<KV8, 4>(a, splits, fin, stream);
    else launch_finish_rt<KV8, kQT / 16>(a, splits, fin, stream);
}

int check_attn(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim, int page_size,
               int max_kv, int n_cap) {
    DLLM_CHECK_ARG(n_seq > 0 && n_rows >= 0 && n_heads > 0 && max_kv > 0 && n_cap >= 0);
    DLLM_CHECK_SUP(dt == DLLM_BF16 || dt == DLLM_F32 || dt == DLLM_BF16_E4M3KV);
    DLLM_CHECK_SUP(page_size == 16);
    DLLM_CHECK_SUP(n_seq <= kMaxSeq);
    if (dt != DLLM_F32) {
        DLLM_CHECK_SUP(head_dim == kHD);
        DLLM_CHECK_SUP(max_kv <= kMaxPages * 16);
    } else {
        DLLM_CHECK_SUP(head_dim == 64 || head_dim == 128);
        DLLM_CHECK_SUP(max_kv <= kF32MaxKv);
    }
    return DLLM_OK;
}

}  // namespace

extern "C" size_t dllm_sched_attention_workspace(dllm_dtype dt, int n_seq, int n_rows,
                                                 int n_heads, int head_dim, int max_kv,
                                                 int n_cap, int max_mass_rows) {
    if (check_attn(dt, n_seq, n_rows, n_heads, head_dim, 16, max_kv, n_cap) != DLLM_OK) return 0;
    if (dt == DLLM_F32 || max_mass_rows < 0 || max_mass_rows > kQT) return 0;
    return bf16_workspace(n_seq, n_rows, n_heads, max_kv, max_mass_rows,
                          choose_splits(dt, n_seq, n_rows, n_heads, max_kv));
}

namespace {

// Both attention entry points: argument checks, then the launches.  The
// workspace is either the caller's (dllm_sched_attention) or the static
// scratch array (dllm_sched_attention_noalloc): get_ws(ws_need, &ptr, &bytes)
// supplies it once the size is known, after every host-side check, or
// returns an error before anything is enqueued.
template <typename GetWs>
int attention_call(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim, int page_size,
                   int max_kv, const void* q, const int32_t* cu_q, const void* k_cache,
                   const void* v_cache, int64_t cache_rows, const int32_t* page_table, int max_pages,
                   const int32_t* kv_len, const uint32_t* mask_bits, const int64_t* mask_off,
                   int64_t mask_words, const int32_t* mass_count, int max_mass_rows, float* mass_accum,
                   int mass_overwrite, int n_cap, void* o, GetWs get_ws, hipStream_t stream) {
    int st = check_attn(dt, n_seq, n_rows, n_heads, head_dim, page_size, max_kv, n_cap);
    if (st != DLLM_OK) return st;
    DLLM_CHECK_ARG(max_pages > 0 && cache_rows >= 16);
    DLLM_CHECK_SUP(max_pages <= kMaxPages);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(q && cu_q && k_cache && v_cache && page_table && kv_len && o);
    DLLM_CHECK_ARG(!mask_bits || (mask_off && mask_words > 0));
    const bool want_mass = mass_count && mass_accum;
    DLLM_CHECK_ARG(!(mass_count || mass_accum) || want_mass);
    if (want_mass) {
        DLLM_CHECK_ARG(n_cap > 0);
        DLLM_CHECK_SUP(max_mass_rows >= 0 && max_mass_rows <= kQT);
        // the bf16 kernel sums a head's column mass in LDS: <= 8704 keys
        if (dt != DLLM_F32) DLLM_CHECK_SUP((max_kv < n_cap ? max_kv : n_cap) <= 8704);
    }
    const int splits = choose_splits(dt, n_seq, n_rows, n_heads, max_kv);
    const int mass_rows = want_mass ? max_mass_rows : 0;
    const size_t ws_need = dt == DLLM_F32 ? 0 : bf16_workspace(n_seq, n_rows, n_heads, max_kv, mass_rows, splits);
    void* workspace = nullptr;
    st = get_ws(ws_need, &workspace);
    if (st != DLLM_OK) return st;

    AttnArgs a{};
    a.n_seq = n_seq;
    a.n_rows = n_rows;
    a.H = n_heads;
    a.head_dim = head_dim;
    a.n_out = n_heads * head_dim;
    a.max_kv = max_kv;
    a.max_pages = max_pages;
    a.n_cap = n_cap;
    a.max_mass = want_mass ? max_mass_rows : 0;
    a.pool_pages = (int)(cache_rows / 16 < (1ll << 30) ? cache_rows / 16 : (1ll << 30));
    a.scale_log2 = kLog2e / sqrtf((float)head_dim);
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_cache;
    a.v = (const uint16_t*)v_cache;
    a.cu_q = cu_q;
    a.page_table = page_table;
    a.kv_len = kv_len;
    a.mask = mask_bits;
    a.mask_off = mask_off;
    a.mask_words = mask_words;
    a.mass_count = want_mass ? mass_count : nullptr;
    a.mass_accum = want_mass ? mass_accum : nullptr;
    a.mass_overwrite = mass_overwrite != 0;
    a.o = (uint16_t*)o;
    a.splits = splits;
    const bool rt1 = split_rt1(n_seq, n_rows, n_heads, splits, mask_bits != nullptr, mass_rows);
    a.qt_rows = rt1 ? kSplitQT : kQT;
    if (splits > 1) {
        const int64_t items = first_items(n_seq, n_rows, n_heads, splits, kSplitQT);   // as the workspace
        a.part_o = (uint16_t*)workspace;
        a.part_ml = (float*)(a.part_o + items * kQT * kHD);
    } else if (dt != DLLM_F32 && mass_rows > 0) {
        a.mass_tiles = mass_tiles(max_kv);
        a.mass_p = (uint16_t*)workspace;
        a.mass_ref = (float*)(a.mass_p + (int64_t)n_seq * n_heads * a.mass_tiles * mass_rows * kKT);
    }
    if (dt != DLLM_F32) {
        // 128-row query tiles: four waves of 32 rows (two 16-row MFMA tiles
        // each); 64-row tiles (one per wave) for the split launches above
        const int64_t items = first_items(n_seq, n_rows, n_heads, splits, a.qt_rows);
        DLLM_CHECK_SUP(items > 0 && items < (1ll << 30));
        const dim3 grid((unsigned)items), block(kAttnThreads);
        if (dt == DLLM_BF16_E4M3KV)
            launch_attn<true>(a, grid, block, mask_bits != nullptr, rt1, stream);
        else
            launch_attn<false>(a, grid, block, mask_bits != nullptr, rt1, stream);
        if (splits > 1) {
            DLLM_CHECK_LAUNCH();
            int64_t fin = (int64_t)n_heads * (n_rows / kMergeRows + n_seq);
            if (want_mass) fin += (int64_t)n_heads * n_seq * ((max_kv + kKT - 1) / kKT);
            DLLM_CHECK_SUP(fin < (1ll << 30));
            if (dt == DLLM_BF16_E4M3KV)
                launch_finish<true>(a, splits, (unsigned)fin, stream);
            else
                launch_finish<false>(a, splits, (unsigned)fin, stream);
        }
    } else {
        hipLaunchKernelGGL(attn_f32_kernel, dim3(n_seq * n_heads), dim3(kF32Threads), 0, stream,
                           a, (const float*)q, (const float*)k_cache, (const float*)v_cache,
                           (float*)o);
    }
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

}  // namespace

// Scratch memory of the allocation-free entry point, at file scope: one copy
// per device (each GPU that loads the library holds it until the process
// ends).  In host code `scratch` names a host-side stand-in; kernels get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[DLLM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = DLLM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (its address as host code must pass
// it), looked up with that device current on its first use
int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DLLM_ERR_HIP;
    if (dev >= kMaxDevices) return DLLM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DLLM_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DLLM_OK;
}

}  // namespace

extern "C" int dllm_sched_attention(dllm_dtype dt, int n_seq, int n_rows, int n_heads,
                                    int head_dim, int page_size, int max_kv, const void* q,
                                    const int32_t* cu_q, const void* k_cache, const void* v_cache,
                                    int64_t cache_rows, const int32_t* page_table, int max_pages,
                                    const int32_t* kv_len, const uint32_t* mask_bits,
                                    const int64_t* mask_off, int64_t mask_words,
                                    const int32_t* mass_count, int max_mass_rows,
                                    float* mass_accum, int mass_overwrite, int n_cap, void* o, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    auto caller_ws = [&](size_t need, void** ws) -> int {
        DLLM_CHECK_ARG(workspace_bytes >= need && (need == 0 || workspace != nullptr));
        *ws = workspace;
        return DLLM_OK;
    };
    return attention_call(dt, n_seq, n_rows, n_heads, head_dim, page_size, max_kv, q, cu_q, k_cache, v_cache,
                          cache_rows, page_table, max_pages, kv_len, mask_bits, mask_off, mask_words,
                          mass_count, max_mass_rows, mass_accum, mass_overwrite, n_cap, o, caller_ws, stream);
}

extern "C" int dllm_sched_attention_noalloc(dllm_dtype dt, int n_seq, int n_rows, int n_heads,
                                            int head_dim, int page_size, int max_kv, const void* q,
                                            const int32_t* cu_q, const void* k_cache, const void* v_cache,
                                            int64_t cache_rows, const int32_t* page_table, int max_pages,
                                            const int32_t* kv_len, const uint32_t* mask_bits,
                                            const int64_t* mask_off, int64_t mask_words,
                                            const int32_t* mass_count, int max_mass_rows,
                                            float* mass_accum, int mass_overwrite, int n_cap, void* o,
                                            hipStream_t stream) {
    auto static_ws = [](size_t need, void** ws) -> int {
        *ws = nullptr;
        if (need == 0) return DLLM_OK;
        DLLM_CHECK_SUP(need <= kNoAllocScratchBytes);
        return scratch_for_current_device(ws);
    };
    return attention_call(dt, n_seq, n_rows, n_heads, head_dim, page_size, max_kv, q, cu_q, k_cache, v_cache,
                          cache_rows, page_table, max_pages, kv_len, mask_bits, mask_off, mask_words,
                          mass_count, max_mass_rows, mass_accum, mass_overwrite, n_cap, o, static_ws, stream);
}
