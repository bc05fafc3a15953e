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
// query tile, key split) item.  Items are decoded on the device from cu_q and
// kv_len: each workgroup scans the per-sequence item counts (no host
// round-trip), and consecutive items (same head and key range, next query
// tile) are placed on the same XCD so they share its L2.  Eight waves own 16
// query rows each; 64-key tiles of K and of V^T are gathered through the
// block table into LDS.  S^T = K Q^T and O^T = V^T P^T run on
// v_mfma_f32_16x16x32_bf16: the K rows fed to the first product are permuted
// so that the P^T fragment a lane holds covers 8 consecutive keys, which makes
// the V^T fragment one 16-byte LDS read.  Softmax is online in fp32 (base 2).
// When a batch has too few items to fill the chip, keys are split across
// workgroups and the last split of a tile merges the partials in split order.
// The finalising workgroup of a sequence's first query tile then makes a
// second pass over K for the masked-window rows (their log-sum-exp is final
// only at that point), forms each key's column mass and, once all heads of the
// sequence are in, adds the head-ordered sum into mass_accum (deterministic).
#include <math.h>

#include "common.h"

namespace {

using namespace dllm;

constexpr int kQT = 128;             // query rows per item
constexpr int kKT = 64;              // keys per tile
constexpr int kHD = 128;             // head dim of the bf16 kernel
constexpr int kThreads = 512;        // 8 waves x 16 rows
constexpr int kLDK = kHD + 8;        // K tile row stride, halfwords (272 B)
constexpr int kLDV = kKT + 8;        // V^T tile row stride, halfwords (144 B)
constexpr int kMaxSeq = 1024;
constexpr int kMaxPages = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

struct AttnArgs {
    int n_seq, n_rows, H, n_out, max_kv, max_pages, n_cap, split_max, max_mass, pool_pages;
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
    float* mass_accum;
    uint16_t* o;
    int32_t* cnt_tile;      // [max_items]
    int32_t* cnt_mass;      // [n_seq]
    float* mass_part;       // [n_seq, H, n_cap]
    float* part_o;          // [max_items, QT, HD]
    float* part_ml;         // [max_items, QT, 2]
};

struct SeqInfo {
    int rows, kv, nqt, splits;
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b) {
    SeqInfo s;
    int r0 = a.cu_q[b], r1 = a.cu_q[b + 1];
    r0 = max(0, min(r0, a.n_rows));
    r1 = max(r0, min(r1, a.n_rows));
    s.rows = r1 - r0;
    int kv = a.kv_len[b];
    kv = max(0, min(kv, min(a.max_kv, a.max_pages * 16)));
    s.kv = kv;
    s.nqt = (s.rows + kQT - 1) / kQT;
    int ktiles = (kv + kKT - 1) / kKT;
    int want = max(1, min(a.split_max, ktiles));
    int per = ktiles > 0 ? (ktiles + want - 1) / want : 1;
    s.splits = ktiles > 0 ? (ktiles + per - 1) / per : 1;    // every split gets keys
    return s;
}

__device__ __forceinline__ float wave_max16(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
// sum over the 16 lanes that share lane >> 4
__device__ __forceinline__ float group_sum16(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// Key (within a 64-key tile) that A-row m of sub-tile t feeds to S^T.
__device__ __forceinline__ int perm_key(int t, int m) {
    return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}
// Key of S^T register e of sub-tile t held by lane group g.
__device__ __forceinline__ int reg_key(int t, int g, int e) {
    return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
}

__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * kLDK];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[kHD * kLDV];
    __shared__ int s_pref[kMaxSeq + 1];
    __shared__ int s_pages[kMaxPages];
    __shared__ float s_col[8][kKT];
    __shared__ int s_total, s_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, ln = lane & 15;

    // ---- schedule: per-sequence item counts, prefix-summed by wave 0 ----
    if (wave == 0) {
        int base = 0;
        for (int c = 0; c < a.n_seq; c += 64) {
            int b = c + lane;
            int items = 0;
            if (b < a.n_seq) {
                SeqInfo s = seq_info(a, b);
                items = s.nqt * s.splits * a.H;
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
            s_total = base;
        }
    }
    __syncthreads();
    // a malformed cu_q (not non-decreasing) can claim more items than were
    // launched: then nothing runs (outputs unspecified, no access past the
    // workspace)
    const int total = s_total;
    if (total > (int)gridDim.x || (int)blockIdx.x >= total) return;
    const int item = xcd_remap(blockIdx.x, total);
    int lo = 0, hi = a.n_seq - 1;                       // last b with s_pref[b] <= item
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const SeqInfo si = seq_info(a, b);
    const int local = item - s_pref[b];
    const int qt = local % si.nqt;
    const int hs = local / si.nqt;
    const int sp = hs % si.splits;
    const int h = hs / si.splits;
    const int seq_r0 = max(0, min(a.cu_q[b], a.n_rows));
    const int r0 = seq_r0 + qt * kQT;
    const int nr = min(kQT, si.rows - qt * kQT);
    const int ktiles = (si.kv + kKT - 1) / kKT;
    const int tiles_per = (ktiles + si.splits - 1) / si.splits;
    const int k_lo = sp * tiles_per * kKT;
    const int k_hi = min(si.kv, k_lo + tiles_per * kKT);
    const int npages = (si.kv + 15) / 16;
    for (int j = tid; j < npages; j += kThreads) {
        int p = a.page_table[(int64_t)b * a.max_pages + j];
        s_pages[j] = (p >= 0 && p < a.pool_pages) ? p : -1;
    }
    __syncthreads();

    // ---- query fragments (B operand of S^T = K Q^T) ----
    const int wrow = wave * 16;                 // this wave's first row within the tile
    const bool active = wrow < nr;
    const int my_row = wrow + ln;               // row (within tile) this lane's column holds
    const bool row_ok = my_row < nr;
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (row_ok) {
            qf[ks] = *(const bf16x8*)(a.q + (int64_t)(r0 + my_row) * a.n_out + h * kHD + ks * 32 + g * 8);
        } else {
            u32x4 z = {0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(bf16x8, z);
        }
    }
    const bool has_mask = a.mask != nullptr;
    const int64_t mrow_base = has_mask ? a.mask_off[b] + (int64_t)(qt * kQT + my_row) * ((si.kv + 31) / 32) : 0;

    u32x4 rk[2], rv[2];
    auto gload = [&](int kbase, bool with_v) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * kThreads;
            int key = c >> 4, dc = c & 15;
            int kg = kbase + key;
            int page = (kg < si.kv) ? s_pages[kg >> 4] : -1;
            u32x4 z = {0u, 0u, 0u, 0u};
            rk[i] = z;
            rv[i] = z;
            if (page >= 0) {
                int64_t off = ((int64_t)page * 16 + (kg & 15)) * a.n_out + h * kHD + dc * 8;
                rk[i] = *(const u32x4*)(a.k + off);
                if (with_v) rv[i] = *(const u32x4*)(a.v + off);
            }
        }
    };
    auto lstore = [&](bool with_v) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * kThreads;
            int key = c >> 4, dc = c & 15;
            *(u32x4*)(sK + key * kLDK + dc * 8) = rk[i];
            if (with_v) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sVt[(dc * 8 + 2 * e) * kLDV + key] = (uint16_t)(rv[i][e] & 0xffffu);
                    sVt[(dc * 8 + 2 * e + 1) * kLDV + key] = (uint16_t)(rv[i][e] >> 16);
                }
            }
        }
    };
    // S^T for one 64-key tile: 4 sub-tiles of 16 keys x this wave's 16 rows
    auto scores = [&](f32x4 (&st)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* krow = sK + perm_key(t, ln) * kLDK + g * 8;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 kf = *(const bf16x8*)(krow + ks * 32);
                st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], st[t], 0, 0, 0);
            }
        }
    };
    // visibility of this lane's 16 scores in the tile starting at kbase
    auto visible_bits = [&](int kbase) -> uint32_t {
        uint32_t bits = 0;
        uint32_t w0 = 0xffffffffu, w1 = 0xffffffffu;
        if (has_mask) {
            w0 = w1 = 0u;
            if (row_ok) {
                int64_t i0 = mrow_base + kbase / 32;
                if (i0 >= 0 && i0 < a.mask_words) w0 = a.mask[i0];
                if (i0 + 1 >= 0 && i0 + 1 < a.mask_words) w1 = a.mask[i0 + 1];
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int kk = reg_key(t, g, e);
                int kg = kbase + kk;
                bool ok = kg < k_hi && kg < si.kv && s_pages[kg >> 4] >= 0;
                uint32_t w = (kk < 32) ? w0 : w1;
                ok = ok && ((w >> (kk & 31)) & 1u);
                bits |= (ok ? 1u : 0u) << (t * 4 + e);
            }
        return bits;
    };

    // ---- main pass over this split's keys ----
    float m_run = kNegBig, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nt_main = (k_hi - k_lo + kKT - 1) / kKT;
    if (nt_main > 0) {
        gload(k_lo, true);
        lstore(true);
    }
    __syncthreads();
    for (int t = 0; t < nt_main; ++t) {
        const int kbase = k_lo + t * kKT;
        if (t + 1 < nt_main) gload(kbase + kKT, true);
        if (active) {
            f32x4 st[4];
            scores(st);
            uint32_t vis = visible_bits(kbase);
            float mx = kNegBig;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float s = st[tt][e] * a.scale_log2;
                    s = ((vis >> (tt * 4 + e)) & 1u) ? s : -INFINITY;
                    st[tt][e] = s;
                    mx = fmaxf(mx, s);
                }
            mx = wave_max16(mx);
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f(m_run - m_new);
            float rs = 0.f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float p = exp2f(st[tt][e] - m_new);
                    st[tt][e] = p;
                    rs += p;
                }
            rs = wave_sum16(rs);
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
            bf16x8 pf[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 u;
                u[0] = pack_bf16x2(st[2 * c][0], st[2 * c][1]);
                u[1] = pack_bf16x2(st[2 * c][2], st[2 * c][3]);
                u[2] = pack_bf16x2(st[2 * c + 1][0], st[2 * c + 1][1]);
                u[3] = pack_bf16x2(st[2 * c + 1][2], st[2 * c + 1][3]);
                pf[c] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    bf16x8 vf = *(const bf16x8*)(sVt + (dt * 16 + ln) * kLDV + c * 32 + g * 8);
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[c], acc[dt], 0, 0, 0);
                }
        }
        __syncthreads();
        if (t + 1 < nt_main) lstore(true);
        __syncthreads();
    }

    // ---- merge key splits (last split of the tile finishes) ----
    const int tile_item = s_pref[b] + (h * si.splits) * si.nqt + qt;   // split-0 item of this tile
    if (si.splits > 1) {
        float* po = a.part_o + (int64_t)item * kQT * kHD;
        float* pml = a.part_ml + (int64_t)item * kQT * 2;
        if (active) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *(f32x4*)(po + my_row * kHD + dt * 16 + g * 4) = acc[dt];
            if (g == 0) {
                pml[my_row * 2] = m_run;
                pml[my_row * 2 + 1] = l_run;
            }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) s_flag = (atomicAdd(&a.cnt_tile[tile_item], 1) == si.splits - 1);
        __syncthreads();
        if (!s_flag) return;
        __threadfence();
        if (active) {
            float m = kNegBig;
            for (int s = 0; s < si.splits; ++s) {
                int it = s_pref[b] + (h * si.splits + s) * si.nqt + qt;
                m = fmaxf(m, a.part_ml[(int64_t)it * kQT * 2 + my_row * 2]);
            }
            float l = 0.f;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < si.splits; ++s) {
                int it = s_pref[b] + (h * si.splits + s) * si.nqt + qt;
                float ms = a.part_ml[(int64_t)it * kQT * 2 + my_row * 2];
                float ls = a.part_ml[(int64_t)it * kQT * 2 + my_row * 2 + 1];
                float f = exp2f(ms - m);
                l += ls * f;
                const float* pos = a.part_o + (int64_t)it * kQT * kHD + my_row * kHD + g * 4;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[dt] += *(const f32x4*)(pos + dt * 16) * f;
            }
            m_run = m;
            l_run = l;
        }
        if (tid == 0) a.cnt_tile[tile_item] = 0;
    }

    // ---- final output ----
    if (row_ok) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t* orow = a.o + (int64_t)(r0 + my_row) * a.n_out + h * kHD + g * 4;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            uint2 u;
            u.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
            u.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
            *(uint2*)(orow + dt * 16) = u;
        }
    }

    // ---- formula (2): column mass of the masked-window rows ----
    if (qt != 0 || a.mass_accum == nullptr || a.mass_count == nullptr) return;
    int mb = a.mass_count[b];
    mb = max(0, min(mb, min(a.max_mass, min(si.rows, kQT))));
    if (mb == 0 || si.kv == 0) return;
    const int mass_waves = (mb + 15) / 16;
    const bool mwave = wave < mass_waves;
    const bool mrow = my_row < mb;
    const float inv_l = (mrow && l_run > 0.f) ? 1.f / l_run : 0.f;
    float* mpart = a.mass_part + ((int64_t)b * a.H + h) * a.n_cap;
    const int nt_all = ktiles;
    __syncthreads();
    gload(0, false);
    lstore(false);
    __syncthreads();
    for (int t = 0; t < nt_all; ++t) {
        const int kbase = t * kKT;
        if (t + 1 < nt_all) gload(kbase + kKT, false);
        if (mwave) {
            f32x4 st[4];
            scores(st);
            // visibility over the whole key range (not just one split)
            uint32_t w0 = 0xffffffffu, w1 = 0xffffffffu;
            if (has_mask) {
                w0 = w1 = 0u;
                if (row_ok) {
                    int64_t i0 = mrow_base + kbase / 32;
                    if (i0 >= 0 && i0 < a.mask_words) w0 = a.mask[i0];
                    if (i0 + 1 >= 0 && i0 + 1 < a.mask_words) w1 = a.mask[i0 + 1];
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int kk = reg_key(tt, g, e);
                    int kg = kbase + kk;
                    uint32_t w = (kk < 32) ? w0 : w1;
                    bool ok = mrow && kg < si.kv && s_pages[kg >> 4] >= 0 && ((w >> (kk & 31)) & 1u);
                    float p = ok ? exp2f(st[tt][e] * a.scale_log2 - m_run) * inv_l : 0.f;
                    p = group_sum16(p);
                    if (ln == 0) s_col[wave][kk] = p;
                }
        }
        __syncthreads();
        if (tid < kKT) {
            float s = 0.f;
            for (int w = 0; w < mass_waves; ++w) s += s_col[w][tid];
            int kg = kbase + tid;
            if (kg < si.kv && kg < a.n_cap) mpart[kg] = s;
        }
        if (t + 1 < nt_all) lstore(false);
        __syncthreads();
    }
    // all heads of this sequence in: add the head-ordered sum into mass_accum
    __threadfence();
    __syncthreads();
    if (tid == 0) s_flag = (atomicAdd(&a.cnt_mass[b], 1) == a.H - 1);
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    const float norm = 1.f / ((float)a.H * (float)mb);
    const int kmax = min(si.kv, a.n_cap);
    const float* base = a.mass_part + (int64_t)b * a.H * a.n_cap;
    for (int i = tid; i < kmax; i += kThreads) {
        float s = 0.f;
        for (int hh = 0; hh < a.H; ++hh) s += base[(int64_t)hh * a.n_cap + i];
        a.mass_accum[(int64_t)b * a.n_cap + i] += s * norm;
    }
    if (tid == 0) a.cnt_mass[b] = 0;
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
    __shared__ int s_flag;
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
    float* mpart = a.mass_part + ((int64_t)b * a.H + h) * a.n_cap;
    __syncthreads();
    for (int j = tid; j < si.kv && j < a.n_cap; j += kF32Threads) mpart[j] = s_colsum[j];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_flag = (atomicAdd(&a.cnt_mass[b], 1) == a.H - 1);
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    const float norm = 1.f / ((float)a.H * (float)mb);
    const float* base = a.mass_part + (int64_t)b * a.H * a.n_cap;
    for (int i = tid; i < si.kv && i < a.n_cap; i += kF32Threads) {
        float s = 0.f;
        for (int hh = 0; hh < a.H; ++hh) s += base[(int64_t)hh * a.n_cap + i];
        a.mass_accum[(int64_t)b * a.n_cap + i] += s * norm;
    }
    if (tid == 0) a.cnt_mass[b] = 0;
}

struct AttnPlan {
    int split_max, max_items;
    size_t cnt_tile_bytes, cnt_mass_bytes, mass_part_bytes, part_o_bytes, part_ml_bytes;
    size_t total() const {
        return cnt_tile_bytes + cnt_mass_bytes + mass_part_bytes + part_o_bytes + part_ml_bytes;
    }
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

AttnPlan plan(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim, int max_kv,
              int n_cap) {
    AttnPlan p{};
    if (dt == DLLM_BF16) {
        int base_tiles = n_rows / kQT + n_seq;
        int est = n_heads * (n_seq > (n_rows + kQT - 1) / kQT ? n_seq : (n_rows + kQT - 1) / kQT);
        int s = 1;
        if (est < 4 * kNumCu) s = (4 * kNumCu + est - 1) / est;
        int ktiles = (max_kv + kKT - 1) / kKT;
        if (s > ktiles) s = ktiles;
        if (s > 16) s = 16;
        if (s < 1) s = 1;
        p.split_max = s;
        p.max_items = n_heads * base_tiles * s;
        p.cnt_tile_bytes = round256((size_t)p.max_items * sizeof(int32_t));
        if (s > 1) {
            p.part_o_bytes = round256((size_t)p.max_items * kQT * kHD * sizeof(float));
            p.part_ml_bytes = round256((size_t)p.max_items * kQT * 2 * sizeof(float));
        }
    } else {
        p.split_max = 1;
        p.max_items = n_seq * n_heads;
    }
    p.cnt_mass_bytes = round256((size_t)n_seq * sizeof(int32_t));
    p.mass_part_bytes = round256((size_t)n_seq * n_heads * n_cap * sizeof(float));
    (void)head_dim;
    return p;
}

int check_attn(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim, int page_size,
               int max_kv, int n_cap) {
    DLLM_CHECK_ARG(n_seq > 0 && n_rows >= 0 && n_heads > 0 && max_kv > 0 && n_cap >= 0);
    DLLM_CHECK_SUP(dt == DLLM_BF16 || dt == DLLM_F32);
    DLLM_CHECK_SUP(page_size == 16);
    DLLM_CHECK_SUP(n_seq <= kMaxSeq);
    if (dt == DLLM_BF16) {
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
                                                 int n_cap) {
    if (check_attn(dt, n_seq, n_rows, n_heads, head_dim, 16, max_kv, n_cap) != DLLM_OK) return 0;
    return plan(dt, n_seq, n_rows, n_heads, head_dim, max_kv, n_cap).total();
}

extern "C" int dllm_sched_attention(dllm_dtype dt, int n_seq, int n_rows, int n_heads,
                                    int head_dim, int page_size, int max_kv, const void* q,
                                    const int32_t* cu_q, const void* k_cache, const void* v_cache,
                                    int64_t cache_rows, const int32_t* page_table, int max_pages,
                                    const int32_t* kv_len, const uint32_t* mask_bits,
                                    const int64_t* mask_off, int64_t mask_words,
                                    const int32_t* mass_count, int max_mass_rows,
                                    float* mass_accum, int n_cap, void* o, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    int st = check_attn(dt, n_seq, n_rows, n_heads, head_dim, page_size, max_kv, n_cap);
    if (st != DLLM_OK) return st;
    DLLM_CHECK_ARG(max_pages > 0 && cache_rows >= 0);
    DLLM_CHECK_SUP(max_pages <= kMaxPages);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(q && cu_q && k_cache && v_cache && page_table && kv_len && o);
    DLLM_CHECK_ARG(!mask_bits || (mask_off && mask_words > 0));
    const bool want_mass = mass_count && mass_accum;
    DLLM_CHECK_ARG(!(mass_count || mass_accum) || want_mass);
    if (want_mass) {
        DLLM_CHECK_ARG(n_cap > 0);
        DLLM_CHECK_SUP(max_mass_rows >= 0 && max_mass_rows <= kQT);
    }
    AttnPlan p = plan(dt, n_seq, n_rows, n_heads, head_dim, max_kv, n_cap);
    DLLM_CHECK_ARG(workspace && workspace_bytes >= p.total());

    AttnArgs a{};
    a.n_seq = n_seq;
    a.n_rows = n_rows;
    a.H = n_heads;
    a.head_dim = head_dim;
    a.n_out = n_heads * head_dim;
    a.max_kv = max_kv;
    a.max_pages = max_pages;
    a.n_cap = n_cap;
    a.split_max = p.split_max;
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
    a.o = (uint16_t*)o;
    char* ws = (char*)workspace;
    a.cnt_tile = (int32_t*)ws;
    ws += p.cnt_tile_bytes;
    a.cnt_mass = (int32_t*)ws;
    ws += p.cnt_mass_bytes;
    a.mass_part = (float*)ws;
    ws += p.mass_part_bytes;
    a.part_o = p.part_o_bytes ? (float*)ws : nullptr;
    ws += p.part_o_bytes;
    a.part_ml = p.part_ml_bytes ? (float*)ws : nullptr;

    if (dt == DLLM_BF16) {
        DLLM_CHECK_SUP(p.max_items > 0 && p.max_items < (1 << 30));
        hipLaunchKernelGGL(attn_bf16_kernel, dim3(p.max_items), dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(attn_f32_kernel, dim3(n_seq * n_heads), dim3(kF32Threads), 0, stream,
                           a, (const float*)q, (const float*)k_cache, (const float*)v_cache,
                           (float*)o);
    }
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}
