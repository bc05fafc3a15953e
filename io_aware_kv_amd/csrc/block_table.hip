// a0: block table over a shared page pool and the per-row cache slot map.
//
// [FD] = "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (paper summary page).  核心方法 and
// 技术新颖性 describe the block table that aligns each sequence's query blocks
// with its KV blocks; 方法步骤详情 step 1 preallocates the flat cache once.
#include <vector>

#include "common.h"

namespace {

__global__ void map_slots_kernel(int n_seq, int n_rows, int page_size, int max_pages,
                                 int pool_pages, const int32_t* __restrict__ cu_q,
                                 const int32_t* __restrict__ q_logical,
                                 const int32_t* __restrict__ page_table,
                                 int32_t* __restrict__ slot) {
    int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= n_rows) return;
    // sequence of row r: the last b with cu_q[b] <= r (binary search)
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_q[mid] <= r) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    int s = -1;
    if (r >= cu_q[b] && r < cu_q[b + 1]) {
        int l = q_logical[r];
        if (l >= 0) {
            int j = l / page_size;
            if (j < max_pages) {
                int page = page_table[(int64_t)b * max_pages + j];
                if (page >= 0 && page < pool_pages) s = page * page_size + l % page_size;
            }
        }
    }
    slot[r] = s;
}

}  // namespace

extern "C" int dllm_map_slots(int n_seq, int n_rows, int page_size, int max_pages, int pool_pages,
                              const int32_t* cu_q, const int32_t* q_logical,
                              const int32_t* page_table, int32_t* slot, hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq > 0 && n_rows >= 0 && page_size > 0 && max_pages > 0 && pool_pages >= 0);
    if (n_rows == 0) return DLLM_OK;
    DLLM_CHECK_ARG(cu_q && q_logical && page_table && slot);
    int threads = 256;
    int blocks = (n_rows + threads - 1) / threads;
    hipLaunchKernelGGL(map_slots_kernel, dim3(blocks), dim3(threads), 0, stream, n_seq, n_rows,
                       page_size, max_pages, pool_pages, cu_q, q_logical, page_table, slot);
    DLLM_CHECK_LAUNCH();
    return DLLM_OK;
}

extern "C" int dllm_build_block_table(int n_seq, int page_size, int pool_pages, int max_pages,
                                      const int32_t* seq_pages, const int32_t* pool_perm,
                                      int32_t* page_table, int n_rows, const int32_t* cu_q,
                                      const int32_t* q_logical, int32_t* slot,
                                      hipStream_t stream) {
    DLLM_CHECK_ARG(n_seq > 0 && page_size > 0 && pool_pages >= 0 && max_pages > 0);
    DLLM_CHECK_ARG(seq_pages && page_table && (pool_pages == 0 || pool_perm));
    const bool with_rows = (cu_q || q_logical || slot || n_rows);
    if (with_rows) DLLM_CHECK_ARG(cu_q && slot && n_rows >= 0 && (n_rows == 0 || q_logical));

    int64_t total = 0;
    for (int b = 0; b < n_seq; ++b) {
        DLLM_CHECK_ARG(seq_pages[b] >= 0);
        if (seq_pages[b] > max_pages) return DLLM_ERR_OUT_OF_RANGE;
        total += seq_pages[b];
    }
    if (total > pool_pages) return DLLM_ERR_OUT_OF_RANGE;
    std::vector<uint8_t> seen(pool_pages, 0);
    for (int i = 0; i < pool_pages; ++i) {
        int p = pool_perm[i];
        if (p < 0 || p >= pool_pages || seen[p]) return DLLM_ERR_OUT_OF_RANGE;
        seen[p] = 1;
    }
    std::vector<int32_t> table((size_t)n_seq * max_pages, -1);
    int64_t taken = 0;
    for (int b = 0; b < n_seq; ++b) {
        for (int j = 0; j < seq_pages[b]; ++j) table[(size_t)b * max_pages + j] = pool_perm[taken + j];
        taken += seq_pages[b];
    }

    std::vector<int32_t> slots;
    if (with_rows) {
        DLLM_CHECK_ARG(cu_q[0] == 0 && cu_q[n_seq] == n_rows);
        for (int b = 0; b < n_seq; ++b) DLLM_CHECK_ARG(cu_q[b] <= cu_q[b + 1]);
        slots.resize(n_rows);
        std::vector<uint8_t> used((size_t)pool_pages * page_size, 0);
        for (int b = 0; b < n_seq; ++b) {
            for (int r = cu_q[b]; r < cu_q[b + 1]; ++r) {
                int l = q_logical[r];
                if (l < 0 || l / page_size >= seq_pages[b]) return DLLM_ERR_OUT_OF_RANGE;
                int s = table[(size_t)b * max_pages + l / page_size] * page_size + l % page_size;
                if (used[s]) return DLLM_ERR_OUT_OF_RANGE;   // two rows, one slot: a write race
                used[s] = 1;
                slots[r] = s;
            }
        }
    }

    if (hipMemcpyAsync(page_table, table.data(), table.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
        return DLLM_ERR_HIP;
    if (with_rows && n_rows > 0 &&
        hipMemcpyAsync(slot, slots.data(), slots.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
        return DLLM_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return DLLM_ERR_HIP;
    return DLLM_OK;
}

extern "C" const char* dllm_status_string(int status) {
    switch (status) {
        case DLLM_OK: return "ok";
        case DLLM_ERR_INVALID_ARG: return "invalid argument";
        case DLLM_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case DLLM_ERR_OUT_OF_RANGE: return "index out of range or duplicate slot";
        case DLLM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int dllm_version(void) { return 100; }
