// Process-wide tuning overrides of the kernel choices (tests and tuning runs
// only; the automatic choices need none).  Each knob takes its first value
// from an environment variable, read once per process at first use, and can
// be changed later through dllm_set_tuning.  A workspace query and the call
// it sizes read the same stored value, so the two agree unless the caller
// changes a knob between them.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"

namespace dllm {
namespace {

constexpr const char* kQkvNames[] = {"tiled", "gemm", "g256x256", "g128x256", "g128x256o2", "g64x256",
                                     "g64x256o2", "g256x128", "g256x128o2", "g128x128", "g128x128o2",
                                     "mid6x6", "mid10x6", "mid12x6", "mid16x6", "mid4x12", "mid8x12"};
constexpr int kNumQkvNames = sizeof(kQkvNames) / sizeof(kQkvNames[0]);

std::atomic<int> g_attn_splits{0};     // 0: automatic
std::atomic<int> g_qkv_kernel{-1};     // -1: automatic, else an index into kQkvNames
std::once_flag g_env_once;

int parse_splits(const char* v, int* out) {
    if (!v || !*v) { *out = 0; return DLLM_OK; }
    char* end = nullptr;
    const long s = strtol(v, &end, 10);
    if (*end || s < 0 || s > 1024) return DLLM_ERR_INVALID_ARG;
    *out = (int)s;
    return DLLM_OK;
}

int parse_qkv(const char* v, int* out) {
    if (!v || !*v) { *out = -1; return DLLM_OK; }
    for (int i = 0; i < kNumQkvNames; ++i)
        if (!strcmp(v, kQkvNames[i])) { *out = i; return DLLM_OK; }
    return DLLM_ERR_INVALID_ARG;
}

void read_env() {
    std::call_once(g_env_once, [] {
        int v;
        if (parse_splits(getenv("DLLM_ATTN_SPLITS"), &v) == DLLM_OK) g_attn_splits.store(v);
        if (parse_qkv(getenv("DLLM_QKV_KERNEL"), &v) == DLLM_OK) g_qkv_kernel.store(v);
    });
}

}  // namespace

int tuning_attn_splits() {
    read_env();
    return g_attn_splits.load(std::memory_order_relaxed);
}

const char* tuning_qkv_kernel() {
    read_env();
    const int i = g_qkv_kernel.load(std::memory_order_relaxed);
    return i < 0 ? nullptr : kQkvNames[i];
}

}  // namespace dllm

extern "C" int dllm_set_tuning(const char* knob, const char* value) {
    using namespace dllm;
    DLLM_CHECK_ARG(knob != nullptr);
    read_env();              // a later first read must not undo this call
    int v;
    if (!strcmp(knob, "attn_splits")) {
        const int st = parse_splits(value, &v);
        if (st == DLLM_OK) g_attn_splits.store(v);
        return st;
    }
    if (!strcmp(knob, "qkv_kernel")) {
        const int st = parse_qkv(value, &v);
        if (st == DLLM_OK) g_qkv_kernel.store(v);
        return st;
    }
    return DLLM_ERR_INVALID_ARG;
}
