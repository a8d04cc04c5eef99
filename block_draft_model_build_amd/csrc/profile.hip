// Measurement hook: brackets the launches of one chosen kernel with hipEvents
// recorded on the launch's stream (dflash_profile_start / dflash_profile_stop).
#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace dflash {

namespace {
std::mutex g_mu;
std::atomic<int> g_kernel{-1};
std::vector<hipEvent_t> g_start, g_stop;
int g_count = 0;

void release_events() {
    for (hipEvent_t e : g_start) (void)hipEventDestroy(e);
    for (hipEvent_t e : g_stop) (void)hipEventDestroy(e);
    g_start.clear();
    g_stop.clear();
    g_count = 0;
}
}  // namespace

ProfScope::ProfScope(int kernel, hipStream_t st) : stream_(st), slot_(-1) {
    if (g_kernel.load(std::memory_order_relaxed) != kernel) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_kernel.load() != kernel || g_count >= (int)g_start.size()) return;
    slot_ = g_count++;
    (void)hipEventRecord(g_start[slot_], stream_);
}

ProfScope::~ProfScope() {
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if (slot_ < (int)g_stop.size()) (void)hipEventRecord(g_stop[slot_], stream_);
}

}  // namespace dflash

using namespace dflash;

extern "C" dflash_status dflash_profile_start(int32_t kernel, int32_t max_launches) {
    if (kernel < 0 || kernel >= DFLASH_KERNEL_COUNT || max_launches < 1) return DFLASH_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_mu);
    g_kernel.store(-1);
    release_events();
    g_start.resize(max_launches);
    g_stop.resize(max_launches);
    for (int i = 0; i < max_launches; ++i) {
        if (hipEventCreate(&g_start[i]) != hipSuccess || hipEventCreate(&g_stop[i]) != hipSuccess) {
            g_start.resize(i);
            g_stop.resize(i);
            release_events();
            return DFLASH_ERR_HIP;
        }
    }
    g_count = 0;
    g_kernel.store(kernel);
    return DFLASH_OK;
}

extern "C" dflash_status dflash_profile_stop(float* elapsed_ms, int32_t* launches) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_kernel.load() < 0) return DFLASH_ERR_INVALID_ARG;
    g_kernel.store(-1);
    dflash_status st = DFLASH_OK;
    for (int i = 0; i < g_count; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_stop[i]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_start[i], g_stop[i]) != hipSuccess)
            st = DFLASH_ERR_HIP;
        if (elapsed_ms) elapsed_ms[i] = ms;
    }
    if (launches) *launches = g_count;
    release_events();
    return st;
}
