// api.hip -- status strings, the scratch pool, launch timing and the share
// knob of the segmented-reduction library.
#include <atomic>
#include <mutex>
#include <vector>

#include "internal.hpp"

namespace segred {

namespace {

std::mutex g_pool_mu;
std::vector<hipMemPool_t> g_pools;  // one per device, created on first use

hipMemPool_t pool_for_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if ((int)g_pools.size() <= dev) g_pools.resize(dev + 1, nullptr);
    if (!g_pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) return nullptr;
        uint64_t keep = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        g_pools[dev] = pool;
    }
    return g_pools[dev];
}

constexpr int kMaxTimed = 4096;
struct Timing {
    bool on = false;
    int used = 0;
    hipEvent_t ev[2 * kMaxTimed] = {};
    bool created = false;
};
Timing g_timing;

std::atomic<int64_t> g_shares{0};

}  // namespace

int scratch_alloc(void **ptr, size_t bytes, hipStream_t stream) {
    *ptr = nullptr;
    if (bytes == 0) return SEGRED_OK;
    hipMemPool_t pool = pool_for_current_device();
    if (!pool) return SEGRED_ERR_HIP;
    hipError_t e = hipMallocFromPoolAsync(ptr, bytes, pool, stream);
    if (e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        return SEGRED_ERR_OUT_OF_MEMORY;
    }
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

void scratch_free(void *ptr, hipStream_t stream) {
    if (ptr) (void)hipFreeAsync(ptr, stream);
}

bool timing_on() { return g_timing.on; }

int timing_begin(hipStream_t stream) {
    if (!g_timing.on || g_timing.used >= kMaxTimed) return -1;
    int slot = g_timing.used++;
    if (hipEventRecord(g_timing.ev[2 * slot], stream) != hipSuccess) return -1;
    return slot;
}

void timing_end(int slot, hipStream_t stream) {
    if (slot >= 0) (void)hipEventRecord(g_timing.ev[2 * slot + 1], stream);
}

int64_t shares_override() { return g_shares.load(std::memory_order_relaxed); }

}  // namespace segred

using namespace segred;

extern "C" const char *segred_status_string(int status) {
    switch (status) {
    case SEGRED_OK: return "success";
    case SEGRED_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SEGRED_ERR_UNSUPPORTED: return "unsupported request (MEAN needs float32 values)";
    case SEGRED_ERR_OUT_OF_MEMORY: return "out of device memory for scratch";
    case SEGRED_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

extern "C" int segred_set_shares(int64_t shares) {
    if (shares != 0 && (shares < 1 || shares > (int64_t(1) << 22))) return SEGRED_ERR_INVALID_ARGUMENT;
    g_shares.store(shares, std::memory_order_relaxed);
    return SEGRED_OK;
}

extern "C" int segred_timing_enable(int enable) {
    if (enable && !g_timing.created) {
        for (int i = 0; i < 2 * kMaxTimed; ++i)
            if (hipEventCreate(&g_timing.ev[i]) != hipSuccess) return SEGRED_ERR_HIP;
        g_timing.created = true;
    }
    g_timing.on = enable != 0;
    g_timing.used = 0;
    return SEGRED_OK;
}

extern "C" int segred_timing_read(double *total_ms, int64_t *launches, float *each_ms, int64_t capacity) {
    if (!total_ms || !launches || capacity < 0 || (capacity > 0 && !each_ms)) return SEGRED_ERR_INVALID_ARGUMENT;
    double sum = 0.0;
    for (int i = 0; i < g_timing.used; ++i) {
        if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return SEGRED_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) return SEGRED_ERR_HIP;
        if (i < capacity) each_ms[i] = ms;
        sum += ms;
    }
    *total_ms = sum;
    *launches = g_timing.used;
    g_timing.used = 0;
    return SEGRED_OK;
}
