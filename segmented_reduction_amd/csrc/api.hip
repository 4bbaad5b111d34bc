// api.hip -- status strings, the scratch pool, launch timing and the share
// knob of the segmented-reduction library.
#include <algorithm>
#include <atomic>
#include <map>
#include <memory>
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

constexpr int kMaxTimed = 8192;  // kernel launches recorded between reads
struct Timing {
    bool on = false;
    int used = 0;
    hipEvent_t start[kMaxTimed] = {};  // start and stop events of each launch, in launch order
    hipEvent_t stop[kMaxTimed] = {};
    bool streaming[kMaxTimed] = {};    // launch i is a streaming (first) kernel
    bool created = false;
};
Timing g_timing;

std::atomic<int64_t> g_shares{0};

struct CacheEntry {
    std::mutex mu;
    void *ptr = nullptr;
    size_t bytes = 0;
};
// keyed by (device, stream handle); entries live until the process ends
std::map<std::pair<int, uintptr_t>, std::unique_ptr<CacheEntry>> g_cache;

int pool_alloc(void **ptr, size_t bytes, hipStream_t stream) {
    *ptr = nullptr;
    hipMemPool_t pool = pool_for_current_device();
    if (!pool) return SEGRED_ERR_HIP;
    hipError_t e = hipMallocFromPoolAsync(ptr, bytes, pool, stream);
    if (e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        return SEGRED_ERR_OUT_OF_MEMORY;
    }
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

CacheEntry *cache_entry(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    const uintptr_t key = reinterpret_cast<uintptr_t>(stream);
    std::lock_guard<std::mutex> lk(g_pool_mu);
    auto it = g_cache.find({dev, key});
    if (it != g_cache.end()) return it->second.get();
    if ((int)g_cache.size() >= kScratchCacheEntries) return nullptr;
    auto &slot = g_cache[{dev, key}];
    slot = std::make_unique<CacheEntry>();
    return slot.get();
}

}  // namespace

ScratchLease::~ScratchLease() {
    if (owned_) (void)hipFreeAsync(owned_, stream_);
}

int scratch_acquire(ScratchLease &lease, size_t bytes, hipStream_t stream) {
    lease.stream_ = stream;
    if (bytes == 0) return SEGRED_OK;
    CacheEntry *e = bytes <= kScratchCacheBytes ? cache_entry(stream) : nullptr;
    if (!e) {
        int rc = pool_alloc(&lease.owned_, bytes, stream);
        lease.ptr = lease.owned_;
        return rc;
    }
    lease.lock_ = std::unique_lock<std::mutex>(e->mu);
    if (e->bytes < bytes) {
        // grow geometrically (1 MiB granules) so a ramp of sizes reallocates rarely
        size_t want = std::max(bytes, std::min(2 * e->bytes, kScratchCacheBytes));
        want = (want + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
        void *p = nullptr;
        int rc = pool_alloc(&p, want, stream);
        if (rc != SEGRED_OK) return rc;
        if (e->ptr) (void)hipFreeAsync(e->ptr, stream);
        e->ptr = p;
        e->bytes = want;
    }
    lease.ptr = e->ptr;
    return SEGRED_OK;
}

bool timing_on() { return g_timing.on; }

TimingEvents timing_events(bool streaming) {
    TimingEvents te;
    if (!g_timing.on || g_timing.used >= kMaxTimed) return te;
    const int slot = g_timing.used++;
    g_timing.streaming[slot] = streaming;
    te.start = g_timing.start[slot];
    te.stop = g_timing.stop[slot];
    return te;
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
    case SEGRED_ERR_SCRATCH_LIMIT: return "the call needs more than the fixed scratch of segred_reduce_noalloc";
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
        // no system-scope cache writeback at each stamp: it would slow the
        // kernels being timed (only this process reads the timestamps)
        for (int i = 0; i < kMaxTimed; ++i)
            if (hipEventCreateWithFlags(&g_timing.start[i], hipEventDisableSystemFence) != hipSuccess ||
                hipEventCreateWithFlags(&g_timing.stop[i], hipEventDisableSystemFence) != hipSuccess)
                return SEGRED_ERR_HIP;
        g_timing.created = true;
    }
    g_timing.on = enable != 0;
    g_timing.used = 0;
    return SEGRED_OK;
}

extern "C" int segred_timing_read(double *total_ms, int64_t *launches, float *each_ms, int64_t capacity) {
    if (!total_ms || !launches || capacity < 0 || (capacity > 0 && !each_ms)) return SEGRED_ERR_INVALID_ARGUMENT;
    double sum = 0.0;
    int64_t n = 0;
    for (int i = 0; i < g_timing.used; ++i) {
        if (!g_timing.streaming[i]) continue;
        if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess) return SEGRED_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]) != hipSuccess) return SEGRED_ERR_HIP;
        sum += ms;
        if (n < capacity) each_ms[n] = ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    g_timing.used = 0;
    return SEGRED_OK;
}
