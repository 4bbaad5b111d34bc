// internal.hpp -- host-side plumbing shared by the library's translation
// units: scratch pool, launch timing, the share-count knob.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <mutex>

#include "segred.h"
#include "segred_instrument.h"

namespace segred {

// Scratch for one call, owned by the library.  Each (device, stream) pair
// keeps one cached buffer that later calls on the same stream reuse: calls
// on one stream run in order, so the reuse is safe, and a cached call costs
// neither an allocation nor a free (each stream-ordered pool operation adds
// tens of microseconds of host time and an idle gap on the GPU).  The buffer
// grows stream-ordered on demand.  Requests above kScratchCacheBytes, or
// beyond kScratchCacheEntries streams per process, take a stream-ordered
// allocation from a per-device pool that keeps its memory (release
// threshold = max) and free it after the call.  The lease holds the
// entry's lock until it is destroyed, after the call's launches are queued,
// so two host threads sharing a stream cannot swap the buffer under each
// other.  Entries are keyed by the stream handle: a stream must have no call
// in flight when it is destroyed, or a new stream that receives the same
// handle could reuse the buffer while the old calls still run.
constexpr size_t kScratchCacheBytes = size_t(256) << 20;
constexpr int kScratchCacheEntries = 64;

struct ScratchLease {
    void *ptr = nullptr;
    ScratchLease() = default;
    ScratchLease(const ScratchLease &) = delete;
    ScratchLease &operator=(const ScratchLease &) = delete;
    ~ScratchLease();

    void *owned_ = nullptr;  // per-call pool allocation, freed on `stream_`
    hipStream_t stream_ = nullptr;
    std::unique_lock<std::mutex> lock_;
};
int scratch_acquire(ScratchLease &lease, size_t bytes, hipStream_t stream);

// Launch timing (segred_timing_enable): while it is on, every kernel the
// library launches carries a start and a stop event that the runtime stamps
// when that kernel begins and ends (hipExtLaunchKernel); otherwise both are
// null.  A streaming kernel's duration is its own stop minus its own start,
// so idle time between launches is not counted.
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
bool timing_on();
TimingEvents timing_events(bool streaming);

// Kernel launches with the timing events of the record.
inline hipError_t timed_launch(bool streaming, const void *kernel, dim3 grid, dim3 block, void **params,
                               size_t lds, hipStream_t st) {
    const TimingEvents te = timing_events(streaming);
    return hipExtLaunchKernel(kernel, grid, block, params, lds, st, te.start, te.stop, 0);
}
template <typename F, typename... Args>
inline void timed_launch_ggl(bool streaming, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                             Args... args) {
    const TimingEvents te = timing_events(streaming);
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, te.start, te.stop, 0, args...);
}

// Process-wide share override (0 = default).
int64_t shares_override();

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace segred
