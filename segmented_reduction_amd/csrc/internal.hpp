// internal.hpp -- host-side plumbing shared by the library's translation
// units: scratch pool, launch timing, the share-count knob.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "segred.h"

namespace segred {

// Stream-ordered scratch from a per-device pool that keeps its memory
// (release threshold = max), so steady-state calls do not hit the driver.
int scratch_alloc(void **ptr, size_t bytes, hipStream_t stream);
void scratch_free(void *ptr, hipStream_t stream);

// Launch timing around the streaming kernel (segred_timing_enable).
bool timing_on();
int timing_begin(hipStream_t stream);  // returns a slot id or -1
void timing_end(int slot, hipStream_t stream);

// Process-wide share override (0 = default).
int64_t shares_override();

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace segred
