// scan.hpp -- workgroup-wide inclusive scan of one int64 per thread.
#pragma once

#include "wave.hpp"

namespace segred {

// Inclusive scan over the kThreads threads of a workgroup; the operation is
// + or (MIN) minimum.  s_tmp holds 2 * kThreads / 64 entries; on return
// s_tmp[kThreads / 64 + w] is the inclusive result of wave w's last lane, and
// `total` that of the whole workgroup.  Every thread must call it.
template <int kThreads, bool MIN>
__device__ __forceinline__ int64_t block_inclusive_scan(int64_t v, int64_t *s_tmp, int64_t &total) {
    static_assert(kThreads % 64 == 0 && kThreads <= 4096, "whole waves, at most 64 of them");
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    constexpr int kWaves = kThreads / 64;
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = lane_get(x, (lane - o) & 63);
        if (lane >= o) x = MIN ? (y < x ? y : x) : x + y;
    }
    if (lane == 63) s_tmp[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int64_t w = lane < kWaves ? s_tmp[lane] : (MIN ? INT64_MAX : 0);
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            const int64_t y = lane_get(w, (lane - o) & 63);
            if (lane >= o) w = MIN ? (y < w ? y : w) : w + y;
        }
        if (lane < kWaves) s_tmp[kWaves + lane] = w;
    }
    __syncthreads();
    if (wid > 0) {
        const int64_t p = s_tmp[kWaves + wid - 1];
        x = MIN ? (p < x ? p : x) : p + x;
    }
    total = s_tmp[2 * kWaves - 1];
    __syncthreads();
    return x;
}

}  // namespace segred
