// probe.hip -- streaming-rate probe: the rate a plain wave-per-share read of
// device memory reaches on this GPU, alone or with a fixed fraction of writes.
// It is measurement context, not part of the method: the reduction kernels
// read their input once and write a fraction of it, so this probe's rate is
// the practical ceiling they are compared with (beside the HBM3E peak).
#include "internal.hpp"
#include "wave.hpp"

namespace segred {
namespace {

constexpr int kProbeThreads = 256;  // 4 waves per workgroup, one share each
constexpr int kProbeUnroll = 8;     // 1 KB blocks in flight per wave
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Wave w reads blocks [nblk*w/waves, nblk*(w+1)/waves) of 1 KB (64 lanes x
// 16 bytes, non-temporal) and keeps a per-lane running sum of the floats it
// has read.  With wevery > 0, after each input block b with (b + 1) %
// wevery == 0 the wave writes its lanes' running sums (as float4, one 1 KB
// block, non-temporal) to output block b / wevery, so the writes are
// 1/wevery of the reads and form 1 KB bursts.  The wave's total goes to
// wave_sums[w] so that no load is dead.
__global__ __launch_bounds__(kProbeThreads) void stream_probe(const uint4 *__restrict__ src, int64_t nblk,
                                                             f32x4 *__restrict__ dst, int32_t wevery,
                                                             float *__restrict__ wave_sums, int32_t waves) {
    const int lane = lane_id();
    // the wave's index, made scalar so that the descriptor lives in SGPRs
    const int w = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)));
    if (w >= waves) return;
    const int64_t jb = nblk * w / waves, je = nblk * (w + 1) / waves;
    // the host keeps a share under 2 GiB, so every lane offset below fits
    const auto r = make_rsrc(src + jb * 64, (uint32_t)((je - jb) * 1024));
    int64_t wnext = wevery > 0 ? (jb / wevery + 1) * wevery - 1 : INT64_MAX;  // next block followed by a write
    // the wave's output blocks start at the first block it writes
    const int64_t ob0 = wevery > 0 ? jb / wevery : 0;
    const auto wr = make_rsrc(dst + ob0 * 64, wevery > 0 ? (uint32_t)(((je - jb) / wevery + 1) * 1024) : 0u);
    uint32_t woff = lane * 16;  // lane offset of the next output block
    // software-pipelined: the loads of the next kProbeUnroll blocks are in
    // flight while the current ones are summed (past the share's end the
    // loads return zeros without a memory access)
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = ld128(r, (uint32_t)(u * 1024 + lane * 16));
    float acc = 0.f;
    for (int64_t j = jb; j < je; j += kProbeUnroll) {
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const uint4 x = v[u];
            v[u] = ld128(r, (uint32_t)((j - jb + kProbeUnroll + u) * 1024 + lane * 16));
            acc += __uint_as_float(x.x) + __uint_as_float(x.y) + __uint_as_float(x.z) + __uint_as_float(x.w);
            if (j + u == wnext && j + u < je) {
                __builtin_amdgcn_raw_buffer_store_b128(f32x4{acc, acc, acc, acc}, wr, (int)woff, 0, kStreamPolicy);
                wnext += wevery;
                woff += 1024;
            }
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) wave_sums[w] = acc;
}

}  // namespace
}  // namespace segred

using namespace segred;

extern "C" int segred_probe_stream(const void *src, int64_t bytes, void *dst, int32_t write_every,
                                   float *wave_sums, int32_t waves, hipStream_t stream) {
    if (!src || !wave_sums || bytes <= 0 || bytes % 1024 != 0 || waves < 1 || waves > (1 << 20) ||
        write_every < 0 || write_every > 1024 || (write_every > 0 && !dst) || !aligned(src, 16) ||
        (dst && !aligned(dst, 16)) || !aligned(wave_sums, 4))
        return SEGRED_ERR_INVALID_ARGUMENT;
    const int64_t nblk = bytes / 1024;
    if ((nblk + waves - 1) / waves >= (int64_t(1) << 21)) return SEGRED_ERR_INVALID_ARGUMENT;  // share < 2 GiB
    timed_launch_ggl(true, stream_probe, dim3((unsigned)((waves + 3) / 4)), dim3(kProbeThreads), 0, stream,
                     (const uint4 *)src, nblk, (f32x4 *)dst, write_every, wave_sums, waves);
    return hipGetLastError() == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}
