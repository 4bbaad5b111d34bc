/*
 * segred_instrument.h -- testing and benchmarking hooks of the
 * segmented-reduction library.  They are not part of the method: the tests
 * use them to force segments across share boundaries and to check the share
 * count, the benchmark to time kernels and to measure the streaming rate the
 * device reaches.  The share and timing hooks are host-side and
 * process-wide; none of them is thread-safe.
 */
#ifndef SEGRED_INSTRUMENT_H
#define SEGRED_INSTRUMENT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Work partition of segred_reduce.  The rows and segment ends of a call are
 * split into equal shares of the merged (rows + segment ends) sequence, one
 * per wave of the streaming kernel; segments cut by a share boundary are
 * finished by a fixed-order combine.  For rows of 32 features read 16 bytes
 * per lane, a share size within 4 KB of rows of a multiple of 64 KB grows
 * to that distance (aligned waves would load from the same memory channels
 * together), and the last shares are then shorter or empty.  By default the share count is a
 * constant of the chosen kernel (one share per wave of a whole MI355X: 256
 * CUs x 4 SIMDs x the waves per SIMD the kernel is built for), so float
 * results do not depend on the device.  segred_set_shares(n) overrides it
 * for later calls (rounded up to a multiple of 4); 0 restores the default.
 * With an override the last bits of float sums change (integer, min/max and
 * row results do not), and for rows of 32 features read 16 bytes per lane
 * one share must not hold 4 GiB or more of rows.  Returns SEGRED_ERR_INVALID_ARGUMENT (1) unless
 * shares == 0 or 1 <= shares <= 2^22.
 */
int segred_set_shares(int64_t shares);

/* The share count segred_reduce uses for this dtype/op/feat (arrays aligned
 * to 16 bytes), or -1 for an invalid request. */
int64_t segred_get_shares(int32_t dtype, int32_t op, int64_t feat);

/* Waves of that call's streaming kernel that fit on the current device at
 * once (0 if the runtime cannot say); a default share count at or below it
 * runs in a single round of waves. */
int64_t segred_resident_waves(int32_t dtype, int32_t op, int64_t feat);

/*
 * Kernel timing.  While enabled, every kernel the library launches carries
 * a start and a stop HIP event that the runtime stamps when that kernel
 * begins and ends (hipExtLaunchKernel), so a launch's duration is its own
 * stop minus its own start and idle time between launches is not counted.
 * segred_timing_read waits for the recorded events and reports the
 * durations of the streaming kernels only (the first kernel of a
 * segred_reduce call, both kernels of segred_scan, the atomic or
 * private-copy kernel of segred_scatter_reduce, the search kernel of
 * segred_galloping_search, the histogram of segred_offsets_from_index, the
 * counting and materialising kernels of segred_offsets_from_rle /
 * segred_unique / segred_offsets_from_flags, and segred_probe_stream).  It
 * returns their summed duration in milliseconds and their number, writes the
 * first `capacity` durations (ms, in launch order) to the host array
 * `each_ms` (may be NULL when capacity is 0), and clears the record.  Up to
 * 8192 launches (streaming or not) are kept; later ones are not timed.
 */
int segred_timing_enable(int enable);
int segred_timing_read(double *total_ms, int64_t *launches, float *each_ms, int64_t capacity);

/*
 * Streaming-rate probe, for measurement context only (it is not part of the
 * method): the rate a plain read of device memory reaches, alone or with a
 * fixed fraction of writes, i.e. the practical ceiling of a kernel that
 * reads its input once and writes a fraction of it.  `src` (device, 16-byte
 * aligned) holds `bytes` bytes of float32, a positive multiple of 1,024.  It
 * is cut into `waves` contiguous shares of whole 1 KB blocks (1 <= waves <=
 * 2^20, each share under 2 GiB), one wave per share, 4 waves per workgroup;
 * each wave reads its share with non-temporal 16-byte loads and keeps a
 * running float sum per lane.  With write_every = 0 nothing else is written;
 * with 1 <= write_every <= 1024, after every input block b with
 * (b + 1) % write_every == 0 the wave writes its 64 lanes' running sums (each
 * as 4 equal floats, non-temporal) to the 1 KB block b / write_every of `dst`
 * (device, 16-byte aligned, at least floor(bytes / 1024 / write_every) KiB),
 * so the writes are 1/write_every of the reads.  `wave_sums` (device, `waves`
 * floats) receives each wave's total.  Asynchronous on `stream`; timed like
 * the streaming kernels above.  Returns SEGRED_ERR_INVALID_ARGUMENT for
 * arguments outside these ranges, SEGRED_ERR_HIP if the launch fails.
 */
int segred_probe_stream(const void *src, int64_t bytes, void *dst, int32_t write_every, float *wave_sums,
                        int32_t waves, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEGRED_INSTRUMENT_H */
