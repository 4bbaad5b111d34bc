/*
 * segred_instrument.h -- testing and benchmarking hooks of the
 * segmented-reduction library.  They are not part of the method: the tests
 * use them to force segments across share boundaries and to check the share
 * count, the benchmark to time kernels.  All of them are host-side and
 * process-wide; none is thread-safe.
 */
#ifndef SEGRED_INSTRUMENT_H
#define SEGRED_INSTRUMENT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Work partition of segred_reduce.  The rows and segment ends of a call are
 * split into equal shares of the merged (rows + segment ends) sequence, one
 * per wave of the streaming kernel; segments cut by a share boundary are
 * finished by a fixed-order combine.  By default the share count is a
 * constant of the chosen kernel (one share per wave of a whole MI355X: 256
 * CUs x 4 SIMDs x the waves per SIMD the kernel is built for), so float
 * results do not depend on the device.  segred_set_shares(n) overrides it
 * for later calls (rounded up to a multiple of 4); 0 restores the default.
 * With an override the last bits of float sums change (integer, min/max and
 * row results do not), and for rows of at most 128 bytes one share must not
 * hold 4 GiB or more of rows.  Returns SEGRED_ERR_INVALID_ARGUMENT (1) unless
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
 * a HIP event that the runtime stamps when that kernel ends
 * (hipExtLaunchKernel).  segred_timing_read waits for the recorded events and
 * reports, for every streaming kernel (the first kernel of a segred_reduce
 * call, both kernels of segred_scan, the atomic or private-copy kernel of
 * segred_scatter_reduce, the search kernel of segred_galloping_search, the
 * histogram of segred_offsets_from_index, the counting and materialising
 * kernels of segred_offsets_from_rle / segred_unique /
 * segred_offsets_from_flags), the time from the end of the launch recorded
 * before it to its own end (-1 for the first launch of the record): when the
 * library's kernels run back to back on one stream (nothing else queued in
 * between), this is the streaming kernel's execution time.  It returns the
 * summed duration of the timed launches in milliseconds and the number of
 * streaming launches, writes the first `capacity` durations (ms, in launch
 * order) to the host array `each_ms` (may be NULL when capacity is 0), and
 * clears the record.  Up to 8192 launches are kept; later ones are not timed.
 */
int segred_timing_enable(int enable);
int segred_timing_read(double *total_ms, int64_t *launches, float *each_ms, int64_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* SEGRED_INSTRUMENT_H */
