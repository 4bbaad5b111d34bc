/*
 * segred.h -- C ABI of the segmented-reduction library for AMD Instinct
 * MI355X (gfx950).
 *
 * Every pointer argument is a DEVICE pointer unless stated otherwise.  Every
 * call is asynchronous and ordered on the HIP stream it is given (0 is the
 * null stream): a non-error return means the work was enqueued; faults during
 * the work surface at the caller's next synchronisation.  Inputs and outputs
 * are owned by the caller; scratch memory is owned by the library: each
 * (device, stream) keeps one cached scratch buffer of up to 256 MiB that
 * later calls on that stream reuse (larger needs, and streams past the 64th,
 * take a stream-ordered pool allocation freed on the same stream).  The
 * cached buffers are held until the process ends.  No call throws.  Calls on
 * distinct streams may run concurrently.  A stream must have no call of this
 * library in flight when it is destroyed (synchronise it first).
 */
#ifndef SEGRED_H
#define SEGRED_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of `values` (4-byte packed scalars). */
enum segred_dtype { SEGRED_U32 = 0, SEGRED_I32 = 1, SEGRED_F32 = 2 };

/* Reductions.  MEAN is float32 only. */
enum segred_op { SEGRED_SUM = 0, SEGRED_MIN = 1, SEGRED_MAX = 2, SEGRED_MEAN = 3 };

/* Return codes. */
enum segred_status {
    SEGRED_OK = 0,
    SEGRED_ERR_INVALID_ARGUMENT = 1, /* rejected on the host before any device work */
    SEGRED_ERR_UNSUPPORTED = 2,      /* a valid request this library does not do (integer MEAN) */
    SEGRED_ERR_OUT_OF_MEMORY = 3,    /* scratch could not be obtained */
    SEGRED_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
    SEGRED_ERR_SCRATCH_LIMIT = 5     /* segred_reduce_noalloc: the call needs more than its fixed scratch */
};

/*
 * segred_reduce -- segmented reduction over offset-delimited segments.
 *
 * Defined by the luma.gl "GPUSegmentedReduction" page (sections "What is an
 * offset-delimited segment?", "What is segmented reduction?", "Contract") and
 * the graph-reduce README ("API": mean and the producing row of min/max;
 * "Method": ties go to the lower row; "Correctness": the row is an index into
 * the source, an empty min/max has row -1).
 *
 *   values        [rows, feat] row-major, 4-byte elements of type `dtype`.
 *                 Rows are absolute: segment s covers rows
 *                 offsets[s] .. offsets[s+1]-1.  Only rows inside
 *                 [offsets[0], offsets[num_segments]) are read.
 *   dtype         SEGRED_U32, SEGRED_I32 or SEGRED_F32.
 *   feat          features per row, >= 1 (each reduced independently).
 *   offsets       int64 [num_segments + 1], nondecreasing.  offsets[0] may be
 *                 above 0.  A repeated offset is an empty segment.
 *   num_segments  S >= 0.  S = 0 enqueues nothing and returns SEGRED_OK.
 *   op            SEGRED_SUM, SEGRED_MIN, SEGRED_MAX or SEGRED_MEAN.
 *   out           [S, feat] of the input type (float32 for MEAN).
 *                 SUM of u32/i32 wraps modulo 2^32.  SUM and MEAN of f32 are
 *                 accumulated in an order fixed by the offsets alone (the
 *                 work partition is a constant of the library, not of the
 *                 device), so results are bitwise identical from run to run
 *                 and from device to device: in float64 and rounded to
 *                 float32 once, except that 1-D inputs (feat = 1) add runs
 *                 of at most 32 consecutive elements and a 64-way tree of
 *                 such runs in float32 first (error below
 *                 38 * 2^-24 * sum|x| in all).  MIN/MAX order u32 unsigned, i32 signed,
 *                 f32 by the monotone bit key (so -0.0 < +0.0 and NaNs sort
 *                 past +-inf by their bits); `out` holds the element's bits.
 *                 An empty segment writes 0 (+0.0 for floats).
 *   arg_out       int64 [S, feat] or NULL.  MIN/MAX only (ignored otherwise):
 *                 the absolute row of the extremum, the lowest such row on
 *                 ties, -1 for an empty segment.
 *   stream        HIP stream the work is ordered on.
 *
 * Rows whose width is a multiple of 4 features are read and written 16
 * bytes per lane when values, out and arg_out start on 16-byte boundaries,
 * other even widths 8 bytes per lane under the same condition, other rows
 * one element per lane; rows of fewer than 32 features (and of 32 features
 * not on 16-byte boundaries) are fetched in whole 1 KB stretches and reach
 * the lanes through LDS.  Results are the same either way.
 *
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for S < 0, feat < 1, an unknown dtype
 * or op, a NULL values/offsets/out with S > 0, values/out not 4-byte aligned,
 * offsets/arg_out not 8-byte aligned.  SEGRED_ERR_UNSUPPORTED for MEAN of an
 * integer type or for feat > 2^24 (rows are addressed with 32-bit offsets
 * inside a chunk).  SEGRED_ERR_OUT_OF_MEMORY if scratch is unavailable.
 * SEGRED_ERR_HIP if a launch fails.  The offsets are NOT read back or checked:
 * offsets that decrease or point outside `values` are undefined behaviour, as
 * is `out`/`arg_out` overlapping the inputs.  The device never needs the row
 * count: N = offsets[S] - offsets[0] stays on the device.
 */
int segred_reduce(const void *values, int32_t dtype, int64_t feat,
                  const int64_t *offsets, int64_t num_segments, int32_t op,
                  void *out, int64_t *arg_out, hipStream_t stream);

/*
 * segred_reduce_noalloc -- segred_reduce for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): it calls no hipMalloc, hipFree or other
 * allocating routine.  Its scratch is a fixed array of 16 MiB in device
 * memory that the library holds on each device it runs on until the process
 * ends (its address is looked up once per device, on the first call there).
 *
 *   Arguments, results and errors: as segred_reduce, plus
 *   SEGRED_ERR_SCRATCH_LIMIT when the call needs more than the fixed
 *   scratch: 32 * NS + 16 * NS * feat bytes, NS = the call's share count
 *   (4,096 for rows of 32 features read 16 bytes per lane, 2,048 for all
 *   other rows and 1-D values), i.e. feat up to 510.  Results are bitwise equal to
 *   segred_reduce's (same kernels, same shares).
 *
 * All calls on one device share that device's array: calls that overlap in
 * time on one device (on different streams, or from different host threads)
 * race on it and must not be issued; calls on one stream run in order and
 * are safe.  Nothing in the array needs clearing between calls (every
 * header is written before it is read).
 */
int segred_reduce_noalloc(const void *values, int32_t dtype, int64_t feat,
                          const int64_t *offsets, int64_t num_segments, int32_t op,
                          void *out, int64_t *arg_out, hipStream_t stream);

/*
 * segred_offsets_from_rle -- run-length encoding of uint32 keys and the
 * offsets of the runs, the producer that feeds segred_reduce.
 *
 * Defined by the luma.gl "GPURunLengthEncode and GPUUnique" page (sections
 * "What is run-length encoding?", "Why RLE matters for GPU grouping",
 * "Contract"): adjacent equal keys form a run; runs keep first-occurrence
 * order; keys are compared bit for bit and need not be sorted (sorting first
 * makes equal keys adjacent); run lengths [3,2,4] correspond to offsets
 * [0,3,5,9]; an empty input gives count 0.
 *
 *   sorted_keys  uint32 [n].
 *   n            0 <= n <= UINT32_MAX.
 *   values       uint32, capacity n: values[r] = key of run r.
 *   lengths      uint32, capacity n: lengths[r] = length of run r.
 *   offsets      int64, capacity n + 1: offsets[r] = first position of run r,
 *                offsets[count] = n.
 *   count        one int64 on the device: the number of runs.
 *   stream       HIP stream the work is ordered on.
 *
 * Only values[0..count), lengths[0..count) and offsets[0..count] are written;
 * the rest of each buffer is left untouched.  To reduce over the runs, read
 * `count` back (8 bytes) and pass it as num_segments with `offsets`, or pass
 * `count` itself to segred_reduce_device_count (no readback).
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for n < 0, n > UINT32_MAX, a NULL
 * output (or NULL keys with n > 0), misalignment (4 bytes for keys, values,
 * lengths; 8 bytes for offsets and count).  SEGRED_ERR_OUT_OF_MEMORY,
 * SEGRED_ERR_HIP as for segred_reduce.
 */
int segred_offsets_from_rle(const uint32_t *sorted_keys, int64_t n,
                            uint32_t *values, uint32_t *lengths,
                            int64_t *offsets, int64_t *count, hipStream_t stream);

/*
 * segred_unique -- the distinct adjacent values of uint32 keys.
 *
 * Defined by the luma.gl "GPURunLengthEncode and GPUUnique" page, section
 * "GPUUnique": the same equality (bit for bit) and first-occurrence order as
 * segred_offsets_from_rle, i.e. its `values` and `count`, without run
 * lengths; [2,2,5,2] gives [2,5,2] (adjacency, not global uniqueness).
 *
 *   keys    uint32 [n], any order.
 *   n       0 <= n <= 2^40.
 *   values  uint32, capacity n: values[r] = key of run r.
 *   count   one int64 on the device: the number of runs.
 *   stream  HIP stream the work is ordered on.
 *
 * Only values[0..count) is written.  Errors: SEGRED_ERR_INVALID_ARGUMENT for
 * n out of range, a NULL values/count (or keys with n > 0), misalignment
 * (4 bytes for keys and values, 8 for count).  SEGRED_ERR_OUT_OF_MEMORY,
 * SEGRED_ERR_HIP as for segred_reduce.
 */
int segred_unique(const uint32_t *keys, int64_t n, uint32_t *values, int64_t *count,
                  hipStream_t stream);

/*
 * segred_offsets_from_flags -- segment offsets from segment-start flags.
 *
 * Defined by the luma.gl "GPUSegmentedReduction" page, section
 * "Composition" (a segmented layout materialises offsets from segment-start
 * flags) with the offsets contract of the same page ("What is an
 * offset-delimited segment?": N segments take N + 1 offsets, the last one
 * closes the last segment).  Position i starts a segment iff flags[i] != 0.
 *
 *   flags    uint32 [n]; any nonzero word marks a start.
 *   n        0 <= n <= 2^40.
 *   offsets  int64, capacity n + 1: offsets[0..count) = the flagged
 *            positions in increasing order, offsets[count] = n.  Positions
 *            before the first flag belong to no segment (offsets[0] > 0 is
 *            allowed by segred_reduce); no flag at all gives count 0 and
 *            offsets[0] = n.
 *   count    one int64 on the device: the number of segments.
 *   stream   HIP stream the work is ordered on.
 *
 * Only offsets[0..count] is written.  The result feeds segred_reduce (read
 * `count` back) or segred_reduce_device_count (no readback).  Errors:
 * SEGRED_ERR_INVALID_ARGUMENT for n out of range, a NULL offsets/count (or
 * flags with n > 0), misalignment (4 bytes for flags, 8 for offsets and
 * count).  SEGRED_ERR_OUT_OF_MEMORY, SEGRED_ERR_HIP as for segred_reduce.
 */
int segred_offsets_from_flags(const uint32_t *flags, int64_t n, int64_t *offsets, int64_t *count,
                              hipStream_t stream);

/*
 * segred_reduce_device_count -- segred_reduce with the segment count read on
 * the device, for the sort -> RLE -> offsets -> reduce composition that the
 * "GPURunLengthEncode and GPUUnique" page draws ("Composition": run lengths
 * become offsets that feed the segmented reduction) without reading the run
 * count back to the host.
 *
 *   num_segments  one int64 on the device (e.g. the `count` written by
 *                 segred_offsets_from_rle), read when the call runs; the
 *                 call reduces S = min(max(*num_segments, 0), max_segments)
 *                 segments.
 *   max_segments  host bound >= 0: `offsets` must hold max_segments + 1
 *                 entries and `out`/`arg_out` max_segments * feat; rows of
 *                 `out`/`arg_out` at or past S are left untouched.
 *   all other arguments and every error: as segred_reduce (plus
 *   SEGRED_ERR_INVALID_ARGUMENT for a NULL or misaligned num_segments).
 *   Only offsets[0..S] are read.
 */
int segred_reduce_device_count(const void *values, int32_t dtype, int64_t feat,
                               const int64_t *offsets, const int64_t *num_segments,
                               int64_t max_segments, int32_t op, void *out,
                               int64_t *arg_out, hipStream_t stream);

/*
 * segred_scatter_reduce -- reduction of rows into the outputs an index names
 * (the scatter form: the index need not be sorted).
 *
 * Defined by the graph-reduce README: "API" (scatter_sum / scatter_mean /
 * scatter_max / scatter_min over src [N, ...] with an int64 index [N] and
 * dim_size outputs; the mean of an output no row reaches is 0; max and min
 * also return the producing row), "Method" (one atomic operation per element;
 * max/min resolve value and row together in one 64-bit atomic on the word
 * (order key << 32) | row code, ties to the lower row).
 *
 *   values     [rows, feat] row-major, 4-byte elements of type `dtype`.
 *   dtype      SEGRED_U32, SEGRED_I32 or SEGRED_F32.
 *   feat       features per row, >= 1.
 *   rows       N >= 0.
 *   index      int64 [rows]: index[r] is the output row r goes to.  Rows whose
 *              index is outside [0, dim_size) take part in no output.
 *   dim_size   number of outputs >= 0 (0: nothing is written).
 *   op         SEGRED_SUM, SEGRED_MIN, SEGRED_MAX or SEGRED_MEAN.
 *   out        [dim_size, feat] of the input type (float32 for MEAN); every
 *              element is written.  An output no row reaches gets 0.
 *              Integer SUM wraps modulo 2^32 and is exact; MIN/MAX use the
 *              same order as segred_reduce and are exact.  Float SUM and MEAN
 *              are float32 additions (error at most (n - 1) * 2^-24 *
 *              sum|x| for an output of n rows, to first order, in any order;
 *              MEAN adds one rounding of the division).  They add in arrival
 *              order, so the last bits can differ from run to run, except on
 *              the few-output path with feat >= 8 (below), which adds in a
 *              fixed order.  Use segred_reduce on destination-sorted rows for
 *              a reproducible sum in every case.
 *   arg_out    int64 [dim_size, feat] or NULL; MIN/MAX only: the row that
 *              produced the value, the lowest such row on ties, -1 for an
 *              output no row reaches.  When given, it also serves as the
 *              call's working memory for the packed words.
 *   stream     HIP stream the work is ordered on.
 *
 * Paths: with many outputs, one global atomic per element (as in "Method").
 * When one copy of the outputs fits 32 KB (4 or 8 bytes per cell, plus 4 per
 * output for MEAN) and there are at least 128 rows x features per cell,
 * each workgroup reduces its rows into a private copy in LDS and the copies
 * are folded in a fixed order; float SUM/MEAN with feat >= 8 take this path
 * only when one copy per wave fits (4 copies).  That path keeps up to one
 * 32 KB copy per resident workgroup in the stream's scratch (tens of MB).
 *
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for rows < 0, dim_size < 0, feat < 1,
 * an unknown dtype or op, a NULL values/index with rows > 0 or out with
 * dim_size > 0, values/out not 4-byte or index/arg_out not 8-byte aligned,
 * dim_size * feat or rows * feat above INT64_MAX.  SEGRED_ERR_UNSUPPORTED for
 * MEAN of an integer type, or MIN/MAX/MEAN with rows > 2^32 - 2 (rows are
 * packed into 32 bits).  SEGRED_ERR_OUT_OF_MEMORY, SEGRED_ERR_HIP as for
 * segred_reduce.  `out`/`arg_out` must not overlap the inputs.
 */
int segred_scatter_reduce(const void *values, int32_t dtype, int64_t feat, int64_t rows,
                          const int64_t *index, int64_t dim_size, int32_t op,
                          void *out, int64_t *arg_out, hipStream_t stream);

/*
 * segred_offsets_from_index -- the CSR offsets of an index: offsets[s] = the
 * number of rows whose index lies in [0, s), for s = 0..dim_size.
 *
 * Defined by the graph-reduce README, "Usage": for an edge list sorted by
 * destination, the pointer that segment_*_csr takes is the per-destination
 * count of the index with a running sum behind a leading 0.  For a sorted
 * index, segment s of segred_reduce(values, ..., offsets, dim_size, ...) then
 * holds exactly the rows with index s.
 *
 *   index     int64 [rows], any order; entries outside [0, dim_size) are not
 *             counted.
 *   rows      >= 0.
 *   dim_size  >= 0.
 *   offsets   int64 [dim_size + 1], every entry written (offsets[0] = 0).
 *   stream    HIP stream the work is ordered on.
 *
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for rows < 0, dim_size < 0, a NULL
 * offsets (or index with rows > 0), misalignment (8 bytes).
 * SEGRED_ERR_UNSUPPORTED above 2^31 workgroups (rows > 2^44 or dim_size >
 * 2^43).  SEGRED_ERR_OUT_OF_MEMORY, SEGRED_ERR_HIP as for segred_reduce.
 */
int segred_offsets_from_index(const int64_t *index, int64_t rows, int64_t dim_size,
                              int64_t *offsets, hipStream_t stream);

/*
 * segred_scan -- segmented inclusive or exclusive scan over offset-delimited
 * segments.
 *
 * GPUSegmentedScan is named by the luma.gl "GPURunLengthEncode and
 * GPUUnique" page ("Composition", beside GPUSegmentedReduction); it is read
 * with the segmented reduction's contract ("GPUSegmentedReduction" page:
 * segments, dtypes, operations, empty -> 0): for row r of segment s,
 *   inclusive (exclusive = 0): out[r] = op of values[offsets[s] .. r]
 *   exclusive (exclusive != 0): out[r] = op of values[offsets[s] .. r-1],
 *                               0 at the first row of each segment.
 *
 *   values        [rows, feat] row-major, 4-byte elements of type `dtype`.
 *   dtype         SEGRED_U32, SEGRED_I32 or SEGRED_F32.
 *   feat          features per row, 1 <= feat <= 2^24 (each scanned on its own).
 *   offsets       int64 [num_segments + 1], nondecreasing (offsets[0] may be > 0).
 *   num_segments  S >= 0 (0: nothing is written).
 *   op            SEGRED_SUM, SEGRED_MIN or SEGRED_MAX.
 *   out           [rows, feat] in the layout of `values` and of its type; only
 *                 rows in [offsets[0], offsets[S]) are written.  Integer sums
 *                 wrap modulo 2^32; float sums accumulate in float64 and each
 *                 output is its prefix rounded to float32 once (results
 *                 repeat bit for bit); min/max order as in segred_reduce.
 *   stream        HIP stream the work is ordered on.
 *
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for S < 0, feat < 1, an unknown dtype
 * or op, NULL values/offsets/out with S > 0, misalignment (4 bytes for values
 * and out, 8 for offsets).  SEGRED_ERR_UNSUPPORTED for SEGRED_MEAN or feat
 * above 2^24.  SEGRED_ERR_OUT_OF_MEMORY, SEGRED_ERR_HIP as for segred_reduce.
 * The offsets are not validated (as for segred_reduce); `out` must not
 * overlap `values` or `offsets`.
 */
int segred_scan(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                int64_t num_segments, int32_t op, int32_t exclusive, void *out,
                hipStream_t stream);

/*
 * segred_galloping_search -- many lower-bound queries over segmented sorted
 * values.
 *
 * Defined by the luma.gl "GPUGallopingSearch" page ("Overview", "Usage",
 * "Validation", "Cost model"): segment record s = (vo, vc, qo, qc) names
 * value positions [vo, vo + vc) and query positions [qo, qo + qc);
 * out[qo + k] = the first position p in [vo, vo + vc) whose value is not
 * less than query k, or vo + vc when there is none -- an absolute position
 * in the value view, or in the order view when `value_order` is given.
 * Queries are processed in tiles of `queries_per_tile` per segment; each
 * tile seeds with a full search and gallops from answer to answer.
 *
 *   values           device array; value i is values[i * value_stride]
 *                    (a strided column), i < value_count.  SEGRED_U32
 *                    (unsigned order) or SEGRED_F32 (IEEE order); each value
 *                    segment must be sorted ascending (caller's invariant).
 *   value_order      uint32 [order_count] or NULL: search position p means
 *                    value row value_order[p] (every entry < value_count,
 *                    the caller's invariant; an entry past it reads as a
 *                    value above every query, without a fault).
 *   queries          [query_count] of the values' type; ascending inside a
 *                    tile for the fast path.
 *   segments         int64 [num_segments][4] records (vo, vc, qo, qc), read
 *                    on the device.
 *   max_query_count  per-segment query capacity the launch covers.
 *   queries_per_tile T >= 1 (the page's default is 32).
 *   out              int64 [query_count]; positions not answered (see
 *                    validation) keep their contents.
 *   validation       one uint32 on the device, cleared first unless
 *                    preserve_validation is nonzero, then OR-ed with:
 *                    1 a value range leaves its view (segment skipped),
 *                    2 a query range leaves the query view or qc exceeds
 *                      max_query_count (segment skipped),
 *                    4 a query is below its predecessor in its tile (it is
 *                      answered by a full search: still exact),
 *                    8 a float32 query is not finite (it and the rest of
 *                      its tile are not written).
 *   stream           HIP stream the work is ordered on.
 *
 * Errors: SEGRED_ERR_INVALID_ARGUMENT for an unknown dtype, negative counts,
 * value_stride < 1, queries_per_tile < 1, NULL or misaligned arrays that are
 * needed (4 bytes for values, order, queries and validation; 8 for segments
 * and out).  SEGRED_ERR_UNSUPPORTED for SEGRED_I32 (the page searches
 * float32 or uint32) or more than 2^31 workgroups.  SEGRED_ERR_HIP if a
 * launch fails.
 */
int segred_galloping_search(const void *values, int32_t dtype, int64_t value_count, int64_t value_stride,
                            const uint32_t *value_order, int64_t order_count,
                            const void *queries, int64_t query_count,
                            const int64_t *segments, int64_t num_segments, int64_t max_query_count,
                            int32_t queries_per_tile, int64_t *out, uint32_t *validation,
                            int32_t preserve_validation, hipStream_t stream);

/* Static, host-side description of a status code (never NULL). */
const char *segred_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SEGRED_H */
