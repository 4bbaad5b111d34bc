/*
 * oracle.c -- the plain, slow CPU oracle for segmented reduction over
 * offset-delimited segments, for the run-length encoding that produces such
 * segments, and for the index-addressed (scatter) form of the same reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this code.  The HIP
 * library never links, loads or calls it, and the two share no code, header,
 * table or helper.
 *
 * Everything here is the plain definition written out, one segment and one
 * feature at a time, rows in ascending order, in one thread:
 *
 *   - luma.gl "GPUSegmentedReduction", sections "What is an offset-delimited
 *     segment?" and "Contract": segment s owns rows [offsets[s], offsets[s+1]);
 *     S segments take S+1 offsets; a repeated offset is an empty segment; the
 *     offsets need not start at 0 (output row i reduces input[o_i..o_{i+1})).
 *   - same page, "What is segmented reduction?" and "Contract": one sum,
 *     minimum or maximum per segment over uint32, sint32 or float32 values;
 *     an empty segment produces zero.
 *   - phanerozoic/graph-reduce README, "API": mean is sum divided by the
 *     segment length, empty outputs are 0; min and max also return the row
 *     that produced them; the input is [N, ...] reduced over dimension 0.
 *   - same README, "Method" and "Correctness": floats are ordered through a
 *     monotone map of their bit pattern to an integer; ties go to the lower
 *     row; an empty min/max segment has arg -1.
 *   - luma.gl "GPURunLengthEncode and GPUUnique", sections "What is run-length
 *     encoding?", "Why RLE matters for GPU grouping" and "Contract": each
 *     adjacent run of equal uint32 values becomes (value, length), first
 *     occurrence order is kept, lengths [3,2,4] correspond to offsets
 *     [0,3,5,9], an empty input gives count 0; "GPUUnique": the distinct
 *     adjacent values under the same equality, without lengths.
 *   - luma.gl "GPUSegmentedReduction", "Composition": a segmented layout
 *     materialises offsets from segment-start flags.
 *   - luma.gl RLE page, "Composition": GPUSegmentedScan beside the
 *     segmented reduction (read as the per-row prefix of the same operation).
 *   - luma.gl "GPUGallopingSearch": lower bounds of queries over segmented
 *     sorted values, with its validation word.
 *   - phanerozoic/graph-reduce README, "API" and "Method": the scatter path
 *     reduces every row into the output its index names (the index need not
 *     be sorted), with the same sum / mean / min / max (+ row) semantics;
 *     "Usage": the CSR pointer of a destination-sorted edge list is a
 *     bincount of the index followed by a cumulative sum with a leading 0.
 *
 * Readings where the pages leave a step open (each one is also listed in the
 * design notes of the repository):
 *   - integer sums wrap modulo 2^32 (the pages are silent on overflow);
 *   - floating-point sums are accumulated in double precision in row order and
 *     rounded to float32 once; the double sum and the sum of magnitudes are
 *     returned as well, for the tolerance |gpu - ref| <= 1e-5 * sum|x| + 1e-6;
 *   - the order used by min/max is the monotone key below for every dtype, so
 *     -0.0 < +0.0 and NaNs sit at the ends ordered by their bits; a tie means
 *     identical bits, hence out == values[arg] bit for bit;
 *   - arg is the absolute row index (int64) per (segment, feature);
 *   - empty min/max: value 0 (luma.gl contract) with arg -1 (graph-reduce);
 *   - scatter: rows whose index lies outside [0, dim_size) take no part; an
 *     output no row names is empty (0, arg -1, mean 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_U32 0
#define ORC_I32 1
#define ORC_F32 2

#define ORC_SUM 0
#define ORC_MIN 1
#define ORC_MAX 2
#define ORC_MEAN 3

/*
 * Monotone order key (graph-reduce README, "Method": a float's bit pattern
 * made monotone as an integer).  Keys compare as unsigned 32-bit integers:
 *   uint32  -> the bits themselves;
 *   int32   -> bits with the sign bit flipped (signed order);
 *   float32 -> negative floats: all bits flipped; others: sign bit set.
 */
uint32_t oracle_order_key(uint32_t bits, int32_t dtype)
{
    if (dtype == ORC_U32)
        return bits;
    if (dtype == ORC_I32)
        return bits ^ 0x80000000u;
    if (bits & 0x80000000u)
        return ~bits;
    return bits | 0x80000000u;
}

static uint32_t load_bits(const void *values, int64_t index)
{
    uint32_t b;
    memcpy(&b, (const unsigned char *)values + 4 * index, 4);
    return b;
}

static float bits_to_float(uint32_t b)
{
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static uint32_t float_to_bits(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

static void store_bits(void *out, int64_t index, uint32_t b)
{
    memcpy((unsigned char *)out + 4 * index, &b, 4);
}

/*
 * oracle_reduce: out[s, f] = op over rows r in [offsets[s], offsets[s+1]) of
 * values[r, f].  values is row-major [rows, feat] of 4-byte elements and
 * rows are absolute indices (offsets[0] may be above 0).
 *
 *   out      [S, feat], same 4-byte type as values (float32 for MEAN);
 *   arg_out  [S, feat] int64, MIN/MAX only, may be NULL;
 *   ref_out  [S, feat] double, float32 SUM/MEAN only, may be NULL:
 *            the double-precision sum (SUM) or sum / length (MEAN);
 *   abs_out  [S, feat] double, float32 SUM/MEAN only, may be NULL:
 *            the double-precision sum of |x| over the segment.
 *
 * Returns 0, or -1 for an argument it does not accept (MEAN of integers,
 * feat < 1, unknown dtype or op).
 */
int oracle_reduce(const void *values, int32_t dtype, int64_t feat,
                  const int64_t *offsets, int64_t num_segments, int32_t op,
                  void *out, int64_t *arg_out, double *ref_out, double *abs_out)
{
    if (dtype < ORC_U32 || dtype > ORC_F32 || op < ORC_SUM || op > ORC_MEAN || feat < 1)
        return -1;
    if (op == ORC_MEAN && dtype != ORC_F32)
        return -1;

    for (int64_t s = 0; s < num_segments; ++s) {
        const int64_t lo = offsets[s];
        const int64_t hi = offsets[s + 1];
        for (int64_t f = 0; f < feat; ++f) {
            const int64_t o = s * feat + f;

            if (op == ORC_SUM || op == ORC_MEAN) {
                if (dtype == ORC_F32) {
                    double sum = 0.0, mag = 0.0;
                    for (int64_t r = lo; r < hi; ++r) {
                        const double x = (double)bits_to_float(load_bits(values, r * feat + f));
                        sum += x;
                        mag += x < 0 ? -x : x;
                    }
                    double result = sum;
                    if (op == ORC_MEAN)
                        result = (hi > lo) ? sum / (double)(hi - lo) : 0.0;
                    store_bits(out, o, float_to_bits((float)result));
                    if (ref_out)
                        ref_out[o] = result;
                    if (abs_out)
                        abs_out[o] = mag;
                } else {
                    uint32_t sum = 0u; /* wraps modulo 2^32 for both integer types */
                    for (int64_t r = lo; r < hi; ++r)
                        sum += load_bits(values, r * feat + f);
                    store_bits(out, o, sum);
                }
                continue;
            }

            /* MIN / MAX with the producing row; strict comparison keeps the
             * first (lowest) row among equal keys. */
            if (hi <= lo) {
                store_bits(out, o, 0u);
                if (arg_out)
                    arg_out[o] = -1;
                continue;
            }
            int64_t best_row = lo;
            uint32_t best_key = oracle_order_key(load_bits(values, lo * feat + f), dtype);
            for (int64_t r = lo + 1; r < hi; ++r) {
                const uint32_t k = oracle_order_key(load_bits(values, r * feat + f), dtype);
                const int better = (op == ORC_MIN) ? (k < best_key) : (k > best_key);
                if (better) {
                    best_key = k;
                    best_row = r;
                }
            }
            store_bits(out, o, load_bits(values, best_row * feat + f));
            if (arg_out)
                arg_out[o] = best_row;
        }
    }
    return 0;
}

/*
 * oracle_rle: run-length encoding of n uint32 keys by adjacency (luma.gl
 * RLE page).  Writes values[0..count), lengths[0..count), offsets[0..count]
 * with offsets[count] = n, and *count.  Entries past the valid prefix are not
 * touched.  Keys are compared bit for bit and need not be sorted.
 */
int oracle_rle(const uint32_t *keys, int64_t n, uint32_t *values, uint32_t *lengths,
               int64_t *offsets, int64_t *count)
{
    if (n < 0)
        return -1;
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || keys[i] != keys[i - 1]) {
            values[c] = keys[i];
            offsets[c] = i;
            ++c;
        }
    }
    offsets[c] = n;
    for (int64_t r = 0; r < c; ++r)
        lengths[r] = (uint32_t)(offsets[r + 1] - offsets[r]);
    *count = c;
    return 0;
}

/*
 * oracle_scan: segmented inclusive or exclusive scan over offset-delimited
 * segments.  GPUSegmentedScan is only named by the luma.gl RLE page
 * ("Composition", next to GPUSegmentedReduction); its reading here follows
 * the segmented reduction's contract (same segments, dtypes, operations and
 * order, empty prefix -> 0): for row r of segment s,
 *   inclusive: out[r, f] = op of values[offsets[s]..r, f]
 *   exclusive: out[r, f] = op of values[offsets[s]..r-1, f], 0 when r is the
 *              segment's first row.
 * Rows are visited in order with one running value per feature: double for
 * float32 sums (ref_out gets the double prefix, abs_out the prefix of |x|),
 * wrapping uint32 for integer sums, the best order key for min/max (out gets
 * that value's bits).  Rows outside [offsets[0], offsets[S]) are not
 * written.  op is ORC_SUM, ORC_MIN or ORC_MAX.
 */
int oracle_scan(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                int64_t num_segments, int32_t op, int32_t exclusive,
                void *out, double *ref_out, double *abs_out)
{
    if (dtype < ORC_U32 || dtype > ORC_F32 || op < ORC_SUM || op > ORC_MAX || feat < 1 || num_segments < 0)
        return -1;
    for (int64_t s = 0; s < num_segments; ++s) {
        const int64_t lo = offsets[s], hi = offsets[s + 1];
        for (int64_t f = 0; f < feat; ++f) {
            double run = 0.0, run_abs = 0.0;
            uint32_t run_int = 0, top_key = 0, top_bits = 0;
            int seen = 0;
            for (int64_t r = lo; r < hi; ++r) {
                const int64_t o = r * feat + f;
                const uint32_t b = load_bits(values, o);
                if (exclusive) {
                    /* the prefix before row r */
                    if (op == ORC_SUM) {
                        if (dtype == ORC_F32) {
                            store_bits(out, o, float_to_bits((float)run));
                            if (ref_out)
                                ref_out[o] = run;
                            if (abs_out)
                                abs_out[o] = run_abs;
                        } else {
                            store_bits(out, o, run_int);
                        }
                    } else {
                        store_bits(out, o, seen ? top_bits : 0u);
                    }
                }
                if (op == ORC_SUM) {
                    if (dtype == ORC_F32) {
                        const double x = (double)bits_to_float(b);
                        run += x;
                        run_abs += x < 0 ? -x : x;
                    } else {
                        run_int += b;
                    }
                } else {
                    const uint32_t k = oracle_order_key(b, dtype);
                    if (!seen || ((op == ORC_MAX) ? (k > top_key) : (k < top_key))) {
                        top_key = k;
                        top_bits = b;
                    }
                    seen = 1;
                }
                if (!exclusive) {
                    if (op == ORC_SUM) {
                        if (dtype == ORC_F32) {
                            store_bits(out, o, float_to_bits((float)run));
                            if (ref_out)
                                ref_out[o] = run;
                            if (abs_out)
                                abs_out[o] = run_abs;
                        } else {
                            store_bits(out, o, run_int);
                        }
                    } else {
                        store_bits(out, o, top_bits);
                    }
                }
            }
        }
    }
    return 0;
}

/*
 * oracle_lower_bounds: many lower-bound queries over segmented sorted values
 * (luma.gl "GPUGallopingSearch": "Overview", "Usage", "Validation").
 *
 * The value at search position p is values[p * stride], or, with an order
 * vector, values[order[p] * stride].  Segment record s is (vo, vc, qo, qc):
 * value positions [vo, vo + vc) and query positions [qo, qo + qc).  For
 * query k of the segment, out[qo + k] = the first position p in
 * [vo, vo + vc) whose value is not less than the query, or vo + vc if
 * there is none (absolute, in the value / order view).  Comparisons are
 * unsigned for uint32 and IEEE for float32.  The validation word:
 *   1  a value range leaves the value view (its segment is not searched),
 *   2  a query range leaves the query view or exceeds the per-segment
 *      capacity max_qc (its segment is not searched),
 *   4  a query is below the one before it in the same tile of T queries
 *      (its lower bound is still exact),
 *   8  a float32 query is not finite: that query and the rest of its tile
 *      are not written.
 * Without `preserve` the word starts from 0.  Outputs that are not written
 * keep their contents.
 */
int oracle_lower_bounds(const void *values, int32_t dtype, int64_t value_count, int64_t stride,
                        const uint32_t *order, int64_t order_count, const void *queries, int64_t query_count,
                        const int64_t *segments, int64_t num_segments, int64_t max_qc, int64_t T,
                        int64_t *out, uint32_t *validation, int32_t preserve)
{
    if ((dtype != ORC_U32 && dtype != ORC_F32) || value_count < 0 || stride < 1 || query_count < 0 ||
        num_segments < 0 || max_qc < 0 || T < 1 || (order && order_count < 0))
        return -1;
    uint32_t word = preserve ? *validation : 0u;
    const int64_t view = order ? order_count : value_count;
    for (int64_t s = 0; s < num_segments; ++s) {
        const int64_t vo = segments[4 * s + 0], vc = segments[4 * s + 1];
        const int64_t qo = segments[4 * s + 2], qc = segments[4 * s + 3];
        const int bad_values = vo < 0 || vc < 0 || vo > view || vc > view - vo;
        const int bad_queries = qo < 0 || qc < 0 || qo > query_count || qc > query_count - qo || qc > max_qc;
        if (bad_values)
            word |= 1u;
        if (bad_queries)
            word |= 2u;
        if (bad_values || bad_queries)
            continue;
        for (int64_t k = 0; k < qc; ++k) {
            const uint32_t qb = load_bits(queries, qo + k);
            if (dtype == ORC_F32 && !isfinite(bits_to_float(qb))) {
                word |= 8u;
                k = (k / T + 1) * T - 1; /* the rest of this tile is skipped */
                continue;
            }
            if (k % T != 0) {
                const uint32_t pb = load_bits(queries, qo + k - 1);
                const int lower = dtype == ORC_F32 ? (bits_to_float(qb) < bits_to_float(pb)) : (qb < pb);
                if (lower)
                    word |= 4u;
            }
            int64_t p = vo;
            while (p < vo + vc) {
                const int64_t row = order ? (int64_t)order[p] : p;
                const uint32_t vb = load_bits(values, row * stride);
                const int less = dtype == ORC_F32 ? (bits_to_float(vb) < bits_to_float(qb)) : (vb < qb);
                if (!less)
                    break;
                ++p;
            }
            out[qo + k] = p;
        }
    }
    *validation = word;
    return 0;
}

/*
 * oracle_unique: the distinct adjacent values of n uint32 keys (luma.gl
 * "GPURunLengthEncode and GPUUnique", section "GPUUnique": the run values of
 * the RLE, with the same bitwise equality and first-occurrence order, and no
 * lengths).  Writes values[0..count) and *count.
 */
int oracle_unique(const uint32_t *keys, int64_t n, uint32_t *values, int64_t *count)
{
    if (n < 0)
        return -1;
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int starts_run = (c == 0) || (keys[i] != values[c - 1]);
        if (starts_run)
            values[c++] = keys[i];
    }
    *count = c;
    return 0;
}

/*
 * oracle_offsets_from_flags: segment offsets from segment-start flags (luma.gl
 * "GPUSegmentedReduction", "Composition": the segmented layout turns start
 * flags into offsets).  Position i starts a segment iff flags[i] != 0; the
 * starts, in position order, are offsets[0..count), offsets[count] = n closes
 * the last segment, *count = number of starts.  Positions before the first
 * start belong to no segment (offsets[0] may be above 0); no flag set gives
 * count 0 and offsets[0] = n.
 */
int oracle_offsets_from_flags(const uint32_t *flags, int64_t n, int64_t *offsets, int64_t *count)
{
    if (n < 0)
        return -1;
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i)
        if (flags[i] != 0)
            offsets[c++] = i;
    offsets[c] = n;
    *count = c;
    return 0;
}

/*
 * oracle_scatter: out[s, f] = op over the rows r with index[r] == s of
 * values[r, f] (graph-reduce README, "API": scatter_sum / scatter_mean /
 * scatter_max / scatter_min).  Rows are visited in ascending order, one at a
 * time; each output keeps its own running sum (double for float32, wrapping
 * uint32 for integers), row count and best (key, row).  Outputs, arg_out,
 * ref_out and abs_out are as for oracle_reduce with dim_size outputs.
 * Returns 0, -1 for an argument it does not accept, -2 if out of memory.
 */
int oracle_scatter(const void *values, int32_t dtype, int64_t feat, int64_t rows,
                   const int64_t *index, int64_t dim_size, int32_t op,
                   void *out, int64_t *arg_out, double *ref_out, double *abs_out)
{
    if (dtype < ORC_U32 || dtype > ORC_F32 || op < ORC_SUM || op > ORC_MEAN || feat < 1 || rows < 0 ||
        dim_size < 0)
        return -1;
    if (op == ORC_MEAN && dtype != ORC_F32)
        return -1;
    const int64_t cells = dim_size * feat;
    double *sum = calloc((size_t)(cells > 0 ? cells : 1), sizeof(double));
    double *mag = calloc((size_t)(cells > 0 ? cells : 1), sizeof(double));
    uint32_t *isum = calloc((size_t)(cells > 0 ? cells : 1), sizeof(uint32_t));
    uint32_t *best_key = calloc((size_t)(cells > 0 ? cells : 1), sizeof(uint32_t));
    int64_t *best_row = malloc((size_t)(cells > 0 ? cells : 1) * sizeof(int64_t));
    int64_t *count = calloc((size_t)(dim_size > 0 ? dim_size : 1), sizeof(int64_t));
    if (!sum || !mag || !isum || !best_key || !best_row || !count) {
        free(sum); free(mag); free(isum); free(best_key); free(best_row); free(count);
        return -2;
    }
    for (int64_t cell = 0; cell < cells; ++cell)
        best_row[cell] = -1;

    for (int64_t r = 0; r < rows; ++r) {
        const int64_t s = index[r];
        if (s < 0 || s >= dim_size)
            continue;
        count[s] += 1;
        for (int64_t f = 0; f < feat; ++f) {
            const int64_t cell = s * feat + f;
            const uint32_t b = load_bits(values, r * feat + f);
            if (op == ORC_SUM || op == ORC_MEAN) {
                if (dtype == ORC_F32) {
                    const double x = (double)bits_to_float(b);
                    sum[cell] += x;
                    mag[cell] += x < 0 ? -x : x;
                } else {
                    isum[cell] += b;
                }
            } else {
                /* the first row seen wins until a strictly better key comes:
                 * ties keep the lower row */
                const uint32_t k = oracle_order_key(b, dtype);
                const int better = best_row[cell] < 0 || ((op == ORC_MIN) ? (k < best_key[cell]) : (k > best_key[cell]));
                if (better) {
                    best_key[cell] = k;
                    best_row[cell] = r;
                }
            }
        }
    }

    for (int64_t s = 0; s < dim_size; ++s) {
        for (int64_t f = 0; f < feat; ++f) {
            const int64_t cell = s * feat + f;
            if (op == ORC_SUM || op == ORC_MEAN) {
                if (dtype == ORC_F32) {
                    double result = sum[cell];
                    if (op == ORC_MEAN)
                        result = count[s] > 0 ? sum[cell] / (double)count[s] : 0.0;
                    store_bits(out, cell, float_to_bits((float)result));
                    if (ref_out)
                        ref_out[cell] = result;
                    if (abs_out)
                        abs_out[cell] = mag[cell];
                } else {
                    store_bits(out, cell, isum[cell]);
                }
            } else {
                const int64_t br = best_row[cell];
                store_bits(out, cell, br < 0 ? 0u : load_bits(values, br * feat + f));
                if (arg_out)
                    arg_out[cell] = br;
            }
        }
    }
    free(sum); free(mag); free(isum); free(best_key); free(best_row); free(count);
    return 0;
}

/*
 * oracle_offsets_from_index: offsets[s] = number of rows whose index is in
 * [0, s), for s = 0..dim_size (graph-reduce README, "Usage": bincount of the
 * index, then a cumulative sum after a leading 0).  Rows outside
 * [0, dim_size) are not counted.
 */
int oracle_offsets_from_index(const int64_t *index, int64_t rows, int64_t dim_size, int64_t *offsets)
{
    if (rows < 0 || dim_size < 0)
        return -1;
    for (int64_t s = 0; s <= dim_size; ++s)
        offsets[s] = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t s = index[r];
        if (s >= 0 && s < dim_size)
            offsets[s + 1] += 1;
    }
    for (int64_t s = 0; s < dim_size; ++s)
        offsets[s + 1] += offsets[s];
    return 0;
}
