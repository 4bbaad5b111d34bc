// galloping.hip -- many lower-bound queries over segmented sorted values
// (luma.gl "GPUGallopingSearch": "Overview", "Usage", "Validation", "Cost
// model").
//
// Segment record s = (vo, vc, qo, qc): value positions [vo, vo + vc) (of the
// value view, or of the order view when an order vector is given: position
// p then means row order[p]), query positions [qo, qo + qc).  out[qo + k] is
// the first position p in [vo, vo + vc) whose value is not less than query
// k, or vo + vc.  The queries of a segment are cut into tiles of T; each
// (segment, tile) pair is one lane and independent of the others, as on the
// page: the tile's first query (and any query below its predecessor) is
// found by a full search of the segment, every later query by galloping
// forward from the previous answer, then a bounded search, then a linear
// scan once at most 16 values remain.
//
// Two kernels compute those answers.  When a record has at most 256 tiles
// (ceil(max_query_count / T) <= 256), gallop_staged gives each record a
// workgroup: a record of at most 4,096 values is copied into LDS once, and
// each thread answers whole queries (consecutive threads on consecutive
// queries) by a binary search in LDS, so every memory access is coalesced
// and no probe leaves the CU.  A lower bound is the same whichever search
// finds it, so the tile rules are kept query by query (bit 4 below); only a
// record with a non-finite query goes tile by tile, since such a query ends
// its tile.  Otherwise gallop_kernel runs one lane per (record, tile) with
// the page's steps below.
//
// For gfx950 each of those steps issues its probes together instead of one
// after another, because a probe is a memory round trip: the gallop loads
// the 16 values after the previous answer (one 64-byte run) and 6
// exponential probes up to 1023 positions on in one round; a bounded
// search splits its range 16 ways per round (15 probes loaded together); the
// final linear scan loads its <= 16 values at once and takes the first one
// not below the query.  The exponential probes join the first window only
// for a lane whose previous gap was wider than the window (each probe is a
// cache line of its own).  The next query is loaded while the current one is
// searched, and answers are stored four at a time.  The answer is the same
// lower bound; only the number of dependent round trips and the memory
// traffic shrink.
//
// Validation word (OR of): 1 a value range leaves its view, 2 a query range
// leaves the query view or exceeds the per-segment capacity (neither
// segment is searched), 4 a query below its predecessor in a tile (answered
// by a full search, still exact), 8 a non-finite float32 query (it and the
// rest of its tile are not written).  Bits are set with an atomic OR, whose
// result does not depend on arrival order; each lane ORs once.
#include "internal.hpp"
#include "keys.hpp"
#include "wave.hpp"

namespace segred {

struct GArgs {
    const uint32_t *values;  // element bits; value i at values[i * stride]
    int64_t value_count, stride;
    const uint32_t *order;   // [order_count] rows of the search positions, or null
    int64_t order_count;
    const uint32_t *queries;  // [query_count]
    int64_t query_count;
    const int64_t *segments;  // [S][4]
    int64_t S, max_qc, T, tiles;  // tiles per segment = ceil(max_qc / T)
    int64_t *out;                 // [query_count]
    uint32_t *validation;
};

constexpr int kGThreads = 256;

__global__ __launch_bounds__(64) void gallop_clear(uint32_t *w) {
    if (threadIdx.x == 0) *w = 0u;
}

template <int DT, bool ORDER>
struct Probe {
    const uint32_t *values;
    const uint32_t *order;
    int64_t value_count, stride;
    // Value bits at search position p (p inside the validated range).  A row
    // past the value view (a broken order vector, which the caller must
    // prevent) reads as a value no query is above, without touching memory.
    __device__ __forceinline__ uint32_t at(int64_t p) const {
        int64_t row = p;
        if constexpr (ORDER) row = (int64_t)order[p];
        if (row >= value_count) return DT == DT_F32 ? 0x7FC00000u : 0xFFFFFFFFu;
        return values[row * stride];
    }
    // The 16 values at positions a .. a+15 (entries at or past `end` are not
    // used).  A plain column (no order vector, stride 1) whose window lies
    // inside the segment is read with four 16-byte loads (the address is
    // only 4-byte aligned, which the type says).
    __device__ __forceinline__ void window16(int64_t a, int64_t end, uint32_t (&w)[16]) const {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
        if (!ORDER && stride == 1 && a + 16 <= end) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(values + a);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = p[j];
                w[4 * j] = v.x;
                w[4 * j + 1] = v.y;
                w[4 * j + 2] = v.z;
                w[4 * j + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) w[j] = a + j < end ? at(a + j) : 0u;
        }
    }
    // value < query, in the value type (IEEE for float32, unsigned for uint32)
    static __device__ __forceinline__ bool less(uint32_t v, uint32_t q) {
        if constexpr (DT == DT_F32) return __uint_as_float(v) < __uint_as_float(q);
        else return v < q;
    }
};

// A record's values staged in LDS: search position p is s_vals[p - vo].
constexpr int kStageValues = 4096;  // 16 KB per workgroup

template <int DT>
struct LdsProbe {
    const uint32_t *vals;
    int64_t vo;
    __device__ __forceinline__ uint32_t at(int64_t p) const { return vals[p - vo]; }
    __device__ __forceinline__ void window16(int64_t a, int64_t end, uint32_t (&w)[16]) const {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = a + j < end ? vals[a + j - vo] : 0u;
    }
    static __device__ __forceinline__ bool less(uint32_t v, uint32_t q) { return Probe<DT, false>::less(v, q); }
};

// Lower bound of q in [lo, hi), knowing every position before lo is below q
// and (when hi is not the segment end) position hi is not.  16-way rounds
// while more than 16 positions remain, then one round over the rest.
template <class P>
__device__ __forceinline__ int64_t bounded(const P &pr, int64_t lo, int64_t hi, uint32_t q) {
    while (hi - lo > 16) {
        const int64_t n = hi - lo;
        int64_t pos[15];
        uint32_t v[15];
#pragma unroll
        for (int j = 0; j < 15; ++j) pos[j] = lo + (n * (j + 1)) / 16;  // strictly inside [lo, hi)
#pragma unroll
        for (int j = 0; j < 15; ++j) v[j] = pr.at(pos[j]);
        int64_t nlo = lo, nhi = hi;
        bool found = false;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
            if (!found) {
                if (P::less(v[j], q)) {
                    nlo = pos[j] + 1;
                } else {
                    nhi = pos[j];
                    found = true;
                }
            }
        }
        lo = nlo;
        hi = nhi;
    }
    // linear finish: the first of the <= 16 remaining values not below q
    uint32_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = lo + j < hi ? pr.at(lo + j) : 0u;
    int64_t lb = hi;
#pragma unroll
    for (int j = 15; j >= 0; --j)
        if (lo + j < hi && !P::less(v[j], q)) lb = lo + j;
    return lb;
}

// Gallop from position a (every position before a is below q): one round
// loads the 16 positions a .. a+15 together with 6 exponential probes at
// a+31, a+63, ... a+1023, so any answer within about a thousand positions is
// bracketed by a single round trip (the lanes of a wave search in lockstep,
// so a wave waits for its slowest lane: every query should cost the same few
// rounds).  If all are below q, the next round starts at a+1024 with a
// window and probes 64 times coarser.  A bracket is finished by `bounded`.
template <class P>
__device__ __forceinline__ int64_t gallop(const P &pr, int64_t a, int64_t end, uint32_t q, bool wide) {
    int64_t base = a;
    int64_t scale = 1;
    for (;;) {
        if (base >= end) return end;
        uint32_t w[16], e[6];
        auto load_probes = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int64_t p = base + ((int64_t)32 << i) * scale - 1;
                e[i] = p < end ? pr.at(p) : 0u;
            }
        };
        if (scale == 1) {
            pr.window16(base, end, w);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) w[j] = base + j * scale < end ? pr.at(base + j * scale) : 0u;
        }
        // the exponential probes ride along with the first window only when
        // this lane's last gap was wide (they cost a cache line each)
        if (wide || scale != 1) load_probes();
        if (scale == 1) {
            // dense window: the first of base .. base+15 not below q is the
            // answer; past the end of the segment, the end is
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (base + j >= end) return end;
                if (!P::less(w[j], q)) return base + j;
            }
        } else {
            // sparse window: bracket the answer between two samples (or
            // between the last sample and the end of the segment)
            int64_t prev = base - 1;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t p = base + j * scale;
                if (p >= end) return bounded(pr, prev + 1, end, q);
                if (!P::less(w[j], q)) return bounded(pr, prev + 1, p, q);
                prev = p;
            }
        }
        if (!wide && scale == 1) load_probes();
        // the window is below q; take the first exponential probe not below
        int64_t prev = base + 15 * scale;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int64_t p = base + ((int64_t)32 << i) * scale - 1;
            if (p >= end) return bounded(pr, prev + 1, end, q);
            if (!P::less(e[i], q)) return bounded(pr, prev + 1, p, q);
            prev = p;
        }
        base = prev + 1;
        scale *= 64;  // farther probes next round
    }
}

// Queries k0 .. k1-1 of a record (one tile), the page's steps: returns the
// validation bits.  Used by gallop_kernel.
template <int DT, class P>
__device__ __forceinline__ uint32_t search_tile(const GArgs &a, const P &pr, int64_t vo, int64_t end, int64_t qo,
                                                int64_t k0, int64_t k1) {
    uint32_t bits = 0;
    int64_t lb = vo;
    uint32_t prevq = 0;
    uint32_t qn = a.queries[qo + k0];
    bool wide = true;
    // answers go out four at a time (32 contiguous bytes per lane rather than
    // 8-byte pieces spread over the search)
    int64_t held[4];
    int nheld = 0;
    int64_t k = k0;
    for (; k < k1; ++k) {
        const uint32_t q = qn;
        if (k + 1 < k1) qn = a.queries[qo + k + 1];  // next query in flight during this search
        if (DT == DT_F32 && !isfinite(__uint_as_float(q))) {
            bits |= 8u;
            break;  // the rest of the tile is not written
        }
        bool full = k == k0;
        if (!full && P::less(q, prevq)) {
            bits |= 4u;
            full = true;
        }
        const int64_t nlb = full ? bounded(pr, vo, end, q) : gallop(pr, lb, end, q, wide);
        wide = full || nlb - lb > 16;
        lb = nlb;
        prevq = q;
        held[nheld++ & 3] = lb;
        if (nheld == 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) a.out[qo + k - 3 + j] = held[j];
            nheld = 0;
        }
    }
    // the answers still held belong to the queries just before k
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (j < nheld) a.out[qo + k - nheld + j] = held[j];
    return bits;
}

// Lower bound of q over a whole record: a plain binary search in LDS (one
// read per step; the waves resident on a CU hide its latency), the 16-way
// rounds of `bounded` through memory.
template <int DT>
__device__ __forceinline__ int64_t record_lower_bound(const LdsProbe<DT> &pr, int64_t vo, int64_t end, uint32_t q) {
    uint32_t lo = 0, n = (uint32_t)(end - vo);  // at most kStageValues
    while (n > 0) {
        const uint32_t half = n >> 1;
        if (LdsProbe<DT>::less(pr.vals[lo + half], q)) {
            lo += half + 1;
            n -= half + 1;
        } else {
            n = half;
        }
    }
    return vo + lo;
}

template <int DT, bool ORDER>
__device__ __forceinline__ int64_t record_lower_bound(const Probe<DT, ORDER> &pr, int64_t vo, int64_t end,
                                                      uint32_t q) {
    return bounded(pr, vo, end, q);
}

// Every query of a record, consecutive threads on consecutive queries
// (coalesced loads and stores): a search of the whole record each, bit 4 for
// a query below its predecessor in the same tile.
template <int DT, class P>
__device__ __forceinline__ uint32_t answer_queries(const GArgs &a, const P &pr, int64_t vo, int64_t end, int64_t qo,
                                                   int64_t qc) {
    uint32_t bits = 0;
    const uint32_t *qs = a.queries + qo;
    // position of query k in its tile, stepped along with k
    const int64_t step = kGThreads % a.T;
    int64_t in_tile = (int64_t)threadIdx.x % a.T;
    for (int64_t k = threadIdx.x; k < qc; k += kGThreads) {
        const uint32_t q = qs[k];
        if (in_tile != 0 && P::less(q, qs[k - 1])) bits |= 4u;
        a.out[qo + k] = record_lower_bound<DT>(pr, vo, end, q);
        in_tile += step;
        if (in_tile >= a.T) in_tile -= a.T;
    }
    return bits;
}

// A record with a non-finite query: one lane per tile, queries in order; a
// non-finite query sets bit 8 and ends its tile (it and the rest are not
// written), a query below its predecessor sets bit 4.  Each answer is the
// same whole-record lower bound.
template <int DT, class P>
__device__ __forceinline__ uint32_t answer_tiles(const GArgs &a, const P &pr, int64_t vo, int64_t end, int64_t qo,
                                                 int64_t qc) {
    uint32_t bits = 0;
    const int64_t ntiles = (qc + a.T - 1) / a.T;
    for (int64_t t = threadIdx.x; t < ntiles; t += kGThreads) {
        const int64_t k0 = t * a.T, k1 = min(k0 + a.T, qc);
        uint32_t prevq = 0;
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t q = a.queries[qo + k];
            if (DT == DT_F32 && !isfinite(__uint_as_float(q))) {
                bits |= 8u;
                break;
            }
            if (k != k0 && P::less(q, prevq)) bits |= 4u;
            a.out[qo + k] = record_lower_bound<DT>(pr, vo, end, q);
            prevq = q;
        }
    }
    return bits;
}

// Record checks (bits 1 and 2); true when the record may be searched.
__device__ __forceinline__ bool record_ok(const GArgs &a, bool order, int64_t vo, int64_t vc, int64_t qo, int64_t qc,
                                          uint32_t &bits) {
    const int64_t view = order ? a.order_count : a.value_count;
    const bool bad_v = vo < 0 || vc < 0 || vo > view || vc > view - vo;
    const bool bad_q = qo < 0 || qc < 0 || qo > a.query_count || qc > a.query_count - qo || qc > a.max_qc;
    bits = (bad_v ? 1u : 0u) | (bad_q ? 2u : 0u);
    return bits == 0;
}

// One lane per (record, tile): for records with more tiles than a workgroup
// has lanes.
template <int DT, bool ORDER>
__global__ __launch_bounds__(kGThreads) void gallop_kernel(const GArgs a) {
    const int64_t id = (int64_t)blockIdx.x * kGThreads + threadIdx.x;
    const int64_t s = id / a.tiles, t = id - s * a.tiles;
    if (s >= a.S) return;
    const int64_t vo = a.segments[4 * s + 0], vc = a.segments[4 * s + 1];
    const int64_t qo = a.segments[4 * s + 2], qc = a.segments[4 * s + 3];
    uint32_t bits = 0;
    if (!record_ok(a, ORDER, vo, vc, qo, qc, bits)) {
        if (t == 0) __hip_atomic_fetch_or(a.validation, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t k0 = t * a.T;
    if (k0 >= qc) return;
    const Probe<DT, ORDER> pr{a.values, a.order, a.value_count, a.stride};
    bits = search_tile<DT>(a, pr, vo, vo + vc, qo, k0, min(k0 + a.T, qc));
    if (bits) __hip_atomic_fetch_or(a.validation, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per record.  A record of at most kStageValues values is
// first copied into LDS (coalesced loads, once); then each thread answers
// whole queries, consecutive threads on consecutive queries, so query loads
// and answer stores are coalesced, and every probe is an LDS read (a larger
// record is searched through memory, query by query).  The answers are the
// lower bounds, the same whatever search finds them; the tile rules still
// hold query by query: a query below its predecessor in the same tile sets
// bit 4.  A record with a non-finite float32 query (bit 8: the rest of its
// tile is not written) goes tile by tile, one lane per tile.
template <int DT, bool ORDER>
__global__ __launch_bounds__(kGThreads) void gallop_staged(const GArgs a) {
    __shared__ uint32_t s_vals[kStageValues];
    const int64_t s = blockIdx.x;
    const int64_t vo = a.segments[4 * s + 0], vc = a.segments[4 * s + 1];
    const int64_t qo = a.segments[4 * s + 2], qc = a.segments[4 * s + 3];
    uint32_t bits = 0;
    if (!record_ok(a, ORDER, vo, vc, qo, qc, bits)) {
        if (threadIdx.x == 0) __hip_atomic_fetch_or(a.validation, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const Probe<DT, ORDER> pr{a.values, a.order, a.value_count, a.stride};
    const int64_t end = vo + vc;
    const bool stage = vc <= kStageValues;  // the same for the whole workgroup
    // every load of the staging (and of the non-finite check of the first
    // kStageValues queries) issued before the first LDS store
    constexpr int kPer = kStageValues / kGThreads;
    uint32_t v[kPer], w[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t i = u * kGThreads + threadIdx.x;
        v[u] = stage && i < vc ? pr.at(vo + i) : 0u;
        w[u] = i < qc ? a.queries[qo + i] : 0u;
    }
    bool nonfinite = false;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t i = u * kGThreads + threadIdx.x;
        if (stage && i < vc) s_vals[i] = v[u];
        if constexpr (DT == DT_F32) nonfinite |= i < qc && !isfinite(__uint_as_float(w[u]));
    }
    if constexpr (DT == DT_F32)
        for (int64_t k = kStageValues + threadIdx.x; k < qc; k += kGThreads)
            nonfinite |= !isfinite(__uint_as_float(a.queries[qo + k]));
    const bool by_tile = __syncthreads_or(nonfinite) != 0;  // also orders the LDS stores before the searches
    if (!by_tile) {
        if (stage)
            bits |= answer_queries<DT>(a, LdsProbe<DT>{s_vals, vo}, vo, end, qo, qc);
        else
            bits |= answer_queries<DT>(a, pr, vo, end, qo, qc);
    } else {
        if (stage)
            bits |= answer_tiles<DT>(a, LdsProbe<DT>{s_vals, vo}, vo, end, qo, qc);
        else
            bits |= answer_tiles<DT>(a, pr, vo, end, qo, qc);
    }
    if (bits) __hip_atomic_fetch_or(a.validation, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT>
static int gallop_launch(const GArgs &a, hipStream_t st) {
    if (a.S == 0) return SEGRED_OK;
    if (a.tiles <= kGThreads) {
        // a workgroup per record (its tiles fit the workgroup's lanes)
        if (a.S > INT32_MAX) return SEGRED_ERR_UNSUPPORTED;
        if (a.order)
            timed_launch_ggl(true, (gallop_staged<DT, true>), dim3((unsigned)a.S), dim3(kGThreads), 0, st, a);
        else
            timed_launch_ggl(true, (gallop_staged<DT, false>), dim3((unsigned)a.S), dim3(kGThreads), 0, st, a);
        return hipGetLastError() == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
    }
    const int64_t lanes = a.S * a.tiles;
    const int64_t wgs = (lanes + kGThreads - 1) / kGThreads;
    if (wgs > INT32_MAX) return SEGRED_ERR_UNSUPPORTED;
    if (a.order)
        timed_launch_ggl(true, (gallop_kernel<DT, true>), dim3((unsigned)wgs), dim3(kGThreads), 0, st, a);
    else
        timed_launch_ggl(true, (gallop_kernel<DT, false>), dim3((unsigned)wgs), dim3(kGThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

}  // namespace segred

using namespace segred;

extern "C" int segred_galloping_search(const void *values, int32_t dtype, int64_t value_count, int64_t value_stride,
                                       const uint32_t *value_order, int64_t order_count, const void *queries,
                                       int64_t query_count, const int64_t *segments, int64_t num_segments,
                                       int64_t max_query_count, int32_t queries_per_tile, int64_t *out,
                                       uint32_t *validation, int32_t preserve_validation, hipStream_t stream) {
    if (dtype < SEGRED_U32 || dtype > SEGRED_F32) return SEGRED_ERR_INVALID_ARGUMENT;
    if (dtype == SEGRED_I32) return SEGRED_ERR_UNSUPPORTED;
    if (value_count < 0 || value_stride < 1 || query_count < 0 || num_segments < 0 || max_query_count < 0 ||
        queries_per_tile < 1 || (value_order && order_count < 0))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (value_count > 0 && value_stride > INT64_MAX / value_count) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!validation || (num_segments > 0 && !segments) || (value_count > 0 && !values) ||
        (query_count > 0 && (!queries || !out)))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (!aligned(validation, 4) || (values && !aligned(values, 4)) || (queries && !aligned(queries, 4)) ||
        (value_order && !aligned(value_order, 4)) || (segments && !aligned(segments, 8)) ||
        (out && !aligned(out, 8)))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (!preserve_validation) {
        timed_launch_ggl(false, gallop_clear, dim3(1), dim3(64), 0, stream, validation);
        if (hipGetLastError() != hipSuccess) return SEGRED_ERR_HIP;
    }
    GArgs a{};
    a.values = static_cast<const uint32_t *>(values);
    a.value_count = value_count;
    a.stride = value_stride;
    a.order = value_order;
    a.order_count = value_order ? order_count : 0;
    a.queries = static_cast<const uint32_t *>(queries);
    a.query_count = query_count;
    a.segments = segments;
    a.S = num_segments;
    a.max_qc = max_query_count;
    a.T = queries_per_tile;
    a.tiles = max_query_count > 0 ? (max_query_count + queries_per_tile - 1) / queries_per_tile : 1;
    a.out = out;
    a.validation = validation;
    return dtype == SEGRED_F32 ? gallop_launch<DT_F32>(a, stream) : gallop_launch<DT_U32>(a, stream);
}
