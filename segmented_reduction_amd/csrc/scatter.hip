// scatter.hip -- reduction of rows into the outputs an index names (the
// scatter form of the segmented reduction), and the CSR offsets of an index.
//
// Operation (phanerozoic/graph-reduce README): "API" -- scatter_sum,
// scatter_mean, scatter_max and scatter_min take rows [N, ...], an int64
// index [N] and dim_size outputs; the mean of an output no row reaches is 0;
// max and min also give the producing row.  "Method" -- one atomic operation
// per element; max and min resolve value and row in a single 64-bit atomic on
// the word (order key << 32) | row code, ties to the lower row.  "Usage" --
// the CSR pointer of a destination-sorted index is the count of rows per
// destination, cumulatively summed behind a leading 0.
//
// These kernels use global atomic operations, so a float sum depends on the
// order in which the atomics arrive and may differ in its last bits from run
// to run (the README's "Correctness" notes the same of its atomic path);
// integer sums, min/max with their rows, counts and offsets are exact.
//
// Scatter launch.  Items are (row, 64-feature chunk) pairs.  Each lane owns
// one feature of one item: L lanes per item (L = the smallest power of two
// >= min(F, 64)), G = 64 / L consecutive items per wave step, kSteps steps per
// wave, all index and value loads of a wave issued before its atomics.  For
// 1-D values (L = 1) a step's 64 consecutive rows are first combined over
// runs of equal index by a segmented scan across the wave (skipped when no
// two neighbours share an index), so a sorted or clustered index sends one
// atomic per run rather than one per row.
//
// With few outputs (one copy fits 32 KB of LDS) and at least 128 rows x
// features per output cell, each workgroup accumulates into a private LDS
// copy, stores it to its own scratch slot, and two fold kernels combine the
// copies in a fixed order with plain stores and write the final values
// (scatter_private, scatter_private_fold_a/_b).  Float sums of rows with
// >= 8 features use one copy per wave and no atomics at all, so they repeat
// bit for bit; float sums of wider rows whose wave copies do not fit stay on
// the element-atomic path (LDS float atomics are slower than global ones
// spread over many cells); other sums and min/max use LDS atomics (integer
// sums and min/max are exact in any order).
//
// Rows whose index lies outside [0, dim_size) are skipped: they take part in
// no output (and no memory outside the outputs is touched for them).
#include <algorithm>

#include "internal.hpp"
#include "keys.hpp"
#include "scan.hpp"
#include "wave.hpp"

namespace segred {

constexpr int kScThreads = 256;
constexpr int kScSteps = 8;
constexpr int kCountTile = 4096;            // counts per tile of the offsets scan
constexpr int kCountThreads = 256;          // 16 counts per thread
constexpr int kCountScanThreads = 1024;
constexpr int kCountScanPer = 4;

struct ScArgs {
    const uint32_t *values;  // element bits, row-major [rows, F]
    const int64_t *index;    // [rows]
    int64_t rows, F, chunks, dim, items;  // chunks = ceil(F / 64) when F > 64, else 1; items = rows * chunks
    int lg;                  // log2 of the lanes per item
    uint32_t *out;           // [dim, F]: sums (SUM, MEAN)
    uint64_t *words;         // [dim, F]: packed key/row words (MIN, MAX)
    uint32_t *counts;        // [dim]: rows per output (MEAN)
    uint32_t *priv;          // [priv_grid][T] private copies: cells (32- or 64-bit), then for MEAN dim counts
    uint32_t *part;          // [<= 64][T] partial folds of the copies (when priv_grid > 64)
    int64_t priv_grid;       // workgroups of the private path, 0 for the element-atomic path
    int word_filter;         // MIN/MAX element atomics: skip those the current word already beats
    int priv_waves;          // private path with one copy per wave (float sums of >= 8 features)
    int priv_lds;            // LDS bytes per workgroup of the private path
};

// Packed word of (key, row): the integer max of MAX words is the largest key
// and, among equal keys, the lowest row (row code ~row); the integer min of
// MIN words is the smallest key, then the lowest row.  Rows are below
// 2^32 - 1, so an untouched word (0 for MAX, all ones for MIN) is no row's.
template <int OP>
__device__ __forceinline__ uint64_t pack(uint32_t key, int64_t row) {
    const uint32_t code = OP == OP_MAX ? ~(uint32_t)row : (uint32_t)row;
    return ((uint64_t)key << 32) | code;
}
template <int OP>
constexpr uint64_t kEmptyWord = OP == OP_MAX ? 0ull : ~0ull;

// Fill kernel for the outputs' starting state (no memset node, so a caller
// may capture the call in a graph).
__global__ __launch_bounds__(kScThreads) void scatter_init(uint32_t *p32, int64_t n32, uint32_t v32, uint64_t *p64,
                                                           int64_t n64, uint64_t v64) {
    const int64_t stride = (int64_t)gridDim.x * kScThreads;
    for (int64_t i = (int64_t)blockIdx.x * kScThreads + threadIdx.x; i < n32; i += stride) p32[i] = v32;
    for (int64_t i = (int64_t)blockIdx.x * kScThreads + threadIdx.x; i < n64; i += stride) p64[i] = v64;
}

template <int DT, int OP>
__device__ __forceinline__ void scatter_apply(const ScArgs &a, int64_t cell, uint32_t x, uint64_t w) {
    if constexpr (OP == OP_MAX) {
        __hip_atomic_fetch_max(a.words + cell, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (OP == OP_MIN) {
        __hip_atomic_fetch_min(a.words + cell, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (DT == DT_F32) {
        unsafeAtomicAdd(reinterpret_cast<float *>(a.out) + cell, __uint_as_float(x));
    } else {
        __hip_atomic_fetch_add(a.out + cell, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Combine two partials of one run (x, w as in scatter_apply).
template <int DT, int OP>
__device__ __forceinline__ void combine(uint32_t &x, uint64_t &w, uint32_t y, uint64_t v) {
    if constexpr (OP == OP_MAX) w = v > w ? v : w;
    else if constexpr (OP == OP_MIN) w = v < w ? v : w;
    else if constexpr (DT == DT_F32) x = __float_as_uint(__uint_as_float(y) + __uint_as_float(x));
    else x = y + x;
}

template <int DT, int OP, bool RUNS>
__global__ __launch_bounds__(kScThreads) void scatter_kernel(ScArgs a) {
    constexpr bool kWord = OP == OP_MIN || OP == OP_MAX;
    const int lane = threadIdx.x & 63;
    const int lg = RUNS ? 0 : a.lg;
    const int64_t G = 64 >> lg;
    const int64_t wave = (int64_t)blockIdx.x * (kScThreads / 64) + (threadIdx.x >> 6);
    const int64_t qbase = wave * kScSteps * G;
    const int sub = lane & ((1 << lg) - 1);

    int64_t s[kScSteps], row[kScSteps], fe[kScSteps];
    uint32_t x[kScSteps];
    bool live[kScSteps];
#pragma unroll
    for (int u = 0; u < kScSteps; ++u) {
        int64_t q = qbase + u * G + (lane >> lg);
        int64_t r = q, f = sub;
        if (!RUNS && a.chunks > 1) {
            // one item per wave step here (64 lanes per item): q is uniform
            q = readfirst(q);
            r = q / a.chunks;
            f = (q - r * a.chunks) * 64 + lane;
        }
        live[u] = q < a.items && f < a.F;
        s[u] = live[u] ? a.index[r] : -1;
        x[u] = live[u] ? a.values[r * a.F + f] : 0u;
        row[u] = r;
        fe[u] = f;
    }

    int64_t wcell[kScSteps];  // MIN/MAX: the cell each step's word goes to, or -1
    uint64_t wv[kScSteps];
#pragma unroll
    for (int u = 0; u < kScSteps; ++u) {
        const int64_t r = row[u], f = fe[u];
        uint64_t w = 0;
        if constexpr (kWord) w = pack<OP>(okey<DT>(x[u]), r);
        uint32_t xv = x[u];
        bool act = s[u] >= 0 && s[u] < a.dim && live[u];
        uint32_t cnt = 1;
        if constexpr (RUNS) {
            // runs of equal index among the step's 64 consecutive rows
            const int64_t prev = lane_get(s[u], (lane - 1) & 63);
            const bool head = lane == 0 || s[u] != prev;
            const uint64_t heads = ballot(head);
            if (heads != ~0ull) {
                bool fl = head;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t yx = lane_get(xv, (lane - o) & 63);
                    uint64_t yw = 0;
                    if constexpr (kWord) yw = lane_get(w, (lane - o) & 63);
                    const bool yf = lane_get(fl, (lane - o) & 63);
                    if (lane >= o && !fl) {
                        combine<DT, OP>(xv, w, yx, yw);
                        fl = yf;
                    }
                }
                const bool last = lane == 63 || ((heads >> (lane + 1)) & 1ull);
                const uint64_t upto = heads & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
                cnt = (uint32_t)(lane - (63 - __clzll((long long)upto)) + 1);
                act = act && last;
            }
        }
        if constexpr (kWord) {
            wcell[u] = act ? s[u] * a.F + f : -1;
            wv[u] = w;
        } else if (act) {
            scatter_apply<DT, OP>(a, s[u] * a.F + f, xv, w);
            if constexpr (OP == OP_MEAN) {
                if (f == 0)
                    __hip_atomic_fetch_add(a.counts + s[u], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if constexpr (kWord) {
        // A word only ever moves one way (up for MAX, down for MIN), so a
        // value that does not beat the word as read cannot win: skip its
        // atomic.  A stale read only lets an atomic through that was not
        // needed; it never drops one that was.  Worth its read when many rows
        // share an output (most values then lose); word_filter says so.
        uint64_t cur[kScSteps];
#pragma unroll
        for (int u = 0; u < kScSteps; ++u)
            cur[u] = a.word_filter && wcell[u] >= 0
                         ? __hip_atomic_load(a.words + wcell[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                         : kEmptyWord<OP>;
#pragma unroll
        for (int u = 0; u < kScSteps; ++u)
            if (wcell[u] >= 0 && (OP == OP_MAX ? wv[u] > cur[u] : wv[u] < cur[u]))
                scatter_apply<DT, OP>(a, wcell[u], 0u, wv[u]);
    }
}

// Few outputs: each workgroup accumulates into its own copy of the outputs
// in LDS (LDS atomics, resolved inside the CU) and stores that copy to its
// scratch slot.  Used when the outputs fit kPrivBytes and the rows are many
// times the output cells (the page's contended case: many rows into a few
// hundred outputs, where element atomics to the same few addresses
// serialise at the memory side).  The LDS is sized per launch (priv_lds),
// so small output sets leave room for more workgroups per CU.
constexpr int kPrivBytes = 32768;
constexpr int kLdsPerCu = 163840;  // 160 KB of LDS per compute unit
constexpr int kWgPerCu = 8;        // 32 waves per CU in workgroups of 4 waves
constexpr int kPrivSteps = 8;      // wave steps whose loads are issued together

//
// WAVES (float sums with rows of >= 8 features): each wave keeps a copy of
// its own and adds with a plain read-modify-write, one row group of the step
// after another (at most 8 turns), so no two lanes touch a cell at once and
// no LDS float atomic (several times slower than the integer ones here) is
// needed; the four copies are added in wave order at the end, so the
// workgroup's partial sums have a fixed order.  Integer sums keep the LDS
// atomics, which are exact in any order and faster than the turns.
template <int DT, int OP, bool WAVES>
__global__ __launch_bounds__(kScThreads) void scatter_private(ScArgs a) {
    constexpr bool kWord = OP == OP_MIN || OP == OP_MAX;
    static_assert(!(WAVES && kWord), "per-wave copies are for sums");
    extern __shared__ __attribute__((aligned(16))) uint64_t s_priv[];  // priv_lds bytes
    uint64_t *c64 = s_priv;
    uint32_t *c32 = reinterpret_cast<uint32_t *>(s_priv);
    const int64_t cells = a.dim * a.F;
    constexpr int kCopies = WAVES ? kScThreads / 64 : 1;
    uint32_t *cnt = c32 + (kWord ? 2 * cells : kCopies * cells);  // MEAN: rows per output
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < kCopies * cells; i += kScThreads) {
        if constexpr (kWord) c64[i] = kEmptyWord<OP>;
        else c32[i] = 0u;
    }
    if constexpr (OP == OP_MEAN)
        for (int64_t i = tid; i < a.dim; i += kScThreads) cnt[i] = 0u;
    __syncthreads();

    const int lane = tid & 63;
    const int lg = a.lg;
    const int64_t G = 64 >> lg;
    const int sub = lane & ((1 << lg) - 1);
    const int64_t stride = (int64_t)gridDim.x * (kScThreads / 64) * kPrivSteps * G;
    for (int64_t qbase = ((int64_t)blockIdx.x * (kScThreads / 64) + (tid >> 6)) * kPrivSteps * G; qbase < a.items;
         qbase += stride) {
        int64_t s[kPrivSteps], fe[kPrivSteps], row[kPrivSteps];
        uint32_t x[kPrivSteps];
#pragma unroll
        for (int u = 0; u < kPrivSteps; ++u) {
            int64_t q = qbase + u * G + (lane >> lg);
            int64_t r = q, f = sub;
            if (a.chunks > 1) {
                q = readfirst(q);  // one item per wave step (64 lanes per item)
                r = q / a.chunks;
                f = (q - r * a.chunks) * 64 + lane;
            }
            const bool live = q < a.items && f < a.F;
            s[u] = live ? a.index[r] : -1;
            x[u] = live ? a.values[r * a.F + f] : 0u;
            fe[u] = f;
            row[u] = r;
        }
        if constexpr (WAVES) {
            uint32_t *mine = c32 + (tid >> 6) * cells;
            const int grp = lane >> lg;
#pragma unroll
            for (int u = 0; u < kPrivSteps; ++u) {
                const bool act = s[u] >= 0 && s[u] < a.dim;
                const int64_t cell = s[u] * a.F + fe[u];
                for (int gg = 0; gg < (int)G; ++gg) {
                    if (grp == gg && act) {
                        if constexpr (DT == DT_F32)
                            mine[cell] = __float_as_uint(__uint_as_float(mine[cell]) + __uint_as_float(x[u]));
                        else
                            mine[cell] += x[u];
                    }
                    // keep the groups' turns apart: a group reads the cells
                    // the previous group of this wave has just written
                    asm volatile("" ::: "memory");
                }
                if constexpr (OP == OP_MEAN) {
                    if (act && fe[u] == 0)
                        __hip_atomic_fetch_add(cnt + s[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
            continue;
        }
#pragma unroll
        for (int u = 0; u < kPrivSteps; ++u) {
            if (s[u] < 0 || s[u] >= a.dim) continue;
            const int64_t cell = s[u] * a.F + fe[u];
            if constexpr (OP == OP_MAX) {
                __hip_atomic_fetch_max(c64 + cell, pack<OP>(okey<DT>(x[u]), row[u]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            } else if constexpr (OP == OP_MIN) {
                __hip_atomic_fetch_min(c64 + cell, pack<OP>(okey<DT>(x[u]), row[u]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            } else if constexpr (DT == DT_F32) {
                __hip_atomic_fetch_add(reinterpret_cast<float *>(c32) + cell, __uint_as_float(x[u]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                __hip_atomic_fetch_add(c32 + cell, x[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if constexpr (OP == OP_MEAN) {
                if (fe[u] == 0) __hip_atomic_fetch_add(cnt + s[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    // the workgroup's copy goes to its own scratch slot with plain stores
    // (global atomics from every workgroup into the same few outputs would
    // serialise at the memory side); scatter_private_fold_a/_b combine them
    if constexpr (kWord) {
        uint64_t *dst = reinterpret_cast<uint64_t *>(a.priv) + blockIdx.x * cells;
        for (int64_t i = tid; i < cells; i += kScThreads) dst[i] = c64[i];
    } else if constexpr (WAVES) {
        uint32_t *dst = a.priv + blockIdx.x * (cells + (OP == OP_MEAN ? a.dim : 0));
        for (int64_t i = tid; i < cells; i += kScThreads) {
            if constexpr (DT == DT_F32) {
                float v = __uint_as_float(c32[i]);
#pragma unroll
                for (int c = 1; c < kCopies; ++c) v += __uint_as_float(c32[c * cells + i]);
                dst[i] = __float_as_uint(v);
            } else {
                uint32_t v = c32[i];
#pragma unroll
                for (int c = 1; c < kCopies; ++c) v += c32[c * cells + i];
                dst[i] = v;
            }
        }
    } else {
        uint32_t *dst = a.priv + blockIdx.x * (cells + (OP == OP_MEAN ? a.dim : 0));
        for (int64_t i = tid; i < cells; i += kScThreads) dst[i] = c32[i];
    }
    if constexpr (OP == OP_MEAN) {
        uint32_t *dst = a.priv + blockIdx.x * (cells + a.dim) + cells;
        for (int64_t i = tid; i < a.dim; i += kScThreads) dst[i] = cnt[i];
    }
}

// Folding the copies.  A workgroup's copy is one row of T columns: the
// output cells (32-bit sums or 64-bit MIN/MAX words), then for MEAN the row
// counts of the dim outputs.  With more than 64 copies, scatter_private_fold_a
// first adds consecutive ranges of `per` copies into 64 partial rows or fewer
// (one wave per 64 columns and range, lanes over consecutive columns, so the
// loads are coalesced); scatter_private_fold_b then folds the remaining rows
// of each cell (one wave per cell, lane l takes rows l, l + 64, ... in order,
// then a fixed tree) and writes the final value: the sum, the mean, or the
// unpacked MIN/MAX value and row.  Every order is fixed, so float sums repeat
// bit for bit.
template <int DT, int OP>
__device__ __forceinline__ uint32_t fold_add(uint32_t acc, uint32_t v, bool count_col) {
    if constexpr (DT == DT_F32) {
        if (!count_col) return __float_as_uint(__uint_as_float(acc) + __uint_as_float(v));
    }
    return acc + v;
}

template <int OP>
__device__ __forceinline__ uint64_t fold_word(uint64_t acc, uint64_t v) {
    return OP == OP_MAX ? (v > acc ? v : acc) : (v < acc ? v : acc);
}

template <int DT, int OP>
__global__ __launch_bounds__(kScThreads) void scatter_private_fold_a(ScArgs a, int64_t nwg, int64_t T, int64_t per,
                                                                     int64_t nparts, uint32_t *part) {
    constexpr bool kWord = OP == OP_MIN || OP == OP_MAX;
    const int lane = threadIdx.x & 63;
    const int64_t cells = a.dim * a.F;
    const int64_t cgroups = (T + 63) / 64;
    const int64_t units = cgroups * nparts;
    for (int64_t u = (int64_t)blockIdx.x * (kScThreads / 64) + (threadIdx.x >> 6); u < units;
         u += (int64_t)gridDim.x * (kScThreads / 64)) {
        const int64_t ch = u / cgroups;
        const int64_t c = (u - ch * cgroups) * 64 + lane;
        if (c >= T) continue;
        const int64_t g0 = ch * per, g1 = g0 + per < nwg ? g0 + per : nwg;
        // loads in batches of 8 ahead of the in-order combine
        constexpr int kB = 8;
        if constexpr (kWord) {
            const uint64_t *src = reinterpret_cast<const uint64_t *>(a.priv);
            uint64_t acc = kEmptyWord<OP>;
            int64_t g = g0;
            for (; g + kB <= g1; g += kB) {
                uint64_t v[kB];
#pragma unroll
                for (int k = 0; k < kB; ++k) v[k] = src[(g + k) * T + c];
#pragma unroll
                for (int k = 0; k < kB; ++k) acc = fold_word<OP>(acc, v[k]);
            }
            for (; g < g1; ++g) acc = fold_word<OP>(acc, src[g * T + c]);
            reinterpret_cast<uint64_t *>(part)[ch * T + c] = acc;
        } else {
            const bool count_col = c >= cells;
            uint32_t acc = 0u;
            int64_t g = g0;
            for (; g + kB <= g1; g += kB) {
                uint32_t v[kB];
#pragma unroll
                for (int k = 0; k < kB; ++k) v[k] = a.priv[(g + k) * T + c];
#pragma unroll
                for (int k = 0; k < kB; ++k) acc = fold_add<DT, OP>(acc, v[k], count_col);
            }
            for (; g < g1; ++g) acc = fold_add<DT, OP>(acc, a.priv[g * T + c], count_col);
            part[ch * T + c] = acc;
        }
    }
}

template <int DT, int OP>
__global__ __launch_bounds__(kScThreads) void scatter_private_fold_b(ScArgs a, const uint32_t *src, int64_t n,
                                                                     int64_t T, int64_t *arg) {
    constexpr bool kWord = OP == OP_MIN || OP == OP_MAX;
    const int lane = threadIdx.x & 63;
    const int64_t cells = a.dim * a.F;
    const int64_t w = (int64_t)blockIdx.x * (kScThreads / 64) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (kScThreads / 64);
    for (int64_t i = w; i < cells; i += nwaves) {
        if constexpr (kWord) {
            const uint64_t *s64 = reinterpret_cast<const uint64_t *>(src);
            uint64_t acc = kEmptyWord<OP>;
            for (int64_t g = lane; g < n; g += 64) acc = fold_word<OP>(acc, s64[g * T + i]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t v = lane_get(acc, (lane + o) & 63);
                if (lane < o) acc = fold_word<OP>(acc, v);
            }
            if (lane == 0) {
                const bool empty = acc == kEmptyWord<OP>;
                const uint32_t code = (uint32_t)acc;
                a.out[i] = empty ? 0u : okey_inv<DT>((uint32_t)(acc >> 32));
                if (arg) arg[i] = empty ? -1 : (int64_t)(OP == OP_MAX ? ~code : code);
            }
        } else {
            uint32_t acc = 0u;
            for (int64_t g = lane; g < n; g += 64) acc = fold_add<DT, OP>(acc, src[g * T + i], false);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint32_t v = lane_get(acc, (lane + o) & 63);
                if (lane < o) acc = fold_add<DT, OP>(acc, v, false);
            }
            if constexpr (OP == OP_MEAN) {
                const int64_t col = cells + i / a.F;
                uint32_t cnt = 0u;
                for (int64_t g = lane; g < n; g += 64) cnt += src[g * T + col];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const uint32_t v = lane_get(cnt, (lane + o) & 63);
                    if (lane < o) cnt += v;
                }
                if (lane == 0) a.out[i] = cnt ? __float_as_uint(__uint_as_float(acc) / (float)cnt) : 0u;
            } else {
                if (lane == 0) a.out[i] = acc;
            }
        }
    }
}

// Final values: MIN/MAX unpack the word (value from its key, row from its
// code; untouched -> 0 and -1); MEAN divides by the row count (0 rows -> 0).
template <int DT, int OP>
__global__ __launch_bounds__(kScThreads) void scatter_finish(ScArgs a, int64_t *arg) {
    const int64_t cells = a.dim * a.F;
    const int64_t stride = (int64_t)gridDim.x * kScThreads;
    for (int64_t c = (int64_t)blockIdx.x * kScThreads + threadIdx.x; c < cells; c += stride) {
        if constexpr (OP == OP_MEAN) {
            const uint32_t n = a.counts[c / a.F];
            const float sum = __uint_as_float(a.out[c]);
            a.out[c] = n ? __float_as_uint(sum / (float)n) : 0u;
        } else {
            const uint64_t w = a.words[c];
            const bool empty = w == kEmptyWord<OP>;
            const uint32_t code = (uint32_t)w;
            a.out[c] = empty ? 0u : okey_inv<DT>((uint32_t)(w >> 32));
            if (arg) arg[c] = empty ? -1 : (int64_t)(OP == OP_MAX ? ~code : code);
        }
    }
}

// ---------------------------------------------------------------- offsets of an index

// Rows per destination, added into counts[s] = offsets[s + 1] (zeroed
// before).  A step's 64 consecutive rows are merged over runs of equal index
// first (run length from the ballot of run heads), so a sorted index costs one
// atomic per run and wave step.
__global__ __launch_bounds__(kScThreads) void index_count(const int64_t *index, int64_t rows, int64_t dim,
                                                          uint64_t *counts) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kScThreads / 64) + (threadIdx.x >> 6);
    const int64_t base = wave * kScSteps * 64;
    int64_t s[kScSteps];
#pragma unroll
    for (int u = 0; u < kScSteps; ++u) {
        const int64_t r = base + u * 64 + lane;
        s[u] = r < rows ? index[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kScSteps; ++u) {
        const int64_t next = lane_get(s[u], (lane + 1) & 63);
        const int64_t prev = lane_get(s[u], (lane - 1) & 63);
        const bool head = lane == 0 || s[u] != prev;
        const bool last = lane == 63 || s[u] != next;
        const uint64_t heads = ballot(head);
        const uint64_t upto = heads & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
        const uint64_t len = (uint64_t)(lane - (63 - __clzll((long long)upto)) + 1);
        if (last && s[u] >= 0 && s[u] < dim)
            __hip_atomic_fetch_add(counts + s[u], len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Tile totals of the counts: tile t covers counts[t * 4096, (t + 1) * 4096).
__global__ __launch_bounds__(kCountThreads) void count_tiles(const int64_t *counts, int64_t dim, int64_t *tsum) {
    __shared__ int64_t s_tmp[2 * (kCountThreads / 64)];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kCountTile;
    int64_t acc = 0;
#pragma unroll
    for (int u = 0; u < kCountTile / kCountThreads; ++u) {
        const int64_t i = t0 + u * kCountThreads + tid;
        acc += i < dim ? counts[i] : 0;
    }
    int64_t total;
    block_inclusive_scan<kCountThreads, false>(acc, s_tmp, total);
    if (tid == 0) tsum[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the tile totals (tile base).
__global__ __launch_bounds__(kCountScanThreads) void count_scan(const int64_t *tsum, int64_t tiles,
                                                                int64_t *tbase) {
    constexpr int K = kCountScanPer;
    constexpr int64_t kBatch = (int64_t)kCountScanThreads * K;
    __shared__ int64_t s_tmp[2 * (kCountScanThreads / 64)];
    const int tid = threadIdx.x;
    int64_t running = 0;
    for (int64_t b = 0; b < tiles; b += kBatch) {
        int64_t v[K], in[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = b + (int64_t)tid * K + j;
            v[j] = t < tiles ? tsum[t] : 0;
        }
        int64_t acc = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            in[j] = acc;
            acc += v[j];
        }
        int64_t total;
        const int64_t ex = block_inclusive_scan<kCountScanThreads, false>(acc, s_tmp, total) - acc;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = b + (int64_t)tid * K + j;
            if (t < tiles) tbase[t] = running + ex + in[j];
        }
        running += total;
    }
}

// Counts -> inclusive sums in place (offsets[s + 1] = rows with index < s + 1).
// The tile goes through LDS so that global reads and writes are coalesced
// while each thread scans 16 consecutive counts.
__global__ __launch_bounds__(kCountThreads) void count_apply(int64_t *counts, int64_t dim, const int64_t *tbase) {
    constexpr int P = kCountTile / kCountThreads;
    __shared__ int64_t s_c[kCountTile];
    __shared__ int64_t s_tmp[2 * (kCountThreads / 64)];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kCountTile;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int64_t i = t0 + u * kCountThreads + tid;
        s_c[u * kCountThreads + tid] = i < dim ? counts[i] : 0;
    }
    __syncthreads();
    int64_t v[P];
    int64_t acc = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        acc += s_c[tid * P + j];
        v[j] = acc;
    }
    int64_t total;
    const int64_t ex = block_inclusive_scan<kCountThreads, false>(acc, s_tmp, total) - acc + tbase[blockIdx.x];
#pragma unroll
    for (int j = 0; j < P; ++j) s_c[tid * P + j] = v[j] + ex;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int64_t i = t0 + u * kCountThreads + tid;
        if (i < dim) counts[i] = s_c[u * kCountThreads + tid];
    }
}

// Compute units of the current device (cached per device; 256 if the query
// fails).
// CUs the private-copy grid is sized for: those of a whole MI355X, a
// constant rather than the current device's count, so the fixed-order float
// sums of that path are the same on every device (a smaller device runs the
// same workgroups in more rounds).
constexpr int64_t kGridCus = 256;

template <int DT, int OP>
int scatter_launch(const ScArgs &a, int64_t *arg, hipStream_t st) {
    const int64_t per_wave = (int64_t)kScSteps * (64 >> a.lg);
    const int64_t waves = (a.items + per_wave - 1) / per_wave;
    const int64_t wgs = (waves + kScThreads / 64 - 1) / (kScThreads / 64);
    if (wgs > INT32_MAX) return SEGRED_ERR_UNSUPPORTED;
    hipError_t e = hipSuccess;
    if (a.priv_grid > 0) {
        const int64_t cells = a.dim * a.F;
        const unsigned lds = (unsigned)a.priv_lds;
        if constexpr (DT == DT_F32 && (OP == OP_SUM || OP == OP_MEAN)) {
            if (a.priv_waves)
                timed_launch_ggl(true, (scatter_private<DT, OP, true>), dim3((unsigned)a.priv_grid),
                                 dim3(kScThreads), lds, st, a);
            else
                timed_launch_ggl(true, (scatter_private<DT, OP, false>), dim3((unsigned)a.priv_grid),
                                 dim3(kScThreads), lds, st, a);
        } else {
            timed_launch_ggl(true, (scatter_private<DT, OP, false>), dim3((unsigned)a.priv_grid), dim3(kScThreads),
                             lds, st, a);
        }
        e = hipGetLastError();
        const int64_t T = cells + (OP == OP_MEAN ? a.dim : 0);
        const uint32_t *rows = a.priv;
        int64_t n = a.priv_grid;
        if (e == hipSuccess && n > 64) {
            const int64_t per = (n + 63) / 64, nparts = (n + per - 1) / per;
            const int64_t units = (T + 63) / 64 * nparts;
            const unsigned ga = (unsigned)std::max<int64_t>(1, std::min<int64_t>((units + 3) / 4, 8192));
            timed_launch_ggl(false, (scatter_private_fold_a<DT, OP>), dim3(ga), dim3(kScThreads), 0, st, a, n, T,
                             per, nparts, a.part);
            e = hipGetLastError();
            rows = a.part;
            n = nparts;
        }
        if (e == hipSuccess) {
            // one wave per output cell
            const unsigned fg = (unsigned)std::max<int64_t>(1, std::min<int64_t>((cells + 3) / 4, 8192));
            timed_launch_ggl(false, (scatter_private_fold_b<DT, OP>), dim3(fg), dim3(kScThreads), 0, st, a, rows, n,
                             T, arg);
            e = hipGetLastError();
        }
        return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
    } else if (wgs > 0) {
        if (a.lg == 0)
            timed_launch_ggl(true, (scatter_kernel<DT, OP, true>), dim3((unsigned)wgs), dim3(kScThreads), 0, st, a);
        else
            timed_launch_ggl(true, (scatter_kernel<DT, OP, false>), dim3((unsigned)wgs), dim3(kScThreads), 0, st, a);
        e = hipGetLastError();
    }
    if (e == hipSuccess && OP != OP_SUM) {
        const int64_t cells = a.dim * a.F;
        const unsigned grid = (unsigned)std::min<int64_t>((cells + kScThreads - 1) / kScThreads, 4096);
        timed_launch_ggl(false, (scatter_finish<DT, OP>), dim3(grid), dim3(kScThreads), 0, st, a, arg);
        e = hipGetLastError();
    }
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

template <int DT>
int scatter_dispatch_op(int op, const ScArgs &a, int64_t *arg, hipStream_t st) {
    switch (op) {
    case OP_SUM: return scatter_launch<DT, OP_SUM>(a, arg, st);
    case OP_MIN: return scatter_launch<DT, OP_MIN>(a, arg, st);
    case OP_MAX: return scatter_launch<DT, OP_MAX>(a, arg, st);
    default:
        if constexpr (DT == DT_F32) return scatter_launch<DT, OP_MEAN>(a, arg, st);
        return SEGRED_ERR_UNSUPPORTED;
    }
}

unsigned fill_grid(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + kScThreads - 1) / kScThreads, 4096)); }

}  // namespace segred

using namespace segred;

extern "C" int segred_scatter_reduce(const void *values, int32_t dtype, int64_t feat, int64_t rows,
                                     const int64_t *index, int64_t dim_size, int32_t op, void *out,
                                     int64_t *arg_out, hipStream_t stream) {
    if (dtype < SEGRED_U32 || dtype > SEGRED_F32 || op < SEGRED_SUM || op > SEGRED_MEAN) return SEGRED_ERR_INVALID_ARGUMENT;
    if (feat < 1 || rows < 0 || dim_size < 0) return SEGRED_ERR_INVALID_ARGUMENT;
    if (dim_size > 0 && feat > INT64_MAX / dim_size) return SEGRED_ERR_INVALID_ARGUMENT;
    if (rows > 0 && feat > INT64_MAX / rows) return SEGRED_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!values || !index)) return SEGRED_ERR_INVALID_ARGUMENT;
    if (dim_size > 0 && !out) return SEGRED_ERR_INVALID_ARGUMENT;
    if ((values && !aligned(values, 4)) || (index && !aligned(index, 8)) || (out && !aligned(out, 4)) ||
        (arg_out && !aligned(arg_out, 8)))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_MEAN && dtype != SEGRED_F32) return SEGRED_ERR_UNSUPPORTED;
    if (op != SEGRED_SUM && rows > (int64_t)0xFFFFFFFE) return SEGRED_ERR_UNSUPPORTED;
    if (dim_size == 0) return SEGRED_OK;

    ScArgs a{};
    a.values = static_cast<const uint32_t *>(values);
    a.index = index;
    a.rows = rows;
    a.F = feat;
    a.dim = dim_size;
    a.chunks = feat > 64 ? (feat + 63) / 64 : 1;
    a.items = rows * a.chunks;
    int lg = 0;
    while ((1 << lg) < std::min<int64_t>(feat, 64)) ++lg;
    a.lg = lg;
    a.out = static_cast<uint32_t *>(out);
    const int64_t cells = dim_size * feat;
    int64_t *arg = (op == SEGRED_MIN || op == SEGRED_MAX) ? arg_out : nullptr;

    // Few outputs: private LDS copies when they fit and there are at least
    // 128 elements per output cell.  Float sums of >= 8 features take it
    // only with one copy per wave: their LDS float atomics run at a fixed
    // rate below that of global atomics spread over thousands of cells.
    // Grid: one workgroup per CU at least, more while the copies stay under
    // an eighth of the input bytes (they are written once and read once by
    // the fold), at most one per item range of the element-atomic grid and
    // no more than fit the chip at once.
    const bool word_op = op == SEGRED_MIN || op == SEGRED_MAX;
    const int64_t count_bytes = op == SEGRED_MEAN ? dim_size * 4 : 0;
    const int64_t priv_bytes = cells * (word_op ? 8 : 4) + count_bytes;  // one copy: T columns
    const int64_t elems = rows * feat;
    const bool float_sum = dtype == SEGRED_F32 && (op == SEGRED_SUM || op == SEGRED_MEAN);
    const bool waves = float_sum && lg >= 3 && cells * 4 * (kScThreads / 64) + count_bytes <= kPrivBytes;
    if (priv_bytes <= kPrivBytes && elems >= 128 * cells && (waves || !float_sum || lg < 3)) {
        a.priv_waves = waves ? 1 : 0;
        a.priv_lds = (int)(waves ? cells * 4 * (kScThreads / 64) + count_bytes : priv_bytes);
        const int64_t per_wave = (int64_t)kScSteps * (64 >> lg);
        const int64_t wgs = ((a.items + per_wave - 1) / per_wave + kScThreads / 64 - 1) / (kScThreads / 64);
        const int64_t cus = kGridCus;
        const int64_t resident = cus * std::min<int64_t>(kWgPerCu, kLdsPerCu / a.priv_lds);
        a.priv_grid = std::max<int64_t>(
            1, std::min<int64_t>({wgs, resident, std::max<int64_t>(cus, elems / (8 * cells))}));
    }

    // MIN/MAX on the element-atomic path: read the word first and skip the
    // atomic when it cannot win, from 32 rows per output on.  Measured on
    // 1M rows into 10,000 outputs: max+row 317 -> 172 us (F = 64), 85 -> 62
    // us (F = 16); at 10 rows per output (1-D into 100,000) the read cost
    // more than it saved (46 -> 53 us).
    a.word_filter = rows / 32 >= dim_size ? 1 : 0;

    // The private path writes every output itself (its fold stores each
    // cell).  The element-atomic path accumulates into zeroed outputs: MIN/MAX
    // words live in arg_out when the caller gives it (8 bytes per cell,
    // unpacked in place), else in scratch; MEAN counts in scratch.
    size_t need = 0;
    if (a.priv_grid == 0) {
        if (word_op && !arg) need = (size_t)cells * 8;
        if (op == SEGRED_MEAN) need = (size_t)dim_size * 4;
    }
    need = (need + 255) & ~size_t(255);
    const size_t copies = (size_t)(a.priv_grid * priv_bytes);
    const size_t parts = a.priv_grid > 64 ? (size_t)(64 * priv_bytes) : 0;
    const size_t priv_need = copies + ((parts + 255) & ~size_t(255));
    ScratchLease scratch;
    if (need + priv_need > 0) {
        const int rc = scratch_acquire(scratch, need + priv_need, stream);
        if (rc != SEGRED_OK) return rc;
    }
    if (a.priv_grid > 0) {
        char *base = static_cast<char *>(scratch.ptr) + need;
        a.priv = reinterpret_cast<uint32_t *>(base);
        a.part = reinterpret_cast<uint32_t *>(base + ((copies + 255) & ~size_t(255)));
    } else if (word_op) {
        a.words = arg ? reinterpret_cast<uint64_t *>(arg) : static_cast<uint64_t *>(scratch.ptr);
        const uint64_t empty = op == SEGRED_MAX ? kEmptyWord<OP_MAX> : kEmptyWord<OP_MIN>;
        timed_launch_ggl(false, scatter_init, dim3(fill_grid(cells)), dim3(kScThreads), 0, stream,
                         (uint32_t *)nullptr, (int64_t)0, 0u, a.words, cells, empty);
    } else {
        if (op == SEGRED_MEAN) a.counts = static_cast<uint32_t *>(scratch.ptr);
        timed_launch_ggl(false, scatter_init, dim3(fill_grid(cells)), dim3(kScThreads), 0, stream, a.out, cells, 0u,
                         (uint64_t *)nullptr, (int64_t)0, 0ull);
        if (op == SEGRED_MEAN && hipGetLastError() == hipSuccess)
            timed_launch_ggl(false, scatter_init, dim3(fill_grid(dim_size)), dim3(kScThreads), 0, stream, a.counts,
                             dim_size, 0u, (uint64_t *)nullptr, (int64_t)0, 0ull);
    }
    if (hipGetLastError() != hipSuccess) return SEGRED_ERR_HIP;
    switch (dtype) {
    case SEGRED_U32: return scatter_dispatch_op<DT_U32>(op, a, arg, stream);
    case SEGRED_I32: return scatter_dispatch_op<DT_I32>(op, a, arg, stream);
    default: return scatter_dispatch_op<DT_F32>(op, a, arg, stream);
    }
}

extern "C" int segred_offsets_from_index(const int64_t *index, int64_t rows, int64_t dim_size, int64_t *offsets,
                                         hipStream_t stream) {
    if (rows < 0 || dim_size < 0 || !offsets || (rows > 0 && !index)) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!aligned(offsets, 8) || (index && !aligned(index, 8))) return SEGRED_ERR_INVALID_ARGUMENT;
    const int64_t per_wg = (int64_t)kScSteps * 64 * (kScThreads / 64);
    const int64_t wgs = (rows + per_wg - 1) / per_wg;
    const int64_t tiles = (dim_size + kCountTile - 1) / kCountTile;
    if (wgs > INT32_MAX || tiles > INT32_MAX) return SEGRED_ERR_UNSUPPORTED;

    ScratchLease scratch;
    if (tiles > 0) {
        const int rc = scratch_acquire(scratch, (size_t)tiles * 2 * sizeof(int64_t), stream);
        if (rc != SEGRED_OK) return rc;
    }
    int64_t *tsum = static_cast<int64_t *>(scratch.ptr);
    int64_t *tbase = tsum + tiles;
    int64_t *counts = offsets + 1;

    timed_launch_ggl(false, scatter_init, dim3(fill_grid(dim_size + 1)), dim3(kScThreads), 0, stream,
                     (uint32_t *)nullptr, (int64_t)0, 0u, reinterpret_cast<uint64_t *>(offsets), dim_size + 1, 0ull);
    if (wgs > 0 && dim_size > 0)
        timed_launch_ggl(true, index_count, dim3((unsigned)wgs), dim3(kScThreads), 0, stream, index, rows, dim_size,
                         reinterpret_cast<uint64_t *>(counts));
    if (tiles > 0) {
        timed_launch_ggl(false, count_tiles, dim3((unsigned)tiles), dim3(kCountThreads), 0, stream,
                         (const int64_t *)counts, dim_size, tsum);
        timed_launch_ggl(false, count_scan, dim3(1), dim3(kCountScanThreads), 0, stream, (const int64_t *)tsum,
                         tiles, tbase);
        timed_launch_ggl(false, count_apply, dim3((unsigned)tiles), dim3(kCountThreads), 0, stream, counts, dim_size,
                         (const int64_t *)tbase);
    }
    return hipGetLastError() == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}
