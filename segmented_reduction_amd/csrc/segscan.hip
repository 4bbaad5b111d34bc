// segscan.hip -- segmented inclusive / exclusive scan over offset-delimited
// segments on gfx950.
//
// Operation (GPUSegmentedScan, named by the luma.gl "GPURunLengthEncode and
// GPUUnique" page, "Composition", beside GPUSegmentedReduction; read with
// the segmented reduction's contract from the "GPUSegmentedReduction" page:
// segment s owns rows [offsets[s], offsets[s+1]), uint32 / int32 / float32
// values, sum / min / max): for row r of segment s,
//   inclusive  out[r, f] = op of values[offsets[s] .. r, f]
//   exclusive  out[r, f] = op of values[offsets[s] .. r-1, f], 0 at the
//              segment's first row (an empty prefix gives 0, as an empty
//              segment does in the reduction).
// Rows outside [offsets[0], offsets[S]) are not written.
//
// Work partition: the merge-path shares of the segmented reduction (rows +
// segment ends, a constant number of shares: one per wave of a whole
// MI355X; partition.hpp), with each share
// boundary moved onto a nearby segment boundary when one lies within a
// quarter share, so only segments longer than that are cut.  Two launches:
//   seg_scan_tails  per share, the partial of the segment the share leaves
//                   open at its end, over the share's rows of that segment
//                   only (so a share of short segments reads few rows), and
//                   a record of the share's coordinates;
//   seg_scan_main   per share, the carry into its first segment (the tails
//                   of the preceding shares that segment spans, folded in a
//                   fixed order), then the share's rows in steps of 64 lanes:
//                   segment starts from the offsets as a bit mask per step,
//                   a per-lane scan of its elements, a segmented scan across
//                   the step's row groups, outputs stored in the input
//                   layout.
// Feature blocks beyond 64 run as further waves on the same shares.  Float
// sums accumulate in float64 throughout (each output is one rounding of a
// float64 prefix), integer sums wrap modulo 2^32, min/max run on the
// monotone order key.  Every order is a fixed function of the offsets and
// the share count, so results repeat bit for bit; no atomic operations.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "internal.hpp"
#include "keys.hpp"
#include "partition.hpp"
#include "wave.hpp"

namespace segred {

struct ScanArgs {
    const uint32_t *values;  // element bits, row-major [rows, F]
    const int64_t *offsets;  // [S + 1]
    int64_t S, F, NW, chunks;  // chunks: 64-feature blocks per row
    uint32_t *out;             // [rows, F], same layout as values
    int64_t *rec;              // [NW][8] share records (see seg_scan_tails)
    uint64_t *tval;            // [NW][F] tail partials
};

template <int DT, int OP>
struct ScanOp {
    static constexpr bool kF64 = DT == DT_F32 && OP == OP_SUM;
    using acc_t = std::conditional_t<kF64, double, uint32_t>;
    static __device__ __forceinline__ acc_t id() {
        if constexpr (kF64) return 0.0;
        else if constexpr (OP == OP_MIN) return 0xFFFFFFFFu;
        else return 0u;
    }
    static __device__ __forceinline__ acc_t lift(uint32_t b) {
        if constexpr (kF64) return (double)__uint_as_float(b);
        else if constexpr (OP == OP_SUM) return b;
        else return okey<DT>(b);
    }
    static __device__ __forceinline__ acc_t comb(acc_t a, acc_t b) {
        if constexpr (OP == OP_SUM) return a + b;
        else if constexpr (OP == OP_MIN) return b < a ? b : a;
        else return b > a ? b : a;
    }
    static __device__ __forceinline__ uint32_t lower(acc_t a) {
        if constexpr (kF64) return __float_as_uint((float)a);
        else if constexpr (OP == OP_SUM) return a;
        else return okey_inv<DT>(a);
    }
    static __device__ __forceinline__ uint64_t word(acc_t a) {
        if constexpr (kF64) return (uint64_t)__double_as_longlong(a);
        else return a;
    }
    static __device__ __forceinline__ acc_t unword(uint64_t w) {
        if constexpr (kF64) return __longlong_as_double((long long)w);
        else return (uint32_t)w;
    }
};

// Share record: [i0, j0, i1, j1, first_row, tail_row, o0, flags], rows
// relative to offsets[0]; flags bit 0: the share's last segment continues
// past it; bit 1: that segment starts inside the share.
constexpr int kRec = 8;

// The shares are sized by the main kernel's occupancy (up to 8 waves per
// SIMD); the tails kernel is held to the same (64 registers, smaller load
// batches) so that all its shares run in one round rather than two.
template <int DT, int OP, int L>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
void seg_scan_tails(const ScanArgs a) {
    using O = ScanOp<DT, OP>;
    using acc_t = typename O::acc_t;
    constexpr int G = 64 / L;
    constexpr int U = L == 1 ? 4 : 16;
    __shared__ int64_t s_probe[kProbesA];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t sblocks = a.NW / 4;
    const int64_t chunk = blockIdx.x / sblocks;
    const int64_t share = (int64_t)(blockIdx.x % sblocks) * 4 + wid;
    const Share sh = find_share<true>(a.offsets, a.S, a.NW, share, lane, s_probe);
    if (chunk == 0 && lane == 0) {
        int64_t *r = a.rec + share * kRec;
        r[0] = sh.i0;
        r[1] = sh.j0;
        r[2] = sh.i1;
        r[3] = sh.j1;
        r[4] = sh.first_row;
        r[5] = sh.tail_row;
        r[6] = sh.o0;
        r[7] = (sh.has_tail ? 1 : 0) | (sh.has_tail && sh.tail_row >= sh.j0 ? 2 : 0);
    }
    if (!sh.has_tail) return;
    const int g = lane / L, c = lane % L;
    const int64_t f = chunk * 64 + c;
    const bool fv = f < a.F;
    const int64_t ta = max(sh.tail_row, sh.j0);
    acc_t acc = O::id();
    // The tail streams in batches, the next fetched before the current one is
    // added (a batch past the tail gets an empty descriptor: its loads return
    // 0 without touching memory and are not added).
    if constexpr (L == 1) {
        // 1-D: 16-byte loads, 4 consecutive elements per lane
        constexpr int64_t E = 64 * 4 * U;
        auto fetch = [&](int64_t rb, uint4 (&q)[U]) __attribute__((always_inline)) {
            const int64_t n = max((int64_t)0, min(E, sh.j1 - rb));
            const auto rs = make_rsrc(a.values + sh.o0 + rb, (uint32_t)(n * 4));
#pragma unroll
            for (int u = 0; u < U; ++u) q[u] = ld128(rs, (uint32_t)(lane * 16 + u * 1024));
        };
        auto add = [&](int64_t rb, const uint4 (&q)[U]) __attribute__((always_inline)) {
            const int64_t n = min(E, sh.j1 - rb);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e = (int64_t)u * 256 + lane * 4;
                if (e + 0 < n) acc = O::comb(acc, O::lift(q[u].x));
                if (e + 1 < n) acc = O::comb(acc, O::lift(q[u].y));
                if (e + 2 < n) acc = O::comb(acc, O::lift(q[u].z));
                if (e + 3 < n) acc = O::comb(acc, O::lift(q[u].w));
            }
        };
        uint4 qa[U], qb[U];
        fetch(ta, qa);
        for (int64_t rb = ta; rb < sh.j1; rb += 2 * E) {
            fetch(rb + E, qb);
            add(rb, qa);
            if (rb + E >= sh.j1) break;
            fetch(rb + 2 * E, qa);
            add(rb + E, qb);
        }
    } else {
        constexpr int64_t E = (int64_t)G * U;
        const uint32_t row_bytes = (uint32_t)(a.F * 4);
        auto fetch = [&](int64_t rb, uint32_t (&x)[U]) __attribute__((always_inline)) {
            const int64_t n = max((int64_t)0, min(E, sh.j1 - rb));
            const auto rs = make_rsrc(a.values + (sh.o0 + rb) * a.F + chunk * 64,
                                      n > 0 ? (uint32_t)(n * a.F - chunk * 64) * 4u : 0u);
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = ld32(rs, (uint32_t)((g * a.F + c) * 4) + (uint32_t)u * (uint32_t)G * row_bytes);
        };
        auto add = [&](int64_t rb, const uint32_t (&x)[U]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t r = rb + (int64_t)u * G + g;
                if (r < sh.j1 && fv) acc = O::comb(acc, O::lift(x[u]));
            }
        };
        uint32_t xa[U], xb[U];
        fetch(ta, xa);
        for (int64_t rb = ta; rb < sh.j1; rb += 2 * E) {
            fetch(rb + E, xb);
            add(rb, xa);
            if (rb + E >= sh.j1) break;
            fetch(rb + 2 * E, xa);
            add(rb + E, xb);
        }
    }
    // groups in a fixed tree: lane l takes lane l + o, for o = 32 .. L
#pragma unroll
    for (int o = 32; o >= L; o >>= 1) {
        const acc_t y = lane_get(acc, (lane + o) & 63);
        if (lane < o) acc = O::comb(acc, y);
    }
    if (lane < L && fv) a.tval[share * a.F + f] = O::word(acc);
}

// Step of SR = G * V rows: lane (g, c) holds feature c of rows
// rb + g * V .. rb + g * V + V - 1 (V > 1 only for 1-D values, L = 1).
// Held to 8 waves per SIMD (64 registers): the 1-D variants used 66, which
// left 7 waves and 12.5 % fewer shares (50M 1-D: 140 -> 132-135 us).
template <int DT, int OP, bool EXCL, int L, int V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void seg_scan_main(const ScanArgs a) {
    using O = ScanOp<DT, OP>;
    using acc_t = typename O::acc_t;
    constexpr int G = 64 / L;
    constexpr int SR = G * V;
    // loads per batch: 16 for rows of 64 lanes; narrower rows keep 8, which
    // fits their group scan in the 64 registers of 8 waves per SIMD
    constexpr int U = V == 1 ? (L == 64 ? 16 : 8) : 4;
    static_assert(V == 1 || L == 1, "several rows per lane only for 1-D values");
    static_assert(SR <= 256, "step masks hold 256 rows");

    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __shared__ uint32_t s_sm[4][8];  // per wave: start flags of a 1-D step (256 rows)
    uint32_t *sm = s_sm[wid];
    const int64_t sblocks = a.NW / 4;
    const int64_t chunk = blockIdx.x / sblocks;
    const int64_t share = readfirst((int64_t)(blockIdx.x % sblocks) * 4 + wid);
    const int64_t *rec = a.rec + share * kRec;
    const int64_t i0 = readfirst(rec[0]), j0 = readfirst(rec[1]), j1 = readfirst(rec[3]);
    const int64_t first_row = readfirst(rec[4]), o0 = readfirst(rec[6]);
    if (j0 >= j1) return;
    const int g = lane / L, c = lane % L;
    const int64_t fbase = chunk * 64;
    const int64_t f = fbase + c;
    const bool fv = f < a.F;

    // Carry into the share's first segment when it began in an earlier
    // share: find the share where it began (lanes look at 64 shares at a
    // time), then fold the tails of that share and all later ones before
    // this one; group g takes shares ws + g, ws + g + G, ...; the groups
    // combine in a fixed tree.
    acc_t carry = O::id();
    if (first_row < j0) {
        int64_t ws = share - 1;
        for (;;) {
            const int64_t w = ws - lane;
            const int64_t fl = a.rec[(w < 0 ? 0 : w) * kRec + 7];
            const uint64_t m = ballot(w <= 0 || (fl & 2));
            if (m) {
                ws -= (int64_t)__builtin_ctzll(m);
                break;
            }
            ws -= 64;
        }
        ws = readfirst(ws < 0 ? (int64_t)0 : ws);
        acc_t part = O::id();
        for (int64_t w = ws + g; w < share; w += G)
            if (fv) part = O::comb(part, O::unword(a.tval[w * a.F + f]));
#pragma unroll
        for (int o = 32; o >= L; o >>= 1) {
            const acc_t y = lane_get(part, (lane + o) & 63);
            if (lane < o) part = O::comb(part, y);
        }
        carry = lane_get(part, c);
    }

    // Segment starts: segments kp, kp + 1, ... start at offsets[k] - o0; a
    // batch of 64 of them sits in the lanes (bst0) with the next batch
    // already loaded (bst1).
    int64_t kp = first_row >= j0 ? i0 : i0 + 1;
    int64_t kb = kp;
    const int64_t S = a.S;
    int64_t bst0 = a.offsets[min(kb + lane, S)] - o0;
    int64_t bst1 = a.offsets[min(kb + 64 + lane, S)] - o0;

    const uint32_t row_bytes = (uint32_t)(a.F * 4);
    // Batches of U steps; the next batch is fetched before the current one
    // is processed (a batch past the share gets an empty descriptor: its
    // loads return 0 without touching memory, so every fetch is issued
    // unconditionally).
    constexpr int64_t B = (int64_t)U * SR;
    auto batch_bytes = [&](int64_t rb0) __attribute__((always_inline)) -> uint32_t {
        const int64_t nrows = min(B, j1 - rb0);
        return nrows > 0 ? (uint32_t)(nrows * a.F - fbase) * 4u : 0u;
    };
    auto fetch = [&](int64_t rb0, uint32_t (&x)[U][V]) __attribute__((always_inline)) {
        const auto rin = make_rsrc(a.values + (o0 + rb0) * a.F + fbase, batch_bytes(rb0));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (V == 4) {
                const uint4 q = ld128(rin, (uint32_t)(lane * 16 + u * SR * 4));
                x[u][0] = q.x;
                x[u][1] = q.y;
                x[u][2] = q.z;
                x[u][3] = q.w;
            } else {
                x[u][0] = ld32(rin, (uint32_t)((g * a.F + c) * 4) + (uint32_t)u * (uint32_t)G * row_bytes);
            }
        }
    };
    auto process = [&](int64_t rb0, const uint32_t (&x)[U][V]) __attribute__((always_inline)) {
        const auto rout = make_rsrc(a.out + (o0 + rb0) * a.F + fbase, batch_bytes(rb0));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t rb = rb0 + (int64_t)u * SR;
            if (rb >= j1) break;
            // start flags of rows [rb, min(rb + SR, j1)), one bit per element
            const int64_t lim = min(rb + SR, j1);
            uint32_t fl;
            if constexpr (V == 4) {
                // Each lane of the batch whose start lies in the step sets
                // its row's bit in the wave's 256-bit mask in LDS (bit-OR:
                // starts of empty segments share a row); a ballot counts
                // them.  The batch moves on once all 64 are used.  (A scalar
                // walk over the starts, two readlanes and a 64-bit OR per
                // start, cost about 150 scalar instructions per step.)
                if (lane < SR / 32) sm[lane] = 0u;
                wave_lds_sync();
                for (;;) {
                    const int used = (int)(kp - kb);  // starts of the batch already placed (0..64)
                    const bool in = lane >= used && bst0 < lim;
                    if (in) {
                        const uint32_t p = (uint32_t)(bst0 - rb);
                        lds_or(&sm[p >> 5], 1u << (p & 31));
                    }
                    kp += popc64(ballot(in));
                    if (kp - kb < 64) break;
                    kb += 64;
                    bst0 = bst1;
                    bst1 = a.offsets[min(kb + 64 + lane, S)] - o0;
                }
                wave_lds_sync();
                fl = (sm[lane >> 3] >> ((lane & 7) * 4)) & 0xFu;
            } else {
                uint64_t m0 = 0;
                for (;;) {
                    if (kp > S) break;
                    if (kp - kb >= 64) {
                        kb += 64;
                        bst0 = bst1;
                        bst1 = a.offsets[min(kb + 64 + lane, S)] - o0;
                        continue;
                    }
                    const int64_t e = readlane64(bst0, (int)(kp - kb));
                    if (e >= lim) break;
                    m0 |= 1ull << (int)(e - rb);
                    ++kp;
                }
                fl = (uint32_t)(m0 >> g) & 1u;
            }
            // per-lane scan with resets at starts
            acc_t p[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const acc_t xv = O::lift(x[u][v]);
                p[v] = (v == 0 || ((fl >> v) & 1u)) ? xv : O::comb(p[v - 1], xv);
            }
            // segmented scan of (lane total, lane has a start) across groups
            // (1-D: across all 64 lanes, by DPP)
            acc_t T = p[V - 1];
            bool has = fl != 0;
            if constexpr (L == 1) {
                seg_scan_wave(T, has, O::id(), [](acc_t a, acc_t b) { return O::comb(a, b); });
            } else {
#pragma unroll
                for (int o = L; o < 64; o <<= 1) {
                    const acc_t y = lane_get(T, (lane - o) & 63);
                    const bool yh = lane_get(has, (lane - o) & 63);
                    if (lane >= o && !has) {
                        T = O::comb(y, T);
                        has = yh;
                    }
                }
            }
            const acc_t lane_incl = has ? T : O::comb(carry, T);
            acc_t prev;
            if constexpr (L == 1) prev = dpp_move<kDppWaveShr1>(O::id(), lane_incl);
            else prev = lane_get(lane_incl, (lane - L) & 63);
            const acc_t E = g == 0 ? carry : prev;  // everything before this lane's first element
            uint32_t ob[V];
            acc_t q = E;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const bool st = (fl >> v) & 1u;
                const acc_t incl = (fl & ((2u << v) - 1u)) ? p[v] : O::comb(E, p[v]);
                if constexpr (EXCL) ob[v] = st ? 0u : O::lower(q);
                else ob[v] = O::lower(incl);
                q = incl;
            }
            carry = lane_get(lane_incl, (G - 1) * L + c);
            // store: whole steps with 16-byte stores, the share's last step
            // one dword at a time (each checked against the share's end)
            if constexpr (V == 4) {
                const uint32_t so = (uint32_t)(u * SR * 4);
                if (rb + SR <= j1) {
                    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
                    const v4u d = {ob[0], ob[1], ob[2], ob[3]};
                    __builtin_amdgcn_raw_buffer_store_b128(d, rout, (int)(lane * 16 + so), 0, 0);
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        __builtin_amdgcn_raw_buffer_store_b32(ob[v], rout, (int)(lane * 16 + v * 4 + so), 0, 0);
                }
            } else {
                if (fv)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        ob[0], rout, (int)((uint32_t)((g * a.F + c) * 4) + (uint32_t)u * (uint32_t)G * row_bytes), 0, 0);
            }
        }
    };
    uint32_t xa[U][V], xb[U][V];
    fetch(j0, xa);
    for (int64_t rb0 = j0; rb0 < j1; rb0 += 2 * B) {
        fetch(rb0 + B, xb);
        process(rb0, xa);
        if (rb0 + B >= j1) break;
        fetch(rb0 + 2 * B, xa);
        process(rb0 + B, xb);
    }
}

// ------------------------------------------------------------------ host side

constexpr int64_t kScanMaxFeat = int64_t(1) << 24;

static int scan_lanes(int64_t feat) {
    if (feat == 1) return 1;
    int64_t l = 2;
    while (l < feat && l < 64) l <<= 1;
    return (int)l;
}

template <int DT, int OP, bool EXCL>
static std::pair<const void *, const void *> scan_kernels(int64_t feat) {
    switch (scan_lanes(feat)) {
    case 1: return {(const void *)&seg_scan_tails<DT, OP, 1>, (const void *)&seg_scan_main<DT, OP, EXCL, 1, 4>};
    case 2: return {(const void *)&seg_scan_tails<DT, OP, 2>, (const void *)&seg_scan_main<DT, OP, EXCL, 2, 1>};
    case 4: return {(const void *)&seg_scan_tails<DT, OP, 4>, (const void *)&seg_scan_main<DT, OP, EXCL, 4, 1>};
    case 8: return {(const void *)&seg_scan_tails<DT, OP, 8>, (const void *)&seg_scan_main<DT, OP, EXCL, 8, 1>};
    case 16: return {(const void *)&seg_scan_tails<DT, OP, 16>, (const void *)&seg_scan_main<DT, OP, EXCL, 16, 1>};
    case 32: return {(const void *)&seg_scan_tails<DT, OP, 32>, (const void *)&seg_scan_main<DT, OP, EXCL, 32, 1>};
    default: return {(const void *)&seg_scan_tails<DT, OP, 64>, (const void *)&seg_scan_main<DT, OP, EXCL, 64, 1>};
    }
}

// Shares per call: one per wave of the main kernel on a whole MI355X (256
// CUs x 4 SIMDs x the 8 waves per SIMD both kernels are built for), a
// constant, so the fixed-order float sums do not depend on the device (a
// smaller device runs the same shares in more rounds).
constexpr int64_t kScanShares = 256 * 4 * 8;
static int64_t scan_shares() {
    const int64_t o = shares_override();
    return o > 0 ? (o + 3) / 4 * 4 : kScanShares;
}

template <int DT, int OP, bool EXCL>
static int scan_run(ScanArgs k, hipStream_t st) {
    const auto kern = scan_kernels<DT, OP, EXCL>(k.F);
    const int64_t nw = scan_shares();
    k.NW = nw;
    k.chunks = (k.F + 63) / 64;
    const size_t rec_bytes = (size_t)nw * kRec * sizeof(int64_t);
    ScratchLease scratch;
    int rc = scratch_acquire(scratch, rec_bytes + (size_t)nw * (size_t)k.F * sizeof(uint64_t), st);
    if (rc != SEGRED_OK) return rc;
    k.rec = static_cast<int64_t *>(scratch.ptr);
    k.tval = reinterpret_cast<uint64_t *>(static_cast<char *>(scratch.ptr) + rec_bytes);
    const int64_t blocks = nw / 4 * k.chunks;
    if (blocks > INT32_MAX) return SEGRED_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)blocks), block(256);
    void *params[] = {&k};
    hipError_t e = timed_launch(true, kern.first, grid, block, params, 0, st);
    if (e == hipSuccess)
        e = timed_launch(true, kern.second, grid, block, params, 0, st);
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

template <int DT, int OP>
static int scan_excl(bool excl, const ScanArgs &k, hipStream_t st) {
    return excl ? scan_run<DT, OP, true>(k, st) : scan_run<DT, OP, false>(k, st);
}

template <int DT>
static int scan_op(int op, bool excl, const ScanArgs &k, hipStream_t st) {
    switch (op) {
    case OP_SUM: return scan_excl<DT, OP_SUM>(excl, k, st);
    case OP_MIN: return scan_excl<DT, OP_MIN>(excl, k, st);
    default: return scan_excl<DT, OP_MAX>(excl, k, st);
    }
}

}  // namespace segred

using namespace segred;

extern "C" int segred_scan(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                           int64_t num_segments, int32_t op, int32_t exclusive, void *out, hipStream_t stream) {
    if (num_segments < 0 || feat < 1) return SEGRED_ERR_INVALID_ARGUMENT;
    if (dtype < SEGRED_U32 || dtype > SEGRED_F32 || op < SEGRED_SUM || op > SEGRED_MEAN)
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_MEAN) return SEGRED_ERR_UNSUPPORTED;
    if (feat > kScanMaxFeat) return SEGRED_ERR_UNSUPPORTED;
    if (num_segments == 0) return SEGRED_OK;
    if (!values || !offsets || !out) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!aligned(values, 4) || !aligned(out, 4) || !aligned(offsets, 8)) return SEGRED_ERR_INVALID_ARGUMENT;
    ScanArgs k{};
    k.values = static_cast<const uint32_t *>(values);
    k.offsets = offsets;
    k.S = num_segments;
    k.F = feat;
    k.out = static_cast<uint32_t *>(out);
    const bool ex = exclusive != 0;
    switch (dtype) {
    case SEGRED_U32: return scan_op<DT_U32>(op, ex, k, stream);
    case SEGRED_I32: return scan_op<DT_I32>(op, ex, k, stream);
    default: return scan_op<DT_F32>(op, ex, k, stream);
    }
}
