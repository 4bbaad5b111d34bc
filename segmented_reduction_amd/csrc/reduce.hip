// reduce.hip -- segmented reduction over offset-delimited segments on gfx950.
//
// Operation (luma.gl "GPUSegmentedReduction": "What is an offset-delimited
// segment?", "What is segmented reduction?", "Contract"; graph-reduce README:
// "API", "Method", "Correctness"): out[s, f] = sum / min / max / mean of
// values[r, f] over rows r in [offsets[s], offsets[s+1]); min and max also
// give the lowest producing row; an empty segment gives 0 (and row -1).
//
// Work partition.  The rows and the segment ends are merged into one
// sequence (a segment's rows, then its end), the merge-path view of
// Merrill & Garland's merge-based SpMV that the graph-reduce README cites.
// The sequence is cut into NW equal shares, one per wave (NW is a constant
// of each kernel: one share per wave of a whole MI355X); the four waves of
// a workgroup find their shares' (segment, row) coordinates with a joint
// search over the offsets.  Long or skewed segments are therefore spread
// over many waves instead of serialising on one.
//
// Inside a share:
//  - rows of 32 features with 16-byte access (seg_reduce_team): the
//    wave's share is cut again into equal parts, one per team of L lanes
//    (one row), and each team walks its part row by row with its own
//    accumulators and queue of segment ends; the teams' partials of cut
//    segments are folded in team order at the end;
//  - all other rows (seg_reduce_rows): the wave walks chunks of G groups x V
//    consecutive rows; a group walks its rows in order, finishing every
//    segment that ends inside it, and a segmented scan over the groups
//    completes the segments cut by group and chunk boundaries;
//  - 1-D values (seg_reduce_flat): a chunk is 2048 elements staged through
//    LDS, 32 consecutive ones per lane, reduced by one branch-free pass per
//    lane over reset masks and a DPP segmented scan across the lanes.
// Segments cut by a share boundary leave one partial per share in scratch; a
// second kernel combines them in share order.  Every summation order is a
// fixed function of the offsets, so results repeat bit for bit on any
// device; no atomic operation touches global memory (the 1-D kernel's reset
// masks are built with a bit-OR in LDS, whose result does not depend on
// arrival order).
//
// Memory: rows are read through buffer descriptors whose range ends with the
// valid rows (reads past it return 0, so no clamping), with the non-temporal
// hint, and the next rows stream into registers while the current ones are
// processed.
//
// Accumulators: float sums in float64 (rounded to float32 once; the 1-D
// kernel adds runs of <= 32 elements and a 64-way tree of them in float32
// first), integer sums in wrapping uint32, min/max as a 64-bit word (order
// key << 32 | row code) whose integer max/min picks the extremum and, on
// equal keys, the lowest row (the packed value/row word of the graph-reduce
// README's "Method"); the team walk, which meets a piece's rows in order,
// steps on the 32-bit key alone with the row kept beside it and packs the
// same word for its partials and results.
#include <mutex>
#include <type_traits>

#include "internal.hpp"
#include "keys.hpp"
#include "partition.hpp"
#include "wave.hpp"

namespace segred {

struct KArgs {
    const uint32_t *values;  // element bits, row-major [rows, F]
    const int64_t *offsets;  // [S + 1]
    int64_t S, F;            // S: segment count, or the capacity when S_dev is set
    int64_t NW;              // waves of the streaming kernel (one merge-path share each)
    int64_t NS;              // shares the combine kernel sees: NW, or NW * teams per wave
    const int64_t *S_dev;    // segment count on the device (min(*S_dev, S) is used), or null
    uint32_t *out;           // [S, F]
    int64_t *arg;            // [S, F] or null
    int64_t *hdr;            // [NS][4]: see write_header
    uint64_t *hval;          // [NS][F]: partial of the share's first segment when it began earlier
    uint64_t *tval;          // [NS][F]: partial of the share's last segment when it continues
};

// The call's segment count: the host value, or the device one clamped to it.
__device__ __forceinline__ int64_t seg_count(const KArgs &a) {
    if (!a.S_dev) return a.S;
    const int64_t s = *a.S_dev;
    return s < 0 ? 0 : (s < a.S ? s : a.S);
}

template <int DT, int OP>
struct Red {
    static constexpr bool kSumF = DT == DT_F32 && (OP == OP_SUM || OP == OP_MEAN);
    static constexpr bool kSumI = DT != DT_F32 && OP == OP_SUM;
    static constexpr bool kMinMax = OP == OP_MIN || OP == OP_MAX;
    using acc_t = std::conditional_t<kSumF, double, std::conditional_t<kSumI, uint32_t, uint64_t>>;

    __device__ static __forceinline__ acc_t id() {
        if constexpr (kSumF) return 0.0;
        else if constexpr (kSumI) return 0u;
        else return OP == OP_MAX ? 0ull : ~0ull;
    }
    // One element; `rel` is its row relative to the first row of the share.
    __device__ static __forceinline__ acc_t lift(uint32_t bits, uint32_t rel) {
        if constexpr (kSumF) return (double)__uint_as_float(bits);
        else if constexpr (kSumI) return bits;
        else {
            const uint64_t k = (uint64_t)okey<DT>(bits) << 32;
            return OP == OP_MAX ? (k | (uint32_t)~rel) : (k | rel);
        }
    }
    // Combine an earlier part `a` with a later part `b`.
    __device__ static __forceinline__ acc_t comb(acc_t a, acc_t b) {
        if constexpr (kSumF || kSumI) return a + b;
        else if constexpr (OP == OP_MAX) return a > b ? a : b;
        else return a < b ? a : b;
    }
    __device__ static __forceinline__ uint64_t to_slot(acc_t a) {
        if constexpr (kSumF) return (uint64_t)__double_as_longlong(a);
        else return (uint64_t)a;
    }
    __device__ static __forceinline__ acc_t from_slot(uint64_t s) {
        if constexpr (kSumF) return __longlong_as_double((long long)s);
        else if constexpr (kSumI) return (uint32_t)s;
        else return s;
    }
    // Row code of a packed min/max word; 0xFFFFFFFF marks "no row yet".
    __device__ static __forceinline__ uint32_t rel_of(uint64_t p) {
        return OP == OP_MAX ? ~(uint32_t)p : (uint32_t)p;
    }
    // Min/max walked in row order: the word a piece (a run of consecutive
    // rows of one segment) starts from, the identity key with the piece's
    // first row.  An element then replaces the word only when its key is
    // strictly better (a 32-bit compare), so equal keys keep the earliest
    // row, and a piece whose keys all equal the identity key ends on its
    // first row -- the same word as folding lift() over the piece with
    // comb().  A piece without rows must be turned back into id().
    __device__ static __forceinline__ uint64_t piece_start(uint32_t rel) {
        return OP == OP_MAX ? (uint64_t)(uint32_t)~rel : (0xFFFFFFFFull << 32) | rel;
    }
    __device__ static __forceinline__ uint32_t code_of(uint32_t rel) { return OP == OP_MAX ? ~rel : rel; }
    __device__ static __forceinline__ void step(uint64_t &w, uint32_t bits, uint32_t code) {
        const uint32_t k = okey<DT>(bits), wk = (uint32_t)(w >> 32);
        const bool better = OP == OP_MAX ? k > wk : k < wk;
        // the new key by max/min, which does not wait for the compare
        const uint32_t nk = OP == OP_MAX ? max(k, wk) : min(k, wk);
        w = ((uint64_t)nk << 32) | (better ? code : (uint32_t)w);
    }
};

// The same partial with its row code counted from `delta` rows earlier.
template <typename acc_t>
__device__ __forceinline__ acc_t rebase_word(acc_t p, uint32_t delta, bool is_max) {
    if constexpr (std::is_same_v<acc_t, uint64_t>) {
        const uint32_t rel = is_max ? ~(uint32_t)p : (uint32_t)p;
        if (rel == 0xFFFFFFFFu) return p;
        const uint32_t r2 = rel + delta;
        return (p & 0xFFFFFFFF00000000ull) | (is_max ? ~r2 : r2);
    } else {
        return p;
    }
}

// Waves per SIMD that each streaming kernel is built for (the compiler keeps
// its registers within 512 / W per lane), and so the share count of a call:
// one share per wave of a whole MI355X, 256 CUs x 4 SIMDs x W.  The count is
// a constant of the kernel, not of the device the call runs on, so every
// summation order -- and with it every float result -- is the same on any
// device and partition mode (a device with fewer CUs runs the same shares in
// several rounds).
constexpr int64_t kShareSimds = 256 * 4;
constexpr int kTeamWpe = 4;  // row walk by teams
// row walk by chunks: 2 ran the 1M x 64 message-passing step 1.4 % faster
// than 3 (fewer shares for the combine, max+row 49.2 -> 49.0 us)
constexpr int kRowsWpe = 2;
// 1-D: 2 for every operation.  Min/max need the registers.  Sums ran faster
// at 2 than at 4 (at 4 the waves keep twice the bytes in flight that the
// memory needs, and the latency-bound steps -- the partition search, the
// first fetch -- wait behind them): the 50M-element heavy-skew sum 41.8-42.3
// us against 42.6-42.9 us, the 16M-key RLE sum 22.7-24.4 us against
// 23.3-25.8 us; at 1 wave per SIMD they took 48.2 and 28.1 us.
template <int DT, int OP>
constexpr int flat_wpe() {
    return 2;
}

// Final value of one (segment, feature); `base` turns a share-relative row
// into an absolute one.
template <int DT, int OP>
__device__ __forceinline__ void final_bits(typename Red<DT, OP>::acc_t acc, int64_t len, int64_t base,
                                           uint32_t &ob, int64_t &ab) {
    using R = Red<DT, OP>;
    ab = -1;
    if constexpr (R::kSumF) {
        double x = acc;
        if constexpr (OP == OP_MEAN) x = len > 0 ? x / (double)len : 0.0;
        ob = __float_as_uint((float)x);
    } else if constexpr (R::kSumI) {
        ob = acc;
    } else {
        const uint32_t rel = R::rel_of(acc);
        if (rel == 0xFFFFFFFFu) {
            ob = 0u;
        } else {
            ob = okey_inv<DT>((uint32_t)(acc >> 32));
            ab = base + (int64_t)rel;
        }
    }
}

template <int DT, int OP, int VEC, bool NT = false>
__device__ __forceinline__ void store_final(const KArgs &a, int64_t seg, int64_t f0,
                                            const typename Red<DT, OP>::acc_t *acc, int64_t base,
                                            int64_t len /* rows of the segment, used by MEAN */) {
    uint32_t ob[VEC];
    int64_t ab[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) final_bits<DT, OP>(acc[v], len, base, ob[v], ab[v]);
    // NT: non-temporal stores, for kernels whose outputs are a large part of
    // their traffic (rows of <= 128 bytes in short segments).  Measured on
    // the power-law graph (32M x 32 -> 2M): max+row 1,106 -> 1,045 us per
    // call; on 1M x 64 -> 10K and on 50M -> 1M (few output bytes) plain
    // stores were 2-5 % faster.
    const int64_t o = seg * a.F + f0;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
    auto put = [](auto *p, auto v) __attribute__((always_inline)) {
        if constexpr (NT) __builtin_nontemporal_store(v, p);
        else *p = v;
    };
    if constexpr (VEC == 4) {
        put(reinterpret_cast<u32x4 *>(a.out + o), u32x4{ob[0], ob[1], ob[2], ob[3]});
        if (Red<DT, OP>::kMinMax && a.arg) {
            put(reinterpret_cast<i64x2 *>(a.arg + o), i64x2{ab[0], ab[1]});
            put(reinterpret_cast<i64x2 *>(a.arg + o) + 1, i64x2{ab[2], ab[3]});
        }
    } else if constexpr (VEC == 2) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        put(reinterpret_cast<u32x2 *>(a.out + o), u32x2{ob[0], ob[1]});
        if (Red<DT, OP>::kMinMax && a.arg) put(reinterpret_cast<i64x2 *>(a.arg + o), i64x2{ab[0], ab[1]});
    } else {
        put(a.out + o, ob[0]);
        if (Red<DT, OP>::kMinMax && a.arg) put(a.arg + o, ab[0]);
    }
}

// Number of entries <= x in the ascending array arr[0..n).
__device__ __forceinline__ int count_le(const uint32_t *arr, int n, uint32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (arr[mid] <= x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// LDS place (in 16-byte units) of unit c of the 8 consecutive units that a
// lane owns, where a load instruction's lanes read 1 KB of consecutive units
// (8 lanes per owner): the low three bits are rotated by the owner so that
// the writes (8 owners x 8 units) and the reads (64 owners, one unit each)
// both spread over the banks.
__device__ __forceinline__ int flat_unit(int owner, int c) {
    return owner * 8 + (c ^ ((owner & 7) ^ ((owner >> 3) & 1)));
}

// Header of a share for the combine kernel: [split head segment or -1,
// continuing tail segment or -1, first row of the share, share holding the
// split head segment's first row].
__device__ __forceinline__ void write_header(const KArgs &a, int64_t wave, const Share &sh) {
    a.hdr[wave * 4 + 0] = sh.split_head ? sh.i0 : -1;
    a.hdr[wave * 4 + 1] = sh.has_tail ? sh.i1 : -1;
    a.hdr[wave * 4 + 2] = sh.o0 + sh.j0;
    a.hdr[wave * 4 + 3] = sh.split_head ? (sh.first_row + sh.cw * sh.i0) / sh.D : wave;
}

// Pass 1 for rows of F >= 2 features: each lane owns VEC consecutive
// features of a row (VEC = 4: 16-byte pieces; VEC = 2: 8-byte pieces for
// other even widths; VEC = 1: one 4-byte feature, for rows whose width or
// alignment rules out the others).
//   L   lanes per row (the power of two >= F / VEC, at most 64; wider rows
//       are done in blocks of 64 * VEC features); G = 64 / L row groups per
//       wave
//   V   consecutive rows per group per chunk; CH = G * V items per chunk
//   FC  the row width F when it is fixed at compile time (0: read from the
//       arguments), which turns every row step into an immediate offset
// With L = 64 a row is the whole wave: segment control is wave-uniform and
// no cross-lane step is needed at all.  A chunk's rows are fetched together
// with its first 64 segment ends before its row count is known (up to CH
// rows; rows past the chunk are fetched again by the next chunk), and the
// next chunk is fetched while the current one is processed: straight into
// the lanes' pieces, or, for rows of fewer than 32 features, as whole 1 KB
// stretches that pass through LDS (the 1-D kernel's placement of 16-byte
// units), so that no load instruction gathers small pieces from many rows.
template <int VEC>
struct Lanes;
template <>
struct Lanes<1> {
    using type = uint32_t;
    __device__ static __forceinline__ uint32_t at(uint32_t x, int) { return x; }
    __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) { return ld32(r, off); }
};
template <>
struct Lanes<2> {
    using type = uint2;
    __device__ static __forceinline__ uint32_t at(const uint2 &x, int v) { return v == 0 ? x.x : x.y; }
    __device__ static __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, uint32_t off) { return ld64(r, off); }
};
template <>
struct Lanes<4> {
    using type = uint4;
    __device__ static __forceinline__ uint32_t at(const uint4 &x, int v) {
        return v == 0 ? x.x : v == 1 ? x.y : v == 2 ? x.z : x.w;
    }
    __device__ static __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, uint32_t off) { return ld128(r, off); }
};

template <int DT, int OP, int L, int V, int VEC, int FC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kRowsWpe))) void seg_reduce_rows(const KArgs a) {
    using R = Red<DT, OP>;
    using acc_t = typename R::acc_t;
    using LN = Lanes<VEC>;
    using x_t = typename LN::type;
    constexpr int G = 64 / L;
    constexpr int CH = G * V;
    constexpr int FB = L * VEC;  // features per block
    constexpr uint32_t kInf = 0xFFFFFFFFu;
    const int64_t F = FC > 0 ? (int64_t)FC : a.F;

    __shared__ __attribute__((aligned(16))) uint32_t s_ends[4][CH];
    // Rows narrower than 32 features (a width fixed at compile time below
    // 32, or any width the one feature block of at most 32 features holds):
    // a chunk's bytes (at most 8 KB) are read by load instructions of 1 KB
    // of consecutive bytes each and reach their lanes through LDS, instead
    // of load instructions whose lanes read pieces of 4 to 16 bytes from up
    // to 64 rows.
    constexpr bool STG = FC > 0 ? FC < 32 : FB <= 32;
    constexpr int CB = STG ? CH * (FC > 0 ? FC : FB) * 4 : 0;  // bytes per chunk (at most)
    constexpr int NL = (CB + 1023) / 1024;                     // 1 KB load instructions per chunk
    static_assert(!STG || (FB >= FC && NL <= 8), "a staged chunk is one feature block of at most 8 KB");
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[4][STG ? NL * 256 : 4];

    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane / L;
    const int c = lane % L;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t *off = a.offsets;
    __shared__ int64_t s_probe[kProbesA];
    const int64_t S = seg_count(a);
    const Share sh = find_share(off, S, a.NW, wave, lane, s_probe);
    const int64_t o0 = sh.o0, base = sh.o0 + sh.j0;
    uint32_t *se = s_ends[wid];
    const uint32_t gv = (uint32_t)(g * V);

    for (int64_t fbase = 0; fbase < F; fbase += FB) {
        const int64_t f0 = fbase + (int64_t)c * VEC;
        // VEC = 4 (2) is used only when F is a multiple of 4 (2), so a lane's
        // features are all inside the row or all past it
        const bool fvalid = f0 < F;

        // Partial of the open segment (the one the next chunk starts in),
        // kept per lane; summed over the groups only when a chunk finishes
        // the segment, so chunks without a segment end need no cross-lane
        // work.
        acc_t open[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) open[v] = R::id();
        bool open_spread = false;  // open partials are in several groups
        // MEAN: first row (relative to offsets[0]) of the open segment, so a
        // finished segment's length comes from the ends already in LDS.
        int64_t open_start = sh.first_row;

        // Fetch: a chunk's first 64 segment ends (index clamped into the
        // array, loaded unconditionally: a load under a branch would be
        // waited for inside the branch) and its rows through a buffer
        // descriptor whose range ends with the chunk's last row, so reads past
        // it return 0 without touching memory (a chunk that does not exist
        // gets an empty descriptor).  Register x[t] is refilled with row t of
        // the next chunk as soon as row t of the current chunk is consumed, so
        // the next chunk streams in while this one is processed without a
        // second register set.
        const uint32_t row_bytes = (uint32_t)(F * 4);
        const uint32_t voff = (uint32_t)((gv * F + c * VEC) * 4);
        auto rows_of = [&](int64_t ic_, int64_t jc_) __attribute__((always_inline)) {
            const int64_t rmax = ic_ + jc_ < sh.d1 ? min((int64_t)CH, sh.j1 - jc_) : 0;
            return make_rsrc(a.values + (o0 + jc_) * F + fbase,
                             rmax > 0 ? (uint32_t)(rmax * row_bytes - fbase * 4) : 0u);
        };
        // Byte offset of row t of a chunk for this lane.  With a fixed row
        // width it is an immediate; otherwise the step is hidden from the
        // optimiser once per chunk so that the V offsets are formed next to
        // their loads instead of being kept in V registers.
        uint32_t rstep = row_bytes;
        auto row_off = [&](int t) __attribute__((always_inline)) -> uint32_t {
            return voff + (uint32_t)t * (FC > 0 ? (uint32_t)(FC * 4) : rstep);
        };
        x_t x[V];
        uint4 xr[STG ? NL : 1] = {};  // STG: the next chunk as loaded
        // STG with the width read at run time: the loads this width needs
        const int nl = FC > 0 ? NL : (int)((CH * F * 4 + 1023) / 1024);
        int64_t ic = sh.i0, jc = sh.j0;
        int64_t en = off[min(ic + 1 + lane, S)];
        {
            const auto rs = rows_of(ic, jc);
            if constexpr (STG) {
#pragma unroll
                for (int u = 0; u < NL; ++u)
                    if (u < nl) xr[u] = ld128(rs, (uint32_t)(lane * 16 + u * 1024));
            } else {
#pragma unroll
                for (int t = 0; t < V; ++t) x[t] = LN::load(rs, row_off(t));
            }
        }
        while (ic + jc < sh.d1) {
            if constexpr (FC == 0) asm volatile("" : "+s"(rstep));
            const int64_t items = min((int64_t)CH, sh.d1 - ic - jc);
            const int64_t ends_left = min((int64_t)CH, sh.i1 - ic);

            // Segment ends inside this chunk: end k (row position e relative
            // to jc) is one of the first `items` items iff e + k + 1 <= items.
            // (Lane 0 holds the first candidate; when it lies past the chunk,
            // which is the common case for long segments, nothing else is
            // looked at.)
            const int64_t e0 = en - o0 - jc;
            const bool c0 = lane < ends_left && e0 + lane + 1 <= items;
            int ne = 0;
            if (ends_left > 0 && readfirst(e0) + 1 <= items) {
                int cnt = popc64(ballot(c0));
                if (c0) se[lane] = (uint32_t)e0;
                ne = cnt;
                for (int b = 64; cnt == 64 && b < CH; b += 64) {
                    const int k = b + lane;
                    const bool valid = k < ends_left;
                    const int64_t e = off[min(ic + 1 + k, S)] - o0 - jc;
                    const bool cond = valid && e + k + 1 <= items;
                    cnt = popc64(ballot(cond));
                    if (cond) se[k] = (uint32_t)e;
                    ne += cnt;
                }
            }
            const int rows = (int)(items - ne);
            const int64_t icn = ic + ne, jcn = jc + rows;
            if (ne > 0) {
                // The next chunk's first 64 ends: the ones this chunk did not
                // use move down (a cross-lane read in every lane, since a
                // disabled source lane would read as 0); only lanes past the
                // old batch load (offsets are not refetched chunk after chunk).
                int64_t nx = lane_get(en, (lane + ne) & 63);
                if (lane + ne >= 64) nx = off[min(icn + 1 + lane, S)];
                en = nx;
            }
            const auto rsn = rows_of(icn, jcn);
            const uint32_t relbase = (uint32_t)(jc - sh.j0);
            if constexpr (STG) {
                // Stage this chunk (16-byte unit k at LDS unit flat_unit(k / 8,
                // k % 8)), start loading the next one, and take the lane's
                // piece of each of its V rows back in row order.  Lanes past
                // the row's features read row 0's piece, which they do not use.
                const char *sb = reinterpret_cast<const char *>(s_stage[wid]);
                uint32_t *sx = s_stage[wid];
#pragma unroll
                for (int u = 0; u < NL; ++u)
                    if (u < nl) *reinterpret_cast<uint4 *>(&sx[flat_unit(8 * u + (lane >> 3), lane & 7) * 4]) = xr[u];
#pragma unroll
                for (int u = 0; u < NL; ++u)
                    if (u < nl) xr[u] = ld128(rsn, (uint32_t)(lane * 16 + u * 1024));
                wave_lds_sync();
                // (The row step is the plain row width here, not the hidden
                // one of the direct loads: the V addresses are the same in
                // every chunk and stay in registers.  Recomputed per chunk,
                // they cost 11 VALU instructions a row: 5 features moved
                // 0.52 of peak on long segments that way, 0.72 with them
                // kept.)
                const uint32_t b0 = fvalid ? voff : 0u;
#pragma unroll
                for (int t = 0; t < V; ++t) {
                    const uint32_t b = b0 + (uint32_t)t * (FC > 0 ? (uint32_t)(FC * 4) : row_bytes);
                    const uint32_t k = b >> 4;
                    x[t] = *reinterpret_cast<const x_t *>(sb + flat_unit((int)(k >> 3), (int)(k & 7u)) * 16 + (b & 15u));
                }
            }

            if (ne == 0) {
                // No segment ends here: every row continues the open segment.
#pragma unroll
                for (int t = 0; t < V; ++t) {
                    const uint32_t r = gv + t;
                    if ((int)r < rows) {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) open[v] = R::comb(open[v], R::lift(LN::at(x[t], v), relbase + r));
                    }
                    if constexpr (!STG) x[t] = LN::load(rsn, row_off(t));
                }
                open_spread = G > 1;
                ic = icn;
                jc = jcn;
                continue;
            }

            // The open segment's partial so far, needed by group 0 only: the
            // groups' parts in group order when they are spread.
            acc_t carry[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) carry[v] = open[v];
            if (G > 1 && open_spread) {
#pragma unroll
                for (int m = L; m < 64; m <<= 1) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const acc_t o = lane_get(carry[v], lane ^ m);
                        carry[v] = (lane & m) ? R::comb(o, carry[v]) : R::comb(carry[v], o);
                    }
                }
            }
            wave_lds_sync();

            // Group g owns rows [gV, gV + V) and the ends at positions
            // (gV, gV + V] (group 0 also those at 0).
            int a_lo = 0, a_hi = ne;
            if constexpr (G > 1) {
                a_lo = g == 0 ? 0 : count_le(se, ne, gv);
                a_hi = count_le(se, ne, gv + V);
            }

            // Walk the group's rows in order (wave-uniform control for G = 1).
            acc_t acc[VEC], hacc[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = hacc[v] = R::id();
            bool hh = false;  // this group finished at least one segment
            int64_t hseg = 0, hlen = 0;
            int k = a_lo;
            int64_t seg = ic + a_lo;
            int64_t seg_start = open_start;  // MEAN only
            if constexpr (OP == OP_MEAN && G > 1) {
                if (a_lo > 0) seg_start = jc + (int64_t)se[a_lo - 1];
            }
            auto end_at = [&](int kk) __attribute__((always_inline)) -> uint32_t {
                if (kk >= a_hi) return kInf;
                const uint32_t e = se[kk];
                return G == 1 ? __builtin_amdgcn_readfirstlane(e) : e;
            };
            uint32_t next_end = end_at(k);

            auto finish = [&]() __attribute__((always_inline)) {
                int64_t len = 0;
                if constexpr (OP == OP_MEAN) {
                    const int64_t e_abs = jc + (int64_t)next_end;
                    len = e_abs - seg_start;
                    seg_start = e_abs;
                }
                if (!hh) {
                    hh = true;
                    hseg = seg;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) hacc[v] = acc[v];
                    hlen = len;
                } else if (fvalid) {
                    store_final<DT, OP, VEC>(a, seg, f0, acc, base, len);
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = R::id();
                ++seg;
                ++k;
                next_end = end_at(k);
            };

#pragma unroll
            for (int t = 0; t < V; ++t) {
                const uint32_t r = gv + t;
                while (next_end <= r) finish();
                if ((int)r < rows) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[v] = R::comb(acc[v], R::lift(LN::at(x[t], v), relbase + r));
                }
                if constexpr (!STG) x[t] = LN::load(rsn, row_off(t));
            }
            while (k < a_hi) finish();

            // Segmented inclusive scan over the groups; the carry enters at
            // group 0.  A group that finished a segment restarts the scan.
            acc_t xs[VEC], ex[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                xs[v] = (g == 0 && !hh) ? R::comb(carry[v], acc[v]) : acc[v];
                ex[v] = carry[v];
            }
            if constexpr (G > 1) {
                bool flag = hh;
#pragma unroll
                for (int o = L; o < 64; o <<= 1) {
                    const int src = (lane - o) & 63;
                    const bool pf = lane_get(flag, src);
                    acc_t px[VEC];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) px[v] = lane_get(xs[v], src);
                    if (lane >= o) {
                        if (!flag) {
#pragma unroll
                            for (int v = 0; v < VEC; ++v) xs[v] = R::comb(px[v], xs[v]);
                        }
                        flag = flag || pf;
                    }
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const acc_t prev = lane_get(xs[v], (lane - L) & 63);
                    if (g != 0) ex[v] = prev;
                }
            }
            if (hh && fvalid) {
                acc_t hv[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) hv[v] = R::comb(ex[v], hacc[v]);
                if (sh.split_head && hseg == sh.i0) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) a.hval[wave * F + f0 + v] = R::to_slot(hv[v]);
                } else {
                    store_final<DT, OP, VEC>(a, hseg, f0, hv, base, hlen);
                }
            }
            // The open segment after this chunk: group G-1's inclusive value,
            // parked in group 0.
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                if constexpr (G > 1) {
                    const acc_t last = lane_get(xs[v], (G - 1) * L + c);
                    open[v] = g == 0 ? last : R::id();
                } else {
                    open[v] = xs[v];
                }
            }
            open_spread = false;
            if constexpr (OP == OP_MEAN) open_start = jc + (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane(se[ne - 1]);

            ic = icn;
            jc = jcn;
            wave_lds_sync();
        }
        if (sh.has_tail) {
            acc_t t[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) t[v] = open[v];
            if (G > 1 && open_spread) {
#pragma unroll
                for (int m = L; m < 64; m <<= 1) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const acc_t o = lane_get(t[v], lane ^ m);
                        t[v] = (lane & m) ? R::comb(o, t[v]) : R::comb(t[v], o);
                    }
                }
            }
            if (g == 0 && fvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) a.tval[wave * F + f0 + v] = R::to_slot(t[v]);
            }
        }
    }
    if (lane == 0) write_header(a, wave, sh);
}

// Pass 1 for rows of F >= 2 features, by teams: a team is the L lanes that
// hold one row (VEC features per lane), G = 64 / L teams per wave.  The
// merge-path partition is made at team granularity: the wave's share is
// split into G equal parts of the (rows + segment ends) sequence, and team
// g walks the rows of part g one at a time, in order, finishing every
// segment whose end it meets.  Each team keeps its own accumulators and its
// own queue of upcoming segment ends, so the walk needs no cross-lane step;
// a load instruction of the wave fetches one row of every team (G rows from
// G places, each a whole number of cache lines).  Loads run V rows ahead of
// the walk.  After the walk the teams' partials of segments cut by part
// boundaries go to LDS and the wave folds them in team order: segments that
// began in this wave are finished there, and the wave leaves at most one
// head and one tail partial in scratch for the combine kernel, as a share
// of the 1-D kernel does.
//   L    lanes per row (power of two >= F / VEC, at most 64; wider rows are
//        walked again per block of 64 * VEC features)
//   V    rows in flight per team
//   FC   F when fixed at compile time (row steps become immediates), else 0
template <int DT, int OP, int L, int V, int VEC, int FC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kTeamWpe))) void seg_reduce_team(const KArgs a) {
    using R = Red<DT, OP>;
    using acc_t = typename R::acc_t;
    using LN = Lanes<VEC>;
    using x_t = typename LN::type;
    constexpr int G = 64 / L;
    constexpr int FB = L * VEC;
    constexpr int P = 4;  // probes per lane per search round
    constexpr uint32_t kNoRow = 0xFFFFFFF0u;  // lane offset past any descriptor
    constexpr uint32_t kNoEnd = 0xFFFFFFFFu;
    const int64_t F = FC > 0 ? (int64_t)FC : a.F;

    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane / L;
    const int c = lane % L;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t *off = a.offsets;
    __shared__ int64_t s_probe[kProbesA];
    const int64_t S = seg_count(a);
    // period: 64 KB of rows, in items
    const Share sh = find_share(off, S, a.NW, wave, lane, s_probe, 1, G, 65536 / (F * 4));
    const int64_t o0 = sh.o0;
    const int64_t dT = sh.D / G;  // items per team part
    auto rebase = [](acc_t p, uint32_t delta) __attribute__((always_inline)) -> acc_t {
        if constexpr (R::kMinMax) return rebase_word(p, delta, OP == OP_MAX);
        else return p;
    };
    // per wave: the teams' head and tail partials of the current feature
    // block, and what the fold needs to know of each part
    struct PartInfo {
        int64_t i0, i1;
        uint32_t delta;  // first row of the part - first row of the share
        uint32_t flags;  // 1: split head, 2: tail, 4: the head began in this wave
    };
    __shared__ uint64_t s_hp[4][2][64 * VEC];
    __shared__ PartInfo s_info[4][G];

    // Part g starts at diagonal t0 = d0 + g dT: i(t0) lies in [i0, i1] and
    // key(i0) <= d0 <= t0.  The team's L lanes narrow it with (L P)-way
    // rounds over consecutive offsets (counts and keys within the team).
    const int64_t t0 = min(sh.d0 + (int64_t)g * dT, sh.d1);
    int64_t lo = sh.i0, hi = g == 0 ? sh.i0 : sh.i1, klo = sh.first_row + sh.i0;
    const uint64_t tmask = (G == 1 ? ~0ull : ((1ull << L) - 1ull)) << (g * L);
    while (lo < hi) {
        const int64_t st = (hi - lo + L * P - 1) / (L * P);
        int64_t kp[P];
        int n = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t pos = lo + (int64_t)(p * L + c + 1) * st;
            const int64_t q = min(pos, S);
            kp[p] = off[q] - o0 + q;
            n += popc64(ballot(pos <= hi && kp[p] <= t0) & tmask);
        }
        if (n > 0) {
            // key of probe n (1-based): slot (n - 1) / L of team lane (n - 1) % L
            const int m = n - 1;
            const int src = g * L + (m % L), slot = m / L;
            int64_t v = 0;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int64_t w = lane_get(kp[p], src);
                v = slot == p ? w : v;
            }
            klo = v;
        }
        hi = min(hi, lo + (int64_t)(n + 1) * st - 1);
        lo += (int64_t)n * st;
    }
    // The part: ends [ti0, ti1), rows [tj0, tj1) relative to o0; its end is
    // the next team's start (the share's end for the last team).
    const int64_t ti0 = lo, tj0 = t0 - lo, tfirst = klo - lo;
    int64_t ti1 = lane_get(ti0, (lane + L) & 63), tj1 = lane_get(tj0, (lane + L) & 63);
    int64_t ttail = lane_get(tfirst, (lane + L) & 63);
    if (g == G - 1) {
        ti1 = sh.i1;
        tj1 = sh.j1;
        ttail = sh.tail_row;
    }
    const bool split_head = ti0 < ti1 && tfirst < tj0;
    const bool has_tail = ti1 < S && ttail < tj1;
    const int64_t base = o0 + tj0;                    // absolute first row of the part
    const uint32_t nrows = (uint32_t)(tj1 - tj0);     // rows of the part
    const uint32_t row_bytes = (uint32_t)(F * 4);
    // relative end of segment k (k < ti1), or kNoEnd
    auto end_rel = [&](int64_t k) __attribute__((always_inline)) -> uint32_t {
        const int64_t e = off[min(k + 1, S)] - o0 - tj0;
        return k < ti1 ? (uint32_t)e : kNoEnd;
    };

    for (int64_t fbase = 0; fbase < F; fbase += FB) {
        const int64_t f0 = fbase + (int64_t)c * VEC;
        const bool fvalid = f0 < F;
        // All rows of the wave's share lie in one descriptor; a team's row r
        // (relative to its part) is at lane offset toff + r * row_bytes, and
        // rows at or past the part's end are asked for at kNoRow (read as 0).
        const auto rs = make_rsrc(a.values + (o0 + sh.j0) * F + fbase,
                                  sh.j1 > sh.j0 ? (uint32_t)((sh.j1 - sh.j0) * F * 4 - fbase * 4) : 0u);
        const uint32_t toff = (uint32_t)((tj0 - sh.j0) * F + c * VEC) * 4u;
        auto row_at = [&](uint32_t r) __attribute__((always_inline)) -> uint32_t {
            return r < nrows ? toff + r * row_bytes : kNoRow;
        };
        // Min/max: each piece starts from R::piece_start (see there); the
        // piece of segment `seg` in this part begins at row pstart.
        acc_t acc[VEC], hacc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            hacc[v] = R::id();
            if constexpr (R::kMinMax) acc[v] = R::piece_start(0u);
            else acc[v] = R::id();
        }
        int64_t seg = ti0;
        uint32_t e1 = end_rel(seg), e2 = end_rel(seg + 1);  // the next two ends
        uint32_t seg_start = (uint32_t)(tfirst - tj0);      // MEAN: start of segment `seg` (wraps if earlier)
        uint32_t pstart = 0;

        auto finish = [&]() __attribute__((always_inline)) {
            if constexpr (R::kMinMax) {
                if (e1 == pstart) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[v] = R::id();
                }
            }
            if (seg == ti0 && split_head) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) hacc[v] = acc[v];
            } else if (fvalid) {
                store_final<DT, OP, VEC, true>(a, seg, f0, acc, base, (int64_t)(e1 - seg_start));
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                if constexpr (R::kMinMax) acc[v] = R::piece_start(e1);
                else acc[v] = R::id();
            }
            pstart = e1;
            seg_start = e1;
            ++seg;
            e1 = e2;
            e2 = end_rel(seg + 1);
        };

        x_t x[V];
#pragma unroll
        for (int t = 0; t < V; ++t) x[t] = LN::load(rs, row_at((uint32_t)t));
        for (uint32_t rb = 0; ballot(rb < nrows) != 0; rb += V) {
#pragma unroll
            for (int t = 0; t < V; ++t) {
                const uint32_t r = rb + t;
                while (e1 <= r) finish();
                if (r < nrows) {
                    if constexpr (R::kMinMax) {
                        const uint32_t code = R::code_of(r);
#pragma unroll
                        for (int v = 0; v < VEC; ++v) R::step(acc[v], LN::at(x[t], v), code);
                    } else {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) acc[v] = R::comb(acc[v], R::lift(LN::at(x[t], v), r));
                    }
                }
                x[t] = LN::load(rs, row_at(r + V));
            }
        }
        while (e1 != kNoEnd) finish();
        if constexpr (R::kMinMax) {
            if (pstart >= nrows) {  // the open piece has no rows
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = R::id();
            }
        }

        // Fold the parts' partials in team order (row codes rebased to the
        // share's first row).
        if constexpr (G > 1) {
            const uint32_t delta = (uint32_t)(tj0 - sh.j0);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                s_hp[wid][0][lane * VEC + v] = R::to_slot(rebase(hacc[v], delta));
                s_hp[wid][1][lane * VEC + v] = R::to_slot(rebase(acc[v], delta));
            }
            if (c == 0) {
                const bool in_wave = (tfirst + ti0) / dT >= wave * G;
                s_info[wid][g] = PartInfo{ti0, ti1, delta,
                                          (split_head ? 1u : 0u) | (has_tail ? 2u : 0u) | (in_wave ? 4u : 0u)};
            }
            wave_lds_sync();
            if (g == 0) {
                acc_t run[VEC];
                bool run_on = false;
                for (int gg = 0; gg < G; ++gg) {
                    const PartInfo pi = s_info[wid][gg];
                    if (pi.flags & 1u) {
                        acc_t val[VEC];
#pragma unroll
                        for (int v = 0; v < VEC; ++v) {
                            const acc_t h = R::from_slot(s_hp[wid][0][(gg * L + c) * VEC + v]);
                            val[v] = run_on ? R::comb(run[v], h) : h;
                        }
                        if (pi.flags & 4u) {
                            if (fvalid) {
                                int64_t len = 0;
                                if constexpr (OP == OP_MEAN) len = off[pi.i0 + 1] - off[pi.i0];
                                store_final<DT, OP, VEC, true>(a, pi.i0, f0, val, o0 + sh.j0, len);
                            }
                        } else if (fvalid) {
#pragma unroll
                            for (int v = 0; v < VEC; ++v) a.hval[wave * F + f0 + v] = R::to_slot(val[v]);
                        }
                        run_on = false;
                    }
                    if (pi.flags & 2u) {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) {
                            const acc_t t = R::from_slot(s_hp[wid][1][(gg * L + c) * VEC + v]);
                            run[v] = (run_on && pi.i0 == pi.i1) ? R::comb(run[v], t) : t;
                        }
                        run_on = true;
                    } else {
                        run_on = false;
                    }
                }
                if (sh.has_tail && fvalid) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) a.tval[wave * F + f0 + v] = R::to_slot(run[v]);
                }
            }
            wave_lds_sync();
        } else {
            if (split_head && fvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) a.hval[wave * F + f0 + v] = R::to_slot(hacc[v]);
            }
            if (has_tail && fvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) a.tval[wave * F + f0 + v] = R::to_slot(acc[v]);
            }
        }
    }
    if (lane == 0) write_header(a, wave, sh);
}

// Weight of a segment end against one 1-D element in the merge-path shares.
// An end costs an offsets read and an output store (and a row for min/max),
// and a chunk holds at most EC of them, against 4 bytes per element; with
// equal weights the shares over stretches of very short segments finish
// last.  Measured on 16M sorted Zipf keys (0.71M runs): sum 30.8 -> 27.3 us,
// min+row 37.1 -> 31.3 us from weight 1 to 8 (4: 29.2 / 33.4, 16: 27.6 /
// 30.6, 32: 28.3 / 35.6); 50M elements in 1M segments unchanged.
constexpr int kFlatEndWeight = 8;

// Pass 1 for one feature per row (1-D values).
//
// A chunk is up to 2048 elements and up to 128 segment ends.  Its elements
// arrive with coalesced 16-byte loads and are staged through LDS (an XOR
// swizzle of 16-byte units keeps both the fill and the per-lane reads free of
// bank conflicts), so that lane l holds elements [32 l, 32 l + 32).  The
// chunk's ends become a reset mask per lane (bit t: a segment ends right
// before element 32 l + t).  Each lane then makes one pass over its 32
// elements that restarts its accumulator at every reset (an AND with the
// sign-extended mask bit, no branches) and leaves its running value at every
// element in LDS; a segmented scan across the lanes (cross-lane moves) gives
// every lane the part of its open segment that lies before it.  The result of
// a segment ending before element p is then the running value at p - 1, plus
// the carried-in part when the segment began before that lane: one lane per
// end looks both up and stores the result, so the stores are coalesced.  The
// next chunk streams into registers while this one is processed.
//
// Float sums: a lane's 32 elements and the scan across a chunk's 64 lanes add
// in float32 (a tree of depth 6 over lane sums of at most 32 terms, so the
// error stays below 38 * 2^-24 of the sum of magnitudes, well inside
// 1e-5 * sum|x|); everything that crosses a chunk or share boundary adds in
// float64.  Min/max: the running value is the packed (key, 32 - t) word of
// the best element so far (MIN complements the key, so both are a maximum);
// only its position byte is kept in LDS and the store looks the element up
// again in the staged chunk.
template <int DT, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(flat_wpe<DT, OP>())))
void seg_reduce_flat(const KArgs a) {
    using R = Red<DT, OP>;
    using acc_t = typename R::acc_t;
    constexpr bool kSumF = R::kSumF, kMM = R::kMinMax;
    constexpr int V = 32, CH = 64 * V, EC = 512, NB = 2;
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    // in-chunk value: float for float sums, else the accumulator itself
    // (min/max in the "maximum" domain)
    using lacc_t = std::conditional_t<kSumF, float, acc_t>;
    auto to_max = [](acc_t v) __attribute__((always_inline)) -> acc_t {
        if constexpr (OP == OP_MIN) return ~v;
        else return v;
    };
    auto widen = [](lacc_t v) __attribute__((always_inline)) -> acc_t {
        if constexpr (kSumF) return (double)v;
        else return v;
    };
    auto lcomb = [](lacc_t e, lacc_t l) __attribute__((always_inline)) -> lacc_t {
        if constexpr (kMM) return l > e ? l : e;
        else return e + l;
    };
    auto acomb = [](acc_t e, acc_t l) __attribute__((always_inline)) -> acc_t {
        if constexpr (kMM) return l > e ? l : e;
        else return e + l;
    };
    // packed word of element t of lane l (row code relative to the share)
    auto mm_word = [&](uint32_t bits, uint32_t rel) __attribute__((always_inline)) -> uint64_t {
        uint32_t key = okey<DT>(bits);
        if constexpr (OP == OP_MIN) key = ~key;
        return ((uint64_t)key << 32) | ~rel;
    };

    __shared__ __attribute__((aligned(16))) uint32_t s_x[4][CH];            // elements (sums: then running values)
    __shared__ __attribute__((aligned(16))) uint32_t s_p[4][kMM ? CH / 4 : 4];  // min/max: position bytes
    __shared__ uint16_t s_e[4][EC];                                         // end positions in the chunk
    __shared__ uint32_t s_m[4][64];                                         // reset masks
    __shared__ uint64_t s_c[4][64];                                         // carried-in part per lane
    // the partition search's probes share wave 0's staging area (the search
    // ends with a barrier, before any wave stages a chunk)
    static_assert(kProbesA * sizeof(int64_t) <= CH * sizeof(uint32_t), "probes must fit one staging area");
    int64_t *s_probe = reinterpret_cast<int64_t *>(s_x[0]);

    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t *off = a.offsets;
    const int64_t S = seg_count(a);
    const Share sh = find_share<false, kFlatEndWeight>(off, S, a.NW, wave, lane, s_probe, (int64_t)CH);
    const int64_t o0 = sh.o0, base = sh.o0 + sh.j0;
    uint32_t *sx = s_x[wid];
    uint8_t *sp = reinterpret_cast<uint8_t *>(s_p[wid]);
    uint16_t *se = s_e[wid];
    uint32_t *sm = s_m[wid];
    uint64_t *sc = s_c[wid];

    // Fetch a chunk: its first EC ends (indices clamped, loads unconditional)
    // and its elements through a descriptor limited to the share's remaining
    // rows (reads past them return 0).
    uint4 X[V / 4];
    int64_t E[NB];
    auto fetch = [&](int64_t ic_, int64_t jc_) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) E[b] = off[min(ic_ + 1 + b * 64 + lane, S)];
        const int64_t rmax = ic_ + jc_ < sh.d1 ? min((int64_t)CH, sh.j1 - jc_) : 0;
        const auto rs = make_rsrc(a.values + (o0 + jc_), (uint32_t)(rmax * 4));
#pragma unroll
        for (int u = 0; u < V / 4; ++u) X[u] = ld128(rs, (uint32_t)(lane * 16 + u * 1024));
    };

    acc_t carry = R::id();
    int64_t ic = sh.i0, jc = sh.j0;
    fetch(ic, jc);
    while (ic + jc < sh.d1) {
        const int64_t rows_avail = min((int64_t)CH, sh.j1 - jc);
        const int64_t ends_avail = min((int64_t)EC, sh.i1 - ic);

        // The chunk's ends: end k (position e relative to jc) belongs to it
        // iff e <= rows_avail; at most EC of them.  Each sets its reset bit.
        sm[lane] = 0u;
        wave_lds_sync();
        int ne = 0;
        bool more = true;
        auto take = [&](int b, int64_t eabs) __attribute__((always_inline)) {
            const int k = b * 64 + lane;
            const int64_t e = eabs - o0 - jc;
            const bool cond = k < ends_avail && e <= rows_avail;
            const int cnt = popc64(ballot(cond));
            if (cond) {
                se[k] = (uint16_t)e;
                if (e < CH) lds_or(&sm[e >> 5], 1u << (e & 31));
            }
            ne += cnt;
            more = cnt == 64;
        };
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (more) take(b, E[b]);
        // Dense stretches: the chunk's further ends, all of their loads
        // issued together once the preloaded ones are used up (one round
        // trip instead of one per batch of 64).
        if (more) {
            int64_t Ex[EC / 64 - NB];
#pragma unroll
            for (int b = NB; b < EC / 64; ++b) Ex[b - NB] = off[min(ic + 1 + b * 64 + lane, S)];
#pragma unroll
            for (int b = NB; b < EC / 64; ++b)
                if (more) take(b, Ex[b - NB]);
        }
        wave_lds_sync();
        // With EC ends the chunk stops at the last of them.
        const int rows = ne == EC ? (int)__builtin_amdgcn_readfirstlane(se[EC - 1]) : (int)rows_avail;

        // Stage the elements (lane l of load u holds elements 256 u + 4 l ..).
#pragma unroll
        for (int u = 0; u < V / 4; ++u)
            *reinterpret_cast<uint4 *>(&sx[flat_unit(8 * u + (lane >> 3), lane & 7) * 4]) = X[u];
        const int64_t icn = ic + ne, jcn = jc + rows;
        fetch(icn, jcn);
        wave_lds_sync();

        uint32_t x[V];
#pragma unroll
        for (int c = 0; c < V / 4; ++c) {
            const uint4 q = *reinterpret_cast<const uint4 *>(&sx[flat_unit(lane, c) * 4]);
            x[4 * c] = q.x;
            x[4 * c + 1] = q.y;
            x[4 * c + 2] = q.z;
            x[4 * c + 3] = q.w;
        }
        const uint32_t keep = ~sm[lane];
        const uint32_t rel0 = (uint32_t)(jc - sh.j0) + (uint32_t)(lane * V);  // row code base of the lane

        // One pass over the lane's elements, restarting at every reset.
        // Elements past `rows` (a partial chunk) are not excluded: nothing
        // reads a running value at or past them (the carry out of the chunk
        // is looked up at position `rows` like a segment end).
        lacc_t acc{};
        {
            uint32_t pk = 0;
#pragma unroll
            for (int t = 0; t < V; ++t) {
                const uint32_t km = sbit(keep, t);
                if constexpr (kMM) {
                    acc &= ((uint64_t)km << 32) | km;
                    uint32_t key = okey<DT>(x[t]);
                    if constexpr (OP == OP_MIN) key = ~key;
                    const uint64_t cand = ((uint64_t)key << 32) | (uint32_t)(V - t);
                    acc = cand > acc ? cand : acc;
                    // position byte of the best element so far (V - t)
                    pk |= ((uint32_t)acc & 0xFFu) << (8 * (t & 3));
                    if ((t & 3) == 3) {
                        reinterpret_cast<uint32_t *>(sp)[lane * (V / 4) + (t >> 2)] = pk;
                        pk = 0;
                    }
                } else {
                    if constexpr (kSumF) acc = __uint_as_float(__float_as_uint(acc) & km) + __uint_as_float(x[t]);
                    else acc = (acc & km) + x[t];
                    x[t] = kSumF ? __float_as_uint(acc) : (uint32_t)acc;
                }
            }
        }
        if constexpr (!kMM) {
#pragma unroll
            for (int c = 0; c < V / 4; ++c)
                *reinterpret_cast<uint4 *>(&sx[flat_unit(lane, c) * 4]) =
                    make_uint4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
        }

        // Segmented scan across the lanes of the lanes' open parts.
        bool fl = keep != 0xFFFFFFFFu;
        lacc_t xs = acc;
        if constexpr (kMM) {
            // local (key, V - t) word -> (key, ~row code)
            if (acc != 0) xs = (acc & 0xFFFFFFFF00000000ull) | ~(rel0 + (uint32_t)V - (uint32_t)acc);
        }
        seg_scan_wave(xs, fl, lacc_t{}, lcomb);
        const acc_t cm = to_max(carry);
        // the scan up to the lane before (lane 0: nothing)
        const lacc_t ex = dpp_move<kDppWaveShr1>(lacc_t{}, xs);
        const bool fx = dpp32<kDppWaveShr1>(0u, fl ? 1u : 0u) != 0u;
        const acc_t cin = fx ? widen(ex) : acomb(cm, widen(ex));
        sc[lane] = R::to_slot(cin);
        wave_lds_sync();

        // Value (maximum domain) of the part of a segment inside this chunk
        // that ends right before element p >= 1, given the previous end pp
        // (kNone: the segment began before the chunk).
        const uint32_t relc = (uint32_t)(jc - sh.j0);
        auto piece = [&](uint32_t p, uint32_t pp) __attribute__((always_inline)) -> acc_t {
            const uint32_t l2 = (p - 1) >> 5, t2 = (p - 1) & 31;
            acc_t v;
            if constexpr (kMM) {
                const uint32_t tb = (uint32_t)V - sp[l2 * V + t2];  // the best element of the piece
                const uint32_t bits = sx[flat_unit((int)l2, (int)(tb >> 2)) * 4 + (int)(tb & 3)];
                v = mm_word(bits, relc + l2 * V + tb);
            } else {
                const uint32_t b = sx[flat_unit((int)l2, (int)(t2 >> 2)) * 4 + (int)(t2 & 3)];
                if constexpr (kSumF) v = (double)__uint_as_float(b);
                else v = b;
            }
            if (pp == kNone || pp < (l2 << 5)) v = acomb(R::from_slot(sc[l2]), v);
            return v;
        };

        // One lane per end: look up the segment's value and store it.
        for (int q = lane; q < ne; q += 64) {
            const uint32_t p = se[q];
            const uint32_t pp = q > 0 ? se[q - 1] : kNone;
            const int64_t seg = ic + q;
            acc_t v;
            if (p == pp) {
                v = to_max(R::id());  // empty
            } else if (p == 0) {
                v = R::from_slot(sc[0]);  // ends where the chunk starts
            } else {
                v = piece(p, pp);
            }
            v = to_max(v);
            if (sh.split_head && seg == sh.i0) {
                a.hval[wave] = R::to_slot(v);
            } else {
                int64_t len = 0;
                if constexpr (OP == OP_MEAN) len = off[seg + 1] - off[seg];
                store_final<DT, OP, 1>(a, seg, 0, &v, base, len);
            }
        }
        // The part of the open segment after the chunk: the chunk's rows
        // after its last end (none when the last end closes the last row).
        {
            const uint32_t last = ne > 0 ? __builtin_amdgcn_readfirstlane(se[ne - 1]) : kNone;
            if (last == (uint32_t)rows) carry = R::id();
            else if (rows > 0) carry = to_max(piece((uint32_t)rows, last));
        }
        ic = icn;
        jc = jcn;
        wave_lds_sync();
    }
    if (lane == 0) {
        if (sh.has_tail) a.tval[wave] = R::to_slot(carry);
        write_header(a, wave, sh);
    }
}

// Pass-2 accumulator: min/max carry the key and the absolute row separately,
// since partials of different shares use different row bases.
template <int DT, int OP, bool MM = Red<DT, OP>::kMinMax>
struct P2 {
    using R = Red<DT, OP>;
    typename R::acc_t v;
    __device__ static P2 id() { return {R::id()}; }
    __device__ static P2 from(uint64_t slot, int64_t) { return {R::from_slot(slot)}; }
    __device__ static P2 comb(P2 a, P2 b) { return {R::comb(a.v, b.v)}; }
    __device__ P2 get(int src) const { return {lane_get(v, src)}; }
    __device__ void bits(int64_t len, uint32_t &ob, int64_t &ab) const { final_bits<DT, OP>(v, len, 0, ob, ab); }
};

template <int DT, int OP>
struct P2<DT, OP, true> {
    using R = Red<DT, OP>;
    uint32_t key;
    int64_t row;  // INT64_MAX: no row
    __device__ static P2 id() { return {OP == OP_MAX ? 0u : 0xFFFFFFFFu, INT64_MAX}; }
    __device__ static P2 from(uint64_t slot, int64_t base) {
        const uint32_t rel = R::rel_of(slot);
        if (rel == 0xFFFFFFFFu) return id();
        return {(uint32_t)(slot >> 32), base + (int64_t)rel};
    }
    __device__ static P2 comb(P2 a, P2 b) {
        const bool better = OP == OP_MAX ? b.key > a.key : b.key < a.key;
        return (better || (b.key == a.key && b.row < a.row)) ? b : a;
    }
    __device__ P2 get(int src) const { return {lane_get(key, src), lane_get(row, src)}; }
    __device__ void bits(int64_t, uint32_t &ob, int64_t &ab) const {
        if (row == INT64_MAX) {
            ob = 0u;
            ab = -1;
        } else {
            ob = okey_inv<DT>(key);
            ab = row;
        }
    }
};

// Pass 2: a share whose first segment began in earlier shares folds the tail
// partials of those shares, in share order, into its head partial.  One wave
// per share; a share without such a segment only reads its header.
template <int DT, int OP>
__global__ __launch_bounds__(256) void seg_reduce_pass2(const KArgs a) {
    using P = P2<DT, OP>;
    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + wid;
    if (w >= a.NS) return;
    const int64_t s = a.hdr[w * 4 + 0];
    const int64_t first = a.hdr[w * 4 + 3];  // share holding the segment's first row
    if (s < 0) return;
    int64_t len = 0;
    if constexpr (OP == OP_MEAN) len = a.offsets[s + 1] - a.offsets[s];

    int fp = 1;
    while (fp < a.F && fp < 64) fp <<= 1;
    const int cols = 64 / fp;  // tail partials folded side by side
    const int cc = lane / fp, fl = lane % fp;

    for (int64_t fb = 0; fb < a.F; fb += fp) {
        const int64_t f = fb + fl;
        const bool valid = f < a.F;
        P acc = P::id();
        if (valid) {
            int64_t t = first + cc;
            for (; t + 3 * cols < w; t += 4 * cols) {
                uint64_t q[4];
                int64_t bs[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    q[u] = a.tval[(t + u * cols) * a.F + f];
                    bs[u] = a.hdr[(t + u * cols) * 4 + 2];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = P::comb(acc, P::from(q[u], bs[u]));
            }
            for (; t < w; t += cols) acc = P::comb(acc, P::from(a.tval[t * a.F + f], a.hdr[t * 4 + 2]));
        }
        for (int m = fp; m < 64; m <<= 1) {
            const P o = acc.get(lane ^ m);
            acc = (lane & m) ? P::comb(o, acc) : P::comb(acc, o);
        }
        if (cc == 0 && valid) {
            acc = P::comb(acc, P::from(a.hval[w * a.F + f], a.hdr[w * 4 + 2]));
            uint32_t ob;
            int64_t ab;
            acc.bits(len, ob, ab);
            a.out[s * a.F + f] = ob;
            if (Red<DT, OP>::kMinMax && a.arg) a.arg[s * a.F + f] = ab;
        }
    }
}

// ------------------------------------------------------------------ host side

constexpr int64_t kMaxFeat = int64_t(1) << 24;

// Lanes per row for rows of `units` lane-sized pieces: the power of two at
// or above it, at most 64.
static int lanes_for(int64_t units, int lo) {
    int64_t l = lo;
    while (l < units && l < 64) l <<= 1;
    return (int)l;
}

// Pass-1 kernel for a row width and the alignment of the arrays, and its
// share count.  When values, out and arg_out start on 16 bytes, rows that
// are whole 16-byte units take 16-byte access (four features per lane) and
// other even widths 8-byte access (two); all other rows one feature per
// lane.  Rows of 32 features with 16-byte access are walked by teams of 8
// lanes (8 whole 128-byte rows per load instruction, no per-chunk
// cross-lane step); all other rows by chunks.  Other rows walked by teams
// would give each team a piece of 4 to 112 bytes per load instruction,
// from up to 64 places, and the L2 request rate caps that: on 512 MB of
// rows of 2 to 24 features the team walk moved 0.04-0.52 of peak, the
// chunked walk 0.10-0.68.  The chunked walk's pieces still come from many
// rows per instruction, so rows of fewer than 32 features read each chunk
// in whole 1 KB stretches through LDS.  The usual widths (2, 3, 4, 6, 8, 12,
// 16, 24) get kernels of their own, with the width fixed and chunks of 6 or
// 8 KB: on the same 512 MB, sum and max+row over segments of 4,096 rows and
// more went from 0.25-0.68 to 0.60-0.80 of peak, over segments of 16 rows
// from 0.14-0.47 to 0.25-0.50.  The other widths below 32 share the kernels
// of their lane count, the width read at run time (chunks of 2 to 8 KB):
// 5, 7, 10, 20 and 30 features on long segments went from 0.24-0.64 to
// 0.39-0.77, on segments of 128 rows from 0.23-0.56 to 0.23-0.60, and lost
// up to 0.05 on segments of 4 and 16 rows.  The same staging for 32
// features (by chunks instead of teams) and for 64 moved less on segments
// of 1 to 16 rows and on the power-law graph (0.58 -> 0.54 of peak), so
// those keep their direct loads.  The kernels that read the width take V
// rows per group so that a chunk holds up to 8 KB (32 for one feature per
// lane, 16 for two): against V = 24 and 8, segments of 16 rows of 10, 14
// and 30 features went from 0.23-0.35 to 0.30-0.46 of peak.
struct Pick {
    const void *kernel;
    int64_t waves;  // shares (one per wave) of a call
};
#define SEGRED_TEAM(L, V, VEC, FC) \
    Pick{reinterpret_cast<const void *>(&seg_reduce_team<DT, OP, L, V, VEC, FC>), kShareSimds * kTeamWpe}
#define SEGRED_ROWS(L, V, VEC, FC) \
    Pick{reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, L, V, VEC, FC>), kShareSimds * kRowsWpe}
template <int DT, int OP>
static Pick pick_kernel(int64_t feat, bool aligned16) {
    if (feat == 1)
        return Pick{reinterpret_cast<const void *>(&seg_reduce_flat<DT, OP>), kShareSimds * flat_wpe<DT, OP>()};
    if (aligned16 && feat % 4 == 0) {
        if (feat == 32) return SEGRED_TEAM(8, 8, 4, 32);
        if (feat == 64) return SEGRED_ROWS(16, 8, 4, 64);
        if (feat == 4) return SEGRED_ROWS(1, 8, 4, 4);
        if (feat == 8) return SEGRED_ROWS(2, 8, 4, 8);
        if (feat == 12) return SEGRED_ROWS(4, 8, 4, 12);
        if (feat == 16) return SEGRED_ROWS(4, 8, 4, 16);
        if (feat == 24) return SEGRED_ROWS(8, 8, 4, 24);
        switch (lanes_for(feat / 4, 1)) {
        case 4: return SEGRED_ROWS(4, 8, 4, 0);
        case 8: return SEGRED_ROWS(8, 8, 4, 0);
        case 16: return SEGRED_ROWS(16, 8, 4, 0);
        case 32: return SEGRED_ROWS(32, 8, 4, 0);
        default: return SEGRED_ROWS(64, 8, 4, 0);
        }
    }
    if (aligned16 && feat % 2 == 0) {
        // even widths that are not whole 16-byte units: 8-byte access
        if (feat == 2) return SEGRED_ROWS(1, 16, 2, 2);
        if (feat == 6) return SEGRED_ROWS(4, 16, 2, 6);
        switch (lanes_for(feat / 2, 1)) {
        case 4: return SEGRED_ROWS(4, 8, 2, 0);
        case 8: return SEGRED_ROWS(8, 16, 2, 0);
        case 16: return SEGRED_ROWS(16, 16, 2, 0);
        case 32: return SEGRED_ROWS(32, 8, 2, 0);
        default: return SEGRED_ROWS(64, 8, 2, 0);
        }
    }
    if (feat == 3) return SEGRED_ROWS(4, 32, 1, 3);
    switch (lanes_for(feat, 2)) {
    case 2: return SEGRED_ROWS(2, 32, 1, 0);
    case 4: return SEGRED_ROWS(4, 32, 1, 0);
    case 8: return SEGRED_ROWS(8, 32, 1, 0);
    case 16: return SEGRED_ROWS(16, 32, 1, 0);
    case 32: return SEGRED_ROWS(32, 32, 1, 0);
    default: return SEGRED_ROWS(64, 24, 1, 0);
    }
}
#undef SEGRED_TEAM
#undef SEGRED_ROWS

static int64_t shares_for(const Pick &pk) {
    const int64_t o = shares_override();
    return o > 0 ? (o + 3) / 4 * 4 : pk.waves;  // whole workgroups of 4 waves
}

// Waves of a kernel that fit on the current device at once (0 if unknown).
static int64_t resident_waves(const void *kernel) {
    int dev = 0, cus = 0, blocks = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return (int64_t)cus * blocks * 4;
}

// Scratch of one call: per share a 32-byte header and two F-wide 8-byte
// partial slots.
static size_t scratch_bytes(int64_t ns, int64_t feat) {
    return (size_t)ns * 4 * sizeof(int64_t) + 2 * (size_t)ns * (size_t)feat * sizeof(uint64_t);
}

// Fixed scratch of segred_reduce_noalloc: one array per device, found at
// set-up with hipGetSymbolAddress (the array's name in host code is not a
// device address).  Every header is written by the streaming kernel before
// the combine kernel reads it, and a partial slot is read only when its
// header says it was written, so nothing in it needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Launch a call's two kernels with scratch at `scratch_ptr` (or, when it is
// null, scratch from the stream's cached buffer).  `noalloc` makes a request
// beyond the fixed scratch an error instead.
template <int DT, int OP>
static int run(KArgs k, hipStream_t st, void *fixed_scratch) {
    const bool a16 = aligned(k.values, 16) && aligned(k.out, 16) && (!k.arg || aligned(k.arg, 16));
    const Pick pk = pick_kernel<DT, OP>(k.F, a16);
    const int64_t nw = shares_for(pk);
    const int64_t ns = nw;
    const size_t bytes = scratch_bytes(ns, k.F);
    ScratchLease lease;
    char *p = static_cast<char *>(fixed_scratch);
    if (p) {
        if (bytes > kNoAllocScratchBytes) return SEGRED_ERR_SCRATCH_LIMIT;
    } else {
        int rc = scratch_acquire(lease, bytes, st);
        if (rc != SEGRED_OK) return rc;
        p = static_cast<char *>(lease.ptr);
    }
    const size_t hdr_bytes = (size_t)ns * 4 * sizeof(int64_t);
    k.NW = nw;
    k.NS = ns;
    k.hdr = reinterpret_cast<int64_t *>(p);
    k.hval = reinterpret_cast<uint64_t *>(p + hdr_bytes);
    k.tval = k.hval + (size_t)ns * (size_t)k.F;

    void *params[] = {&k};
    hipError_t e = timed_launch(true, pk.kernel, dim3((unsigned)(nw / 4)), dim3(256), params, 0, st);
    if (e == hipSuccess)
        e = timed_launch(false, reinterpret_cast<const void *>(&seg_reduce_pass2<DT, OP>),
                         dim3((unsigned)((ns + 3) / 4)), dim3(256), params, 0, st);
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

static int dispatch(int32_t dtype, int32_t op, const KArgs &k, hipStream_t st, void *fixed_scratch) {
    switch (dtype * 4 + op) {
    case DT_U32 * 4 + OP_SUM: return run<DT_U32, OP_SUM>(k, st, fixed_scratch);
    case DT_U32 * 4 + OP_MIN: return run<DT_U32, OP_MIN>(k, st, fixed_scratch);
    case DT_U32 * 4 + OP_MAX: return run<DT_U32, OP_MAX>(k, st, fixed_scratch);
    case DT_I32 * 4 + OP_SUM: return run<DT_I32, OP_SUM>(k, st, fixed_scratch);
    case DT_I32 * 4 + OP_MIN: return run<DT_I32, OP_MIN>(k, st, fixed_scratch);
    case DT_I32 * 4 + OP_MAX: return run<DT_I32, OP_MAX>(k, st, fixed_scratch);
    case DT_F32 * 4 + OP_SUM: return run<DT_F32, OP_SUM>(k, st, fixed_scratch);
    case DT_F32 * 4 + OP_MIN: return run<DT_F32, OP_MIN>(k, st, fixed_scratch);
    case DT_F32 * 4 + OP_MAX: return run<DT_F32, OP_MAX>(k, st, fixed_scratch);
    case DT_F32 * 4 + OP_MEAN: return run<DT_F32, OP_MEAN>(k, st, fixed_scratch);
    default: return SEGRED_ERR_UNSUPPORTED;
    }
}

template <int DT, int OP>
static int64_t shares_of(int64_t feat, bool resident) {
    const Pick pk = pick_kernel<DT, OP>(feat, true);
    return resident ? resident_waves(pk.kernel) : shares_for(pk);
}

static int64_t shares_query(int32_t dtype, int32_t op, int64_t feat, bool resident) {
    if (feat < 1) return -1;
    switch (dtype * 4 + op) {
    case DT_U32 * 4 + OP_SUM: return shares_of<DT_U32, OP_SUM>(feat, resident);
    case DT_U32 * 4 + OP_MIN: return shares_of<DT_U32, OP_MIN>(feat, resident);
    case DT_U32 * 4 + OP_MAX: return shares_of<DT_U32, OP_MAX>(feat, resident);
    case DT_I32 * 4 + OP_SUM: return shares_of<DT_I32, OP_SUM>(feat, resident);
    case DT_I32 * 4 + OP_MIN: return shares_of<DT_I32, OP_MIN>(feat, resident);
    case DT_I32 * 4 + OP_MAX: return shares_of<DT_I32, OP_MAX>(feat, resident);
    case DT_F32 * 4 + OP_SUM: return shares_of<DT_F32, OP_SUM>(feat, resident);
    case DT_F32 * 4 + OP_MIN: return shares_of<DT_F32, OP_MIN>(feat, resident);
    case DT_F32 * 4 + OP_MAX: return shares_of<DT_F32, OP_MAX>(feat, resident);
    case DT_F32 * 4 + OP_MEAN: return shares_of<DT_F32, OP_MEAN>(feat, resident);
    default: return -1;
    }
}

}  // namespace segred

using namespace segred;

extern "C" int64_t segred_get_shares(int32_t dtype, int32_t op, int64_t feat) {
    return shares_query(dtype, op, feat, false);
}

extern "C" int64_t segred_resident_waves(int32_t dtype, int32_t op, int64_t feat) {
    return shares_query(dtype, op, feat, true);
}

// Device address of this device's fixed scratch array (null on failure),
// looked up once per device with that device current.
static void *fixed_scratch_for_current_device() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (!ptrs[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptrs[dev] = ptr;
    }
    return ptrs[dev];
}

static int reduce_impl(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                       int64_t num_segments, const int64_t *num_segments_dev, int32_t op, void *out,
                       int64_t *arg_out, hipStream_t stream, bool noalloc = false) {
    if (num_segments < 0 || feat < 1 || dtype < SEGRED_U32 || dtype > SEGRED_F32 || op < SEGRED_SUM ||
        op > SEGRED_MEAN)
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_MEAN && dtype != SEGRED_F32) return SEGRED_ERR_UNSUPPORTED;
    if (feat > kMaxFeat) return SEGRED_ERR_UNSUPPORTED;  // 32-bit in-chunk byte offsets
    if (num_segments == 0) return SEGRED_OK;
    if (!values || !offsets || !out) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!aligned(values, 4) || !aligned(out, 4) || !aligned(offsets, 8) || (arg_out && !aligned(arg_out, 8)) ||
        !aligned(num_segments_dev, 8))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_SUM || op == SEGRED_MEAN) arg_out = nullptr;

    KArgs k{};
    k.values = static_cast<const uint32_t *>(values);
    k.offsets = offsets;
    k.S = num_segments;
    k.S_dev = num_segments_dev;
    k.F = feat;
    k.out = static_cast<uint32_t *>(out);
    k.arg = arg_out;
    void *fixed = nullptr;
    if (noalloc) {
        fixed = fixed_scratch_for_current_device();
        if (!fixed) return SEGRED_ERR_HIP;
    }
    return dispatch(dtype, op, k, stream, fixed);
}

extern "C" int segred_reduce(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                             int64_t num_segments, int32_t op, void *out, int64_t *arg_out,
                             hipStream_t stream) {
    return reduce_impl(values, dtype, feat, offsets, num_segments, nullptr, op, out, arg_out, stream);
}

extern "C" int segred_reduce_device_count(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                                          const int64_t *num_segments, int64_t max_segments, int32_t op, void *out,
                                          int64_t *arg_out, hipStream_t stream) {
    if (!num_segments) return SEGRED_ERR_INVALID_ARGUMENT;
    return reduce_impl(values, dtype, feat, offsets, max_segments, num_segments, op, out, arg_out, stream);
}

extern "C" int segred_reduce_noalloc(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                                     int64_t num_segments, int32_t op, void *out, int64_t *arg_out,
                                     hipStream_t stream) {
    return reduce_impl(values, dtype, feat, offsets, num_segments, nullptr, op, out, arg_out, stream, true);
}
