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
// The sequence is cut into NW equal shares, one per resident wave; the four
// waves of a workgroup find their shares' (segment, row) coordinates with a
// joint search over the offsets.  Long or skewed segments are therefore
// spread over many waves instead of serialising on one.
//
// Inside a share the wave walks chunks.  For rows of F >= 2 features each
// lane owns one feature; a chunk's rows are split into G groups of V
// consecutive rows (G = 1 for F >= 64, where segment control is
// wave-uniform); a group walks its rows in order, finishing every segment
// that ends inside it, and a segmented scan over the groups completes the
// segments cut by group and chunk boundaries.  For 1-D values a chunk is 2048
// elements staged through LDS, 32 consecutive ones per lane, reduced by one
// branch-free pass per lane over reset masks (see seg_reduce_flat).  Segments
// cut by a share boundary leave one partial per share in scratch; a second
// kernel combines them in share order.  Every summation order is a fixed
// function of the offsets and NW, so results repeat bit for bit; no atomic
// operation touches global memory (the only atomic is a bit-OR in LDS).
//
// Memory: rows are read through buffer descriptors that cover exactly the
// valid part of a chunk (reads past it return 0, so no clamping), and the
// next chunk streams into registers while the current one is processed.
//
// Accumulators: float sums in float64 (rounded to float32 once; the 1-D
// kernel adds runs of <= 32 elements and a 64-way tree of them in float32
// first), integer sums in wrapping uint32, min/max as a 64-bit word (order
// key << 32 | row code) whose integer max/min picks the extremum and, on
// equal keys, the lowest row (the packed value/row word of the graph-reduce
// README's "Method").
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "internal.hpp"
#include "keys.hpp"
#include "partition.hpp"
#include "wave.hpp"

namespace segred {

struct KArgs {
    const uint32_t *values;  // element bits, row-major [rows, F]
    const int64_t *offsets;  // [S + 1]
    int64_t S, F, NW;        // S: segment count, or the capacity when S_dev is set
    const int64_t *S_dev;    // segment count on the device (min(*S_dev, S) is used), or null
    uint32_t *out;           // [S, F]
    int64_t *arg;            // [S, F] or null
    int64_t *hdr;            // [NW][4]: see write_header
    uint64_t *hval;          // [NW][F]: partial of the share's first segment when it began earlier
    uint64_t *tval;          // [NW][F]: partial of the share's last segment when it continues
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
};

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

template <int DT, int OP, int VEC>
__device__ __forceinline__ void store_final(const KArgs &a, int64_t seg, int64_t f0,
                                            const typename Red<DT, OP>::acc_t *acc, int64_t base,
                                            int64_t len /* rows of the segment, used by MEAN */) {
    uint32_t ob[VEC];
    int64_t ab[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) final_bits<DT, OP>(acc[v], len, base, ob[v], ab[v]);
    const int64_t o = seg * a.F + f0;
    if constexpr (VEC == 4) {
        *reinterpret_cast<uint4 *>(a.out + o) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        if (Red<DT, OP>::kMinMax && a.arg) {
            reinterpret_cast<longlong2 *>(a.arg + o)[0] = make_longlong2(ab[0], ab[1]);
            reinterpret_cast<longlong2 *>(a.arg + o)[1] = make_longlong2(ab[2], ab[3]);
        }
    } else {
        a.out[o] = ob[0];
        if (Red<DT, OP>::kMinMax && a.arg) a.arg[o] = ab[0];
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

// Header of a share for the combine kernel: [split head segment or -1,
// continuing tail segment or -1, first row of the share, share holding the
// split head segment's first row].
__device__ __forceinline__ void write_header(const KArgs &a, int64_t wave, const Share &sh) {
    a.hdr[wave * 4 + 0] = sh.split_head ? sh.i0 : -1;
    a.hdr[wave * 4 + 1] = sh.has_tail ? sh.i1 : -1;
    a.hdr[wave * 4 + 2] = sh.o0 + sh.j0;
    a.hdr[wave * 4 + 3] = sh.split_head ? (sh.first_row + sh.cw * sh.i0) / sh.D : wave;
}

// Pass 1 for rows of F >= 2 features: each lane owns one feature of a row.
//   L   lanes per row (next power of two >= F, at most 64; wider rows are
//       done in blocks of 64 features); G = 64 / L row groups per wave
//   V   consecutive rows per group per chunk; CH = G * V items per chunk
// With F >= 64 a row is the whole wave: segment control is wave-uniform and
// no cross-lane step is needed at all.  A chunk's rows are fetched together
// with its first 64 segment ends before its row count is known (up to CH
// rows; rows past the chunk are fetched again by the next chunk), and the
// next chunk is fetched while the current one is processed.
template <int DT, int OP, int L, int V>
__global__ __launch_bounds__(256) void seg_reduce_rows(const KArgs a) {
    using R = Red<DT, OP>;
    using acc_t = typename R::acc_t;
    constexpr int G = 64 / L;
    constexpr int CH = G * V;
    constexpr uint32_t kInf = 0xFFFFFFFFu;

    __shared__ __attribute__((aligned(16))) uint32_t s_ends[4][CH];

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

    for (int64_t fbase = 0; fbase < a.F; fbase += L) {
        const int64_t f = fbase + c;
        const bool fvalid = f < a.F;

        // Partial of the open segment (the one the next chunk starts in),
        // kept per lane; summed over the groups only when a chunk finishes
        // the segment, so chunks without a segment end need no cross-lane
        // work.
        acc_t open = R::id();
        bool open_spread = false;  // open partials are in several groups
        // MEAN: first row (relative to offsets[0]) of the open segment, so a
        // finished segment's length comes from the ends already in LDS.
        int64_t open_start = sh.first_row;

        // Fetch: a chunk's first 64 segment ends (index clamped into the
        // array, loaded unconditionally: a load under a branch would be
        // waited for inside the branch) and its rows through a buffer
        // descriptor that covers only the rows inside the share, so rows past
        // it read as 0 without touching memory (a chunk that does not exist
        // gets an empty descriptor).  One lane offset serves all rows; the row
        // step is a scalar offset.  Register x[t] is refilled with row t of
        // the next chunk as soon as row t of the current chunk is consumed, so
        // the next chunk streams in while this one is processed without a
        // second register set.
        const uint32_t row_bytes = (uint32_t)(a.F * 4);
        const uint32_t voff = (uint32_t)((gv * a.F + c) * 4);
        auto rows_of = [&](int64_t ic_, int64_t jc_) __attribute__((always_inline)) {
            const int64_t rmax = ic_ + jc_ < sh.d1 ? min((int64_t)CH, sh.j1 - jc_) : 0;
            return make_rsrc(a.values + (o0 + jc_) * a.F + fbase, (uint32_t)(rmax * row_bytes));
        };
        uint32_t x[V];
        int64_t ic = sh.i0, jc = sh.j0;
        int64_t en = off[min(ic + 1 + lane, S)];
        {
            const auto rs = rows_of(ic, jc);
#pragma unroll
            for (int t = 0; t < V; ++t) x[t] = ld32(rs, voff, t * row_bytes);
        }
        while (ic + jc < sh.d1) {
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

            if (ne == 0) {
                // No segment ends here: every row continues the open segment.
#pragma unroll
                for (int t = 0; t < V; ++t) {
                    const uint32_t r = gv + t;
                    if ((int)r < rows) open = R::comb(open, R::lift(x[t], relbase + r));
                    x[t] = ld32(rsn, voff, t * row_bytes);
                }
                open_spread = G > 1;
                ic = icn;
                jc = jcn;
                continue;
            }

            // The open segment's partial so far, needed by group 0 only: the
            // groups' parts in group order when they are spread.
            acc_t carry = open;
            if (G > 1 && open_spread) {
#pragma unroll
                for (int m = L; m < 64; m <<= 1) {
                    const acc_t o = lane_get(carry, lane ^ m);
                    carry = (lane & m) ? R::comb(o, carry) : R::comb(carry, o);
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
            acc_t acc = R::id(), hacc = R::id();
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
                    hacc = acc;
                    hlen = len;
                } else if (fvalid) {
                    store_final<DT, OP, 1>(a, seg, f, &acc, base, len);
                }
                acc = R::id();
                ++seg;
                ++k;
                next_end = end_at(k);
            };

#pragma unroll
            for (int t = 0; t < V; ++t) {
                const uint32_t r = gv + t;
                while (next_end <= r) finish();
                if ((int)r < rows) acc = R::comb(acc, R::lift(x[t], relbase + r));
                x[t] = ld32(rsn, voff, t * row_bytes);
            }
            while (k < a_hi) finish();

            // Segmented inclusive scan over the groups; the carry enters at
            // group 0.  A group that finished a segment restarts the scan.
            acc_t xs = (g == 0 && !hh) ? R::comb(carry, acc) : acc;
            acc_t ex = carry;
            if constexpr (G > 1) {
                bool flag = hh;
#pragma unroll
                for (int o = L; o < 64; o <<= 1) {
                    const int src = (lane - o) & 63;
                    const bool pf = lane_get(flag, src);
                    const acc_t px = lane_get(xs, src);
                    if (lane >= o) {
                        if (!flag) xs = R::comb(px, xs);
                        flag = flag || pf;
                    }
                }
                const acc_t prev = lane_get(xs, (lane - L) & 63);
                if (g != 0) ex = prev;
            }
            if (hh && fvalid) {
                const acc_t hv = R::comb(ex, hacc);
                if (sh.split_head && hseg == sh.i0) a.hval[wave * a.F + f] = R::to_slot(hv);
                else store_final<DT, OP, 1>(a, hseg, f, &hv, base, hlen);
            }
            // The open segment after this chunk: group G-1's inclusive value,
            // parked in group 0.
            if constexpr (G > 1) {
                const acc_t last = lane_get(xs, (G - 1) * L + c);
                open = g == 0 ? last : R::id();
            } else {
                open = xs;
            }
            open_spread = false;
            if constexpr (OP == OP_MEAN) open_start = jc + (int64_t)__builtin_amdgcn_readfirstlane(se[ne - 1]);

            ic = icn;
            jc = jcn;
            wave_lds_sync();
        }
        if (sh.has_tail) {
            acc_t t = open;
            if (G > 1 && open_spread) {
#pragma unroll
                for (int m = L; m < 64; m <<= 1) {
                    const acc_t o = lane_get(t, lane ^ m);
                    t = (lane & m) ? R::comb(o, t) : R::comb(t, o);
                }
            }
            if (g == 0 && fvalid) a.tval[wave * a.F + f] = R::to_slot(t);
        }
    }
    if (lane == 0) write_header(a, wave, sh);
}

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
__device__ __forceinline__ int flat_unit(int owner, int c) {
    return owner * 8 + (c ^ ((owner & 7) ^ ((owner >> 3) & 1)));
}

// Weight of a segment end against one 1-D element in the merge-path shares.
// An end costs an offsets read and an output store (and a row for min/max),
// and a chunk holds at most EC of them, against 4 bytes per element; with
// equal weights the shares over stretches of very short segments finish
// last.  Measured on 16M sorted Zipf keys (0.71M runs): sum 30.8 -> 27.3 us,
// min+row 37.1 -> 31.3 us from weight 1 to 8 (4: 29.2 / 33.4, 16: 27.6 /
// 30.6, 32: 28.3 / 35.6); 50M elements in 1M segments unchanged.
constexpr int kFlatEndWeight = 8;

template <int DT, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Red<DT, OP>::kMinMax ? 2 : 4)))
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
        for (int u = 0; u < V / 4; ++u) X[u] = ld128(rs, (uint32_t)(lane * 16), (uint32_t)(u * 1024));
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
        // dense stretches: further ends, fetched on demand
        for (int b = NB; more && b < EC / 64; ++b) take(b, off[min(ic + 1 + b * 64 + lane, S)]);
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
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int src = (lane - o) & 63;
            const bool pf = lane_get(fl, src);
            const lacc_t px = lane_get(xs, src);
            if (lane >= o) {
                if (!fl) xs = lcomb(px, xs);
                fl = fl || pf;
            }
        }
        const acc_t cm = to_max(carry);
        lacc_t ex = lane_get(xs, (lane - 1) & 63);
        bool fx = lane_get(fl, (lane - 1) & 63);
        if (lane == 0) {
            ex = lacc_t{};
            fx = false;
        }
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
// partials of those shares, in share order, into its head partial.
template <int DT, int OP>
__global__ __launch_bounds__(256) void seg_reduce_pass2(const KArgs a) {
    using P = P2<DT, OP>;
    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + wid;
    if (w >= a.NW) return;
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

constexpr int64_t kFallbackShares = 8192;
constexpr int64_t kMaxFeat = int64_t(1) << 24;


// Waves of `kernel` that fit on the device at once (CUs x resident
// workgroups x 4): one share per resident wave, so every wave streams its
// share from start to end without a second generation of workgroups.
static int64_t resident_waves(const void *kernel) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return kFallbackShares;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end()) return it->second;
    int cus = 0, blocks = 0;
    int64_t w = kFallbackShares;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0) == hipSuccess && cus > 0 &&
        blocks > 0)
        w = (int64_t)cus * blocks * 4;
    (void)hipGetLastError();
    cache[{dev, kernel}] = w;
    return w;
}

static int lanes_for(int64_t feat) {
    int64_t l = 2;
    while (l < feat && l < 64) l <<= 1;
    return (int)l;
}

template <int DT, int OP>
static const void *pick_kernel(int64_t feat) {
    if (feat == 1) return reinterpret_cast<const void *>(&seg_reduce_flat<DT, OP>);
    switch (lanes_for(feat)) {
    case 2: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 2, 16>);
    case 4: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 4, 16>);
    case 8: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 8, 16>);
    case 16: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 16, 16>);
    case 32: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 32, 24>);
    default: return reinterpret_cast<const void *>(&seg_reduce_rows<DT, OP, 64, 24>);
    }
}

// Shares per call: one per wave that fits on the device at once.
static int64_t shares_for(const void *kernel) {
    const int64_t o = shares_override();
    return ((o > 0 ? o : resident_waves(kernel)) + 3) / 4 * 4;  // whole workgroups of 4 waves
}

template <int DT, int OP>
static int run(KArgs k, hipStream_t st) {
    const void *kernel = pick_kernel<DT, OP>(k.F);
    const int64_t nw = shares_for(kernel);
    const size_t hdr_bytes = (size_t)nw * 4 * sizeof(int64_t);
    const size_t val_bytes = (size_t)nw * (size_t)k.F * sizeof(uint64_t);
    ScratchLease scratch;
    int rc = scratch_acquire(scratch, hdr_bytes + 2 * val_bytes, st);
    if (rc != SEGRED_OK) return rc;
    char *p = static_cast<char *>(scratch.ptr);
    k.NW = nw;
    k.hdr = reinterpret_cast<int64_t *>(p);
    k.hval = reinterpret_cast<uint64_t *>(p + hdr_bytes);
    k.tval = k.hval + (size_t)nw * (size_t)k.F;

    const dim3 grid((unsigned)(nw / 4)), block(256);
    void *params[] = {&k};
    hipError_t e = hipExtLaunchKernel(kernel, grid, block, params, 0, st, nullptr, timing_stop(true), 0);
    if (e == hipSuccess)
        e = hipExtLaunchKernel(reinterpret_cast<const void *>(&seg_reduce_pass2<DT, OP>), grid, block, params, 0,
                               st, nullptr, timing_stop(false), 0);
    return e == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

static int dispatch(int32_t dtype, int32_t op, const KArgs &k, hipStream_t st) {
    switch (dtype * 4 + op) {
    case DT_U32 * 4 + OP_SUM: return run<DT_U32, OP_SUM>(k, st);
    case DT_U32 * 4 + OP_MIN: return run<DT_U32, OP_MIN>(k, st);
    case DT_U32 * 4 + OP_MAX: return run<DT_U32, OP_MAX>(k, st);
    case DT_I32 * 4 + OP_SUM: return run<DT_I32, OP_SUM>(k, st);
    case DT_I32 * 4 + OP_MIN: return run<DT_I32, OP_MIN>(k, st);
    case DT_I32 * 4 + OP_MAX: return run<DT_I32, OP_MAX>(k, st);
    case DT_F32 * 4 + OP_SUM: return run<DT_F32, OP_SUM>(k, st);
    case DT_F32 * 4 + OP_MIN: return run<DT_F32, OP_MIN>(k, st);
    case DT_F32 * 4 + OP_MAX: return run<DT_F32, OP_MAX>(k, st);
    case DT_F32 * 4 + OP_MEAN: return run<DT_F32, OP_MEAN>(k, st);
    default: return SEGRED_ERR_UNSUPPORTED;
    }
}

template <int DT, int OP>
static int64_t shares_of(int64_t feat) {
    return shares_for(pick_kernel<DT, OP>(feat));
}

}  // namespace segred

using namespace segred;

extern "C" int64_t segred_get_shares(int32_t dtype, int32_t op, int64_t feat) {
    if (feat < 1) return -1;
    switch (dtype * 4 + op) {
    case DT_U32 * 4 + OP_SUM: return shares_of<DT_U32, OP_SUM>(feat);
    case DT_U32 * 4 + OP_MIN: return shares_of<DT_U32, OP_MIN>(feat);
    case DT_U32 * 4 + OP_MAX: return shares_of<DT_U32, OP_MAX>(feat);
    case DT_I32 * 4 + OP_SUM: return shares_of<DT_I32, OP_SUM>(feat);
    case DT_I32 * 4 + OP_MIN: return shares_of<DT_I32, OP_MIN>(feat);
    case DT_I32 * 4 + OP_MAX: return shares_of<DT_I32, OP_MAX>(feat);
    case DT_F32 * 4 + OP_SUM: return shares_of<DT_F32, OP_SUM>(feat);
    case DT_F32 * 4 + OP_MIN: return shares_of<DT_F32, OP_MIN>(feat);
    case DT_F32 * 4 + OP_MAX: return shares_of<DT_F32, OP_MAX>(feat);
    case DT_F32 * 4 + OP_MEAN: return shares_of<DT_F32, OP_MEAN>(feat);
    default: return -1;
    }
}

static int reduce_impl(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                       int64_t num_segments, const int64_t *num_segments_dev, int32_t op, void *out,
                       int64_t *arg_out, hipStream_t stream) {
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
    return dispatch(dtype, op, k, stream);
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
