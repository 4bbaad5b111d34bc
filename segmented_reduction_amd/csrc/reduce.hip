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
// The sequence is cut into NW equal shares, one per wave; a wave finds its
// share's (segment, row) coordinates with a 64-way search over the offsets.
// Long or skewed segments are therefore spread over many waves instead of
// serialising on one.
//
// Inside a share the wave walks chunks of CH items.  A chunk's rows are
// split into G groups of V consecutive rows; each group is L lanes wide and
// each lane holds VEC features of a row.  A group walks its rows in order,
// finishing every segment that ends inside it; a segmented scan over the G
// groups (cross-lane moves) completes segments cut by group and chunk
// boundaries.  Segments cut by a share boundary leave one partial per share
// in scratch; a second kernel combines them in share order.  No atomics are
// used anywhere, and every summation order is a fixed function of the
// offsets and NW, so results repeat bit for bit.
//
// Accumulators: float sums in float64 (rounded to float32 once), integer sums
// in wrapping uint32, min/max as a 64-bit word (order key << 32 | row code)
// whose integer max/min picks the extremum and, on equal keys, the lowest row
// (the packed value/row word of the graph-reduce README's "Method").
#include <type_traits>

#include "internal.hpp"
#include "wave.hpp"

namespace segred {

enum { DT_U32 = 0, DT_I32 = 1, DT_F32 = 2 };
enum { OP_SUM = 0, OP_MIN = 1, OP_MAX = 2, OP_MEAN = 3 };

struct KArgs {
    const uint32_t *values;  // element bits, row-major [rows, F]
    const int64_t *offsets;  // [S + 1]
    int64_t S, F, NW;
    uint32_t *out;           // [S, F]
    int64_t *arg;            // [S, F] or null
    int64_t *hdr;            // [NW][3]: head segment, tail segment, first row of the share
    uint64_t *hval;          // [NW][F]: partial of the share's first segment when it began earlier
    uint64_t *tval;          // [NW][F]: partial of the share's last segment when it continues
};

// Monotone order key: u32 as is, i32 with the sign flipped, f32 with all bits
// flipped when negative and the sign set otherwise (graph-reduce, "Method").
template <int DT>
__device__ __forceinline__ uint32_t okey(uint32_t b) {
    if constexpr (DT == DT_U32) return b;
    else if constexpr (DT == DT_I32) return b ^ 0x80000000u;
    else return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
template <int DT>
__device__ __forceinline__ uint32_t okey_inv(uint32_t k) {
    if constexpr (DT == DT_U32) return k;
    else if constexpr (DT == DT_I32) return k ^ 0x80000000u;
    else return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
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
                                            const typename Red<DT, OP>::acc_t *acc, int64_t base) {
    int64_t len = 0;
    if constexpr (OP == OP_MEAN) len = a.offsets[seg + 1] - a.offsets[seg];
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

// Pass 1: streaming reduction of every share.
//   VEC   features per lane (4: 16-byte loads, F % 4 == 0; 1: 4-byte loads)
//   L     lanes per row (power of two); G = 64 / L row groups per wave
//   V     consecutive rows per group per chunk; CH = G * V items per chunk
//   STAGE rows staged through LDS (F == 1: a lane's V consecutive elements)
template <int DT, int OP, int VEC, int L, int V, bool STAGE>
__global__ __launch_bounds__(256) void seg_reduce_pass1(const KArgs a) {
    using R = Red<DT, OP>;
    using acc_t = typename R::acc_t;
    constexpr int G = 64 / L;
    constexpr int CH = G * V;
    constexpr int FB = L * VEC;
    constexpr uint32_t kInf = 0xFFFFFFFFu;
    static_assert(!STAGE || (VEC == 1 && L == 1), "staging is for one-feature rows");
    struct AccV {
        acc_t v[VEC];
        __device__ static __forceinline__ AccV identity() {
            AccV r;
#pragma unroll
            for (int i = 0; i < VEC; ++i) r.v[i] = R::id();
            return r;
        }
    };

    __shared__ __attribute__((aligned(16))) uint32_t s_ends[4][CH];
    __shared__ __attribute__((aligned(16))) uint32_t s_vals[4][STAGE ? CH : 1];

    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane / L;
    const int c = lane % L;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t *off = a.offsets;
    const int64_t S = a.S;

    const int64_t o0 = off[0];
    const int64_t T = (off[S] - o0) + S;
    const int64_t D = (T + a.NW - 1) / a.NW;
    const int64_t d0 = min(wave * D, T);
    const int64_t d1 = min(d0 + D, T);

    // 64-way search for i(d) = max{ i in [0, S] : offsets[i] - o0 + i <= d }
    // at both ends of the share.
    int64_t lo0 = 0, hi0 = S, lo1 = 0, hi1 = S;
    while (lo0 < hi0 || lo1 < hi1) {
        const int64_t st0 = (hi0 - lo0 + 63) >> 6, st1 = (hi1 - lo1 + 63) >> 6;
        const int64_t p0 = lo0 + (int64_t)(lane + 1) * st0, p1 = lo1 + (int64_t)(lane + 1) * st1;
        const bool ok0 = lo0 < hi0 && p0 <= hi0, ok1 = lo1 < hi1 && p1 <= hi1;
        const int64_t k0 = ok0 ? off[p0] - o0 + p0 : 0;
        const int64_t k1 = ok1 ? off[p1] - o0 + p1 : 0;
        const int c0 = popc64(ballot(ok0 && k0 <= d0));
        const int c1 = popc64(ballot(ok1 && k1 <= d1));
        if (lo0 < hi0) {
            hi0 = min(hi0, lo0 + (int64_t)(c0 + 1) * st0 - 1);
            lo0 += (int64_t)c0 * st0;
        }
        if (lo1 < hi1) {
            hi1 = min(hi1, lo1 + (int64_t)(c1 + 1) * st1 - 1);
            lo1 += (int64_t)c1 * st1;
        }
    }
    const int64_t i0 = lo0, j0 = d0 - lo0, i1 = lo1, j1 = d1 - lo1;
    const bool split_head = i0 < i1 && off[i0] - o0 < j0;  // first segment began in an earlier share
    const bool has_tail = i1 < S && off[i1] - o0 < j1;      // last segment continues past the share
    const int64_t base = o0 + j0;

    for (int64_t fbase = 0; fbase < a.F; fbase += FB) {
        const int64_t f0 = fbase + (int64_t)c * VEC;
        const bool fvalid = f0 < a.F;
        acc_t carry[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) carry[v] = R::id();

        int64_t ic = i0, jc = j0;
        while (ic + jc < d1) {
            const int64_t items = min((int64_t)CH, d1 - ic - jc);
            const int64_t ends_left = min((int64_t)CH, i1 - ic);

            // Rows of a staged chunk are fetched before its length is known
            // (at most CH rows; the ones past the chunk are fetched again by
            // the next chunk).
            uint32_t sv[STAGE ? CH / 64 : 1];
            if constexpr (STAGE) {
                const int64_t rmax = min((int64_t)CH, j1 - jc);
                const uint32_t *src = a.values + (o0 + jc);
#pragma unroll
                for (int u = 0; u < CH / 64; ++u) {
                    const int r = u * 64 + lane;
                    sv[u] = r < rmax ? src[r] : 0u;
                }
            }

            // Segment ends inside this chunk: end k (row position e relative
            // to jc) is one of the first `items` items iff e + k + 1 <= items.
            int ne = 0;
            for (int b = 0; b < CH; b += 64) {
                const int k = b + lane;
                const bool valid = k < ends_left;
                const int64_t e = valid ? off[ic + 1 + k] - o0 - jc : 0;
                const bool cond = valid && e + k + 1 <= items;
                const int cnt = popc64(ballot(cond));
                if (cond) s_ends[wid][k] = (uint32_t)e;
                ne += cnt;
                if (cnt < 64) break;
            }
            const int rows = (int)(items - ne);
            if constexpr (STAGE) {
#pragma unroll
                for (int u = 0; u < CH / 64; ++u) s_vals[wid][u * 64 + lane] = sv[u];
            }
            wave_lds_sync();

            // Group g owns rows [gV, gV + V) and the ends at positions
            // (gV, gV + V] (group 0 also those at 0).
            const uint32_t gv = (uint32_t)(g * V);
            const int a_lo = g == 0 ? 0 : count_le(s_ends[wid], ne, gv);
            const int a_hi = count_le(s_ends[wid], ne, gv + V);

            uint32_t x[V][VEC];
            if constexpr (STAGE) {
#pragma unroll
                for (int t = 0; t < V; t += 4) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(&s_vals[wid][gv + t]);
                    x[t][0] = q.x;
                    x[t + 1][0] = q.y;
                    x[t + 2][0] = q.z;
                    x[t + 3][0] = q.w;
                }
            } else {
#pragma unroll
                for (int t = 0; t < V; ++t) {
                    const int r = (int)gv + t;
                    const int64_t idx = (o0 + jc + r) * a.F + f0;
                    if (r < rows && fvalid) {
                        if constexpr (VEC == 4) {
                            const uint4 q = *reinterpret_cast<const uint4 *>(a.values + idx);
                            x[t][0] = q.x;
                            x[t][1] = q.y;
                            x[t][2] = q.z;
                            x[t][3] = q.w;
                        } else {
                            x[t][0] = a.values[idx];
                        }
                    } else {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) x[t][v] = 0u;
                    }
                }
            }

            // Walk the group's rows in order.
            AccV acc = AccV::identity(), hacc = AccV::identity();
            bool hh = false;  // this group finished at least one segment
            int64_t hseg = 0;
            int k = a_lo;
            int64_t seg = ic + a_lo;
            uint32_t next_end = k < a_hi ? s_ends[wid][k] : kInf;
            const uint32_t relbase = (uint32_t)(jc - j0);

            auto finish = [&]() __attribute__((always_inline)) {
                if (!hh) {
                    hh = true;
                    hseg = seg;
                    hacc = acc;
                } else if (fvalid) {
                    store_final<DT, OP, VEC>(a, seg, f0, acc.v, base);
                }
                acc = AccV::identity();
                ++seg;
                ++k;
                next_end = k < a_hi ? s_ends[wid][k] : kInf;
            };

#pragma unroll
            for (int t = 0; t < V; ++t) {
                const uint32_t r = gv + t;
                while (next_end <= r) finish();
                if ((int)r < rows) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc.v[v] = R::comb(acc.v[v], R::lift(x[t][v], relbase + r));
                }
            }
            while (k < a_hi) finish();

            // Segmented inclusive scan over the groups; the chunk carry enters
            // at group 0.  A group that finished a segment restarts the scan.
            bool flag = hh;
            acc_t xs[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) xs[v] = (g == 0 && !flag) ? R::comb(carry[v], acc.v[v]) : acc.v[v];
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
            acc_t ex[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const acc_t prev = lane_get(xs[v], (lane - L) & 63);
                ex[v] = g == 0 ? carry[v] : prev;
            }
            if (hh && fvalid) {
                acc_t hv[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) hv[v] = R::comb(ex[v], hacc.v[v]);
                if (split_head && hseg == i0) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) a.hval[wave * a.F + f0 + v] = R::to_slot(hv[v]);
                } else {
                    store_final<DT, OP, VEC>(a, hseg, f0, hv, base);
                }
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) carry[v] = lane_get(xs[v], (G - 1) * L + c);

            ic += ne;
            jc += rows;
            wave_lds_sync();
        }
        if (has_tail && fvalid) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) a.tval[wave * a.F + f0 + v] = R::to_slot(carry[v]);
        }
    }
    if (lane == 0) {
        a.hdr[wave * 3 + 0] = split_head ? i0 : -1;
        a.hdr[wave * 3 + 1] = has_tail ? i1 : -1;
        a.hdr[wave * 3 + 2] = base;
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
    const int64_t s = a.hdr[w * 3 + 0];
    if (s < 0) return;

    const int64_t *off = a.offsets;
    const int64_t o0 = off[0];
    const int64_t T = (off[a.S] - o0) + a.S;
    const int64_t D = (T + a.NW - 1) / a.NW;
    const int64_t first = (off[s] - o0 + s) / D;  // share holding the segment's first row
    int64_t len = 0;
    if constexpr (OP == OP_MEAN) len = off[s + 1] - off[s];

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
                    bs[u] = a.hdr[(t + u * cols) * 3 + 2];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = P::comb(acc, P::from(q[u], bs[u]));
            }
            for (; t < w; t += cols) acc = P::comb(acc, P::from(a.tval[t * a.F + f], a.hdr[t * 3 + 2]));
        }
        for (int m = fp; m < 64; m <<= 1) {
            const P o = acc.get(lane ^ m);
            acc = (lane & m) ? P::comb(o, acc) : P::comb(acc, o);
        }
        if (cc == 0 && valid) {
            acc = P::comb(acc, P::from(a.hval[w * a.F + f], a.hdr[w * 3 + 2]));
            uint32_t ob;
            int64_t ab;
            acc.bits(len, ob, ab);
            a.out[s * a.F + f] = ob;
            if (Red<DT, OP>::kMinMax && a.arg) a.arg[s * a.F + f] = ab;
        }
    }
}

// ------------------------------------------------------------------ host side

enum Variant { VAR_FLAT, VAR_VEC4, VAR_VEC1 };

struct Plan {
    Variant var;
    int lanes;  // lanes per row (VEC4)
    int64_t shares;
};

constexpr int64_t kDefaultShares = 8192;

static int lanes_for_vec4(int64_t feat) {
    int64_t q = feat / 4, l = 1;
    while (l < q && l < 64) l <<= 1;
    return (int)l;
}

static Plan make_plan(const void *values, int64_t feat, const void *out, const int64_t *arg) {
    Plan p;
    if (feat == 1) {
        p.var = VAR_FLAT;
        p.lanes = 1;
    } else if (feat % 4 == 0 && aligned(values, 16) && aligned(out, 16) && (!arg || aligned(arg, 16))) {
        p.var = VAR_VEC4;
        p.lanes = lanes_for_vec4(feat);
    } else {
        p.var = VAR_VEC1;
        p.lanes = 64;
    }
    const int64_t o = shares_override();
    p.shares = ((o > 0 ? o : kDefaultShares) + 3) / 4 * 4;  // whole workgroups of 4 waves
    return p;
}

template <int DT, int OP, int VEC, int L, int V, bool STAGE>
static void launch_pass1(const KArgs &k, int64_t blocks, hipStream_t st) {
    hipLaunchKernelGGL((seg_reduce_pass1<DT, OP, VEC, L, V, STAGE>), dim3((unsigned)blocks), dim3(256), 0, st, k);
}

template <int DT, int OP>
static int run(const Plan &p, const KArgs &k, hipStream_t st) {
    const int64_t blocks = p.shares / 4;
    const int slot = timing_begin(st);
    switch (p.var) {
    case VAR_FLAT: launch_pass1<DT, OP, 1, 1, 16, true>(k, blocks, st); break;
    case VAR_VEC1: launch_pass1<DT, OP, 1, 64, 32, false>(k, blocks, st); break;
    case VAR_VEC4:
        switch (p.lanes) {
        case 1: launch_pass1<DT, OP, 4, 1, 8, false>(k, blocks, st); break;
        case 2: launch_pass1<DT, OP, 4, 2, 8, false>(k, blocks, st); break;
        case 4: launch_pass1<DT, OP, 4, 4, 8, false>(k, blocks, st); break;
        case 8: launch_pass1<DT, OP, 4, 8, 8, false>(k, blocks, st); break;
        case 16: launch_pass1<DT, OP, 4, 16, 8, false>(k, blocks, st); break;
        case 32: launch_pass1<DT, OP, 4, 32, 8, false>(k, blocks, st); break;
        default: launch_pass1<DT, OP, 4, 64, 8, false>(k, blocks, st); break;
        }
        break;
    }
    timing_end(slot, st);
    if (hipGetLastError() != hipSuccess) return SEGRED_ERR_HIP;
    hipLaunchKernelGGL((seg_reduce_pass2<DT, OP>), dim3((unsigned)blocks), dim3(256), 0, st, k);
    if (hipGetLastError() != hipSuccess) return SEGRED_ERR_HIP;
    return SEGRED_OK;
}

static int dispatch(int32_t dtype, int32_t op, const Plan &p, const KArgs &k, hipStream_t st) {
    switch (dtype * 4 + op) {
    case DT_U32 * 4 + OP_SUM: return run<DT_U32, OP_SUM>(p, k, st);
    case DT_U32 * 4 + OP_MIN: return run<DT_U32, OP_MIN>(p, k, st);
    case DT_U32 * 4 + OP_MAX: return run<DT_U32, OP_MAX>(p, k, st);
    case DT_I32 * 4 + OP_SUM: return run<DT_I32, OP_SUM>(p, k, st);
    case DT_I32 * 4 + OP_MIN: return run<DT_I32, OP_MIN>(p, k, st);
    case DT_I32 * 4 + OP_MAX: return run<DT_I32, OP_MAX>(p, k, st);
    case DT_F32 * 4 + OP_SUM: return run<DT_F32, OP_SUM>(p, k, st);
    case DT_F32 * 4 + OP_MIN: return run<DT_F32, OP_MIN>(p, k, st);
    case DT_F32 * 4 + OP_MAX: return run<DT_F32, OP_MAX>(p, k, st);
    case DT_F32 * 4 + OP_MEAN: return run<DT_F32, OP_MEAN>(p, k, st);
    default: return SEGRED_ERR_UNSUPPORTED;
    }
}

}  // namespace segred

using namespace segred;

extern "C" int64_t segred_get_shares(int32_t dtype, int32_t op, int64_t feat) {
    (void)dtype;
    (void)op;
    (void)feat;
    const int64_t o = shares_override();
    return ((o > 0 ? o : kDefaultShares) + 3) / 4 * 4;
}

extern "C" int segred_reduce(const void *values, int32_t dtype, int64_t feat, const int64_t *offsets,
                             int64_t num_segments, int32_t op, void *out, int64_t *arg_out,
                             hipStream_t stream) {
    if (num_segments < 0 || feat < 1 || dtype < SEGRED_U32 || dtype > SEGRED_F32 || op < SEGRED_SUM ||
        op > SEGRED_MEAN)
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_MEAN && dtype != SEGRED_F32) return SEGRED_ERR_UNSUPPORTED;
    if (num_segments == 0) return SEGRED_OK;
    if (!values || !offsets || !out) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!aligned(values, 4) || !aligned(out, 4) || !aligned(offsets, 8) || (arg_out && !aligned(arg_out, 8)))
        return SEGRED_ERR_INVALID_ARGUMENT;
    if (op == SEGRED_SUM || op == SEGRED_MEAN) arg_out = nullptr;

    const Plan plan = make_plan(values, feat, out, arg_out);
    const int64_t nw = plan.shares;
    const size_t hdr_bytes = (size_t)nw * 3 * sizeof(int64_t);
    const size_t val_bytes = (size_t)nw * (size_t)feat * sizeof(uint64_t);
    void *scratch = nullptr;
    int rc = scratch_alloc(&scratch, hdr_bytes + 2 * val_bytes, stream);
    if (rc != SEGRED_OK) return rc;

    KArgs k;
    k.values = static_cast<const uint32_t *>(values);
    k.offsets = offsets;
    k.S = num_segments;
    k.F = feat;
    k.NW = nw;
    k.out = static_cast<uint32_t *>(out);
    k.arg = arg_out;
    k.hdr = static_cast<int64_t *>(scratch);
    k.hval = reinterpret_cast<uint64_t *>(static_cast<char *>(scratch) + hdr_bytes);
    k.tval = k.hval + (size_t)nw * (size_t)feat;

    rc = dispatch(dtype, op, plan, k, stream);
    scratch_free(scratch, stream);
    return rc;
}
