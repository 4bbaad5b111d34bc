// partition.hpp -- merge-path partition of (rows + segment ends) into equal
// shares, one per wave, found by a workgroup-cooperative search over the
// offsets.  Shared by the segmented reduction and the segmented scan.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "wave.hpp"

namespace segred {

// Item d is preceded by i(d) = max{ i in [0, S] : key(i) <= d } segment ends,
// key(i) = offsets[i] - o0 + CW * i (strictly increasing in i).  CW is the
// weight of a segment end in rows: with CW = 1 every row and every end is
// one item; a larger CW counts an end as CW items (an end costs more than a
// row when rows are single values), and a diagonal that falls inside an
// end's weight is moved back to just before that end (the end goes to the
// next share), so shares still split the merged sequence at valid points.  The four waves
// of a workgroup own four consecutive shares, so their five boundary
// diagonals lie close together and the workgroup searches for them jointly:
//   round A: 256 evenly spaced offsets (the same for every workgroup, so
//            they stay cached), which also give o0 and the item count T;
//   round B: 64 evenly spaced offsets over the range round A leaves for the
//            workgroup's first and last diagonal;
//   round C: each wave narrows its own two diagonals with 256-way rounds
//            (one round unless the workgroup's range is wider than 16K
//            ends); the last round probes consecutive offsets, which also
//            gives the key just past each diagonal's end, key(i(d) + 1).
// Round A is one cache line per probe and every workgroup asks for all of
// them at once: on MI355X 1,024 such probes took 3.4-6 us (the L2s' request
// rate, ~131K requests per XCD), 256 take about a quarter of that.  The
// workgroup-specific loads touch about 64 + 2 * 2 cache lines of the
// offsets, most of which its waves read again for their segment ends.
// Every probe is clamped into the array and loaded unconditionally (a load
// under a branch would be waited for inside the branch).  The key of the
// last probe at or below a diagonal is kept, which gives offsets[i(d)]
// without another load.

// A wave's share of the merged (rows + segment ends) sequence: items
// [d0, d1), i.e. segment ends [i0, i1) and rows [j0, j1) (rows relative to
// offsets[0]).
struct Share {
    int64_t o0, D, d0, d1, i0, j0, i1, j1;  // D in weighted items; d0 = i0 + j0, d1 = i1 + j1 (unweighted)
    int64_t cw;                             // weight of a segment end
    int64_t first_row; // first row of segment i0 (relative to offsets[0])
    int64_t tail_row;  // first row of segment i1 (relative to offsets[0])
    bool split_head;   // segment i0 ends in the share but began in an earlier one
    bool has_tail;     // segment i1 has rows in the share and continues past it
};

// Where d falls among N probes p_k = lo + k * step (k < N - 1) and
// p_{N-1} = hi whose raw offsets are in s[]: the last probe with key <= d
// (there is one) and its key; i(d) then lies in [lo', hi'].
struct Bracket {
    int64_t lo, hi, klo;
};
template <int N>
__device__ __forceinline__ int64_t probe_pos(int k, int64_t lo, int64_t step, int64_t hi) {
    return k == N - 1 ? hi : min(lo + (int64_t)k * step, hi);
}
template <int N, int CW = 1>
__device__ __forceinline__ Bracket bracket(const int64_t *s, int64_t lo, int64_t step, int64_t hi, int64_t o0,
                                           int64_t d, int lane) {
    constexpr int U = N / 64;
    int cnt = 0;
    int64_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = u * 64 + lane;
        kk[u] = s[k] - o0 + CW * probe_pos<N>(k, lo, step, hi);
        cnt += popc64(ballot(kk[u] <= d));
    }
    // cnt >= 1: probe 0 has key <= d
    const int last = cnt - 1, ul = last >> 6;
    int64_t klast = kk[0];
#pragma unroll
    for (int u = 1; u < U; ++u) klast = ul == u ? kk[u] : klast;
    Bracket b;
    b.klo = readlane64(klast, last & 63);
    b.lo = probe_pos<N>(last, lo, step, hi);
    b.hi = cnt >= N ? hi : probe_pos<N>(cnt, lo, step, hi) - 1;
    if (b.hi < b.lo) b.hi = b.lo;
    return b;
}

constexpr int kProbesA = 256, kProbesB = 64;

//
// `wave` is the share index (4 * share block + wave in the workgroup); every
// wave of the workgroup must call this together (it synchronises).  `gran`
// rounds the share size up to a multiple of itself (see D below).  A
// nonzero `period` (items per 64 KB of rows) moves the share size out of
// the band within period / 16 items of a multiple of period (see D below).
//
// SNAP moves each share boundary d onto the nearer edge of the block of the
// segment it falls in (block i = segment i's rows and its end item, items
// [key(i), key(i+1))) when that edge is at most D / 4 items away, so short
// segments are rarely cut; it is a function of d alone, so the two shares
// on either side of a boundary agree on it, and it keeps the boundaries in
// order.
template <bool SNAP = false, int CW = 1>
__device__ __forceinline__ Share find_share(const int64_t *off, int64_t S, int64_t NW, int64_t wave, int lane,
                                            int64_t *s_probe /* LDS [kProbesA], workgroup-wide */,
                                            int64_t min_share = 1, int64_t gran = 1, int64_t period = 0) {
    static_assert(!(SNAP && CW != 1), "snapping is defined for unit weights");
    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int64_t blk = wave >> 2;  // the workgroup's four shares are 4 * blk .. 4 * blk + 3

    // Round A (one probe per thread).
    const int64_t stepA = (S + kProbesA - 2) / (kProbesA - 1);
#pragma unroll
    for (int u = 0; u < kProbesA / 256; ++u) {
        const int k = u * 256 + tid;
        s_probe[k] = off[probe_pos<kProbesA>(k, 0, stepA, S)];
    }
    __syncthreads();
    const int64_t o0 = s_probe[0];
    const int64_t T = (s_probe[kProbesA - 1] - o0) + CW * S;
    // Shares of at least min_share items: small inputs use fewer waves (the
    // rest get empty shares and only write their header).  A share is a
    // whole number of granules of `gran` items, so that a wave can split its
    // share into `gran` equal parts that are also a uniform partition of the
    // whole sequence.
    const int64_t Dg = max((T + NW * gran - 1) / (NW * gran), (min_share + gran - 1) / gran);
    int64_t D = Dg * gran;
    // Waves that start whole multiples of 64 KB apart and stream at the same
    // pace stay aligned and load from the same memory channels at the same
    // time: on a few long segments the 32-feature team walk moved 0.59-0.67
    // of peak with shares of 1,024 or 1,032 rows, 0.76-0.78 with 1,040 and
    // 0.81-0.83 with 1,056.  Share sizes within 4 KB of rows of a multiple
    // of 64 KB grow to that distance; the waves past the last share get
    // empty ones.  (A function of T only, so the partition stays
    // a constant of the input.)
    if (period > 0 && D >= period) {
        const int64_t m = period / 16, r = D % period;
        if (r < m) D += m - r;
        else if (r > period - m) D += period - r + m;
        D = (D + gran - 1) / gran * gran;
    }
    const int64_t g0 = min(blk * 4 * D, T), g4 = min((blk * 4 + 4) * D, T);
    const int64_t d0 = min((blk * 4 + wid) * D, T), d1 = min(d0 + D, T);
    const Bracket a0 = bracket<kProbesA, CW>(s_probe, 0, stepA, S, o0, g0, lane);
    const Bracket a4 = bracket<kProbesA, CW>(s_probe, 0, stepA, S, o0, g4, lane);
    __syncthreads();  // every wave is done with round A

    // Round B over [L, H], which holds i(d) for every diagonal of the group.
    const int64_t L = a0.lo, H = a4.hi;
    const int64_t stepB = max((H - L + kProbesB - 2) / (kProbesB - 1), (int64_t)1);
    if (tid < kProbesB) s_probe[tid] = off[probe_pos<kProbesB>(tid, L, stepB, H)];
    __syncthreads();
    Bracket b0 = bracket<kProbesB, CW>(s_probe, L, stepB, H, o0, d0, lane);
    Bracket b1 = bracket<kProbesB, CW>(s_probe, L, stepB, H, o0, d1, lane);
    __syncthreads();  // the probe array is free from here on

    // Round C: 256-way rounds on both diagonals of this wave, probes j =
    // 1..256 at lo + j * st with st = ceil((hi - lo) / 255), so the probes
    // reach past hi and a step-1 round leaves probe n + 1 (n: the probes at
    // or below the diagonal) at the new lo + 1.  Kernels that need key(lo +
    // 1) -- the end of the block the diagonal falls in -- make one step-1
    // round even when round B has already fixed lo (NEXT).
    constexpr bool NEXT = SNAP || CW != 1;
    int64_t lo0 = b0.lo, hi0 = b0.hi, k0lo = b0.klo, k0nx = 0;
    int64_t lo1 = b1.lo, hi1 = b1.hi, k1lo = b1.klo, k1nx = 0;
    bool nx0 = !NEXT, nx1 = !NEXT;  // key(lo + 1) known, or not needed
    while (lo0 < hi0 || lo1 < hi1 || !nx0 || !nx1) {
        const bool go0 = lo0 < hi0 || !nx0, go1 = lo1 < hi1 || !nx1;
        const int64_t st0 = max((hi0 - lo0 + 254) / 255, (int64_t)1);
        const int64_t st1 = max((hi1 - lo1 + 254) / 255, (int64_t)1);
        int64_t k0[4], k1[4];
        bool ok0[4], ok1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = (int64_t)(u * 64 + lane + 1);
            const int64_t p0 = lo0 + j * st0, p1 = lo1 + j * st1;
            // probes past the bracket only matter as the next key (probe
            // hi + 1); the rest load hi + 1 again (same cache line)
            ok0[u] = go0 && p0 <= hi0;
            ok1[u] = go1 && p1 <= hi1;
            const int64_t q0 = min(min(p0, hi0 + 1), S), q1 = min(min(p1, hi1 + 1), S);
            k0[u] = off[q0] - o0 + CW * q0;
            k1[u] = off[q1] - o0 + CW * q1;
        }
        int n0 = 0, n1 = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            n0 += popc64(ballot(ok0[u] && k0[u] <= d0));
            n1 += popc64(ballot(ok1[u] && k1[u] <= d1));
        }
        // key of probe n (1-based, n <= 256), held by lane (n - 1) % 64 in
        // slot (n - 1) / 64
        auto key_of = [&](int64_t v0, int64_t v1, int64_t v2, int64_t v3, int n)
            __attribute__((always_inline)) -> int64_t {
            const int m = n - 1, u = m >> 6;
            const int64_t v = u == 0 ? v0 : u == 1 ? v1 : u == 2 ? v2 : v3;
            return readlane64(v, m & 63);
        };
        if (go0) {
            if (n0 > 0) k0lo = key_of(k0[0], k0[1], k0[2], k0[3], n0);
            hi0 = min(hi0, lo0 + (int64_t)(n0 + 1) * st0 - 1);
            lo0 += (int64_t)n0 * st0;
            if (st0 == 1) {  // n0 <= 255: probe n0 + 1 is at lo0 + 1 (or clamped to S)
                k0nx = key_of(k0[0], k0[1], k0[2], k0[3], n0 + 1);
                nx0 = true;
            }
        }
        if (go1) {
            if (n1 > 0) k1lo = key_of(k1[0], k1[1], k1[2], k1[3], n1);
            hi1 = min(hi1, lo1 + (int64_t)(n1 + 1) * st1 - 1);
            lo1 += (int64_t)n1 * st1;
            if (st1 == 1) {
                k1nx = key_of(k1[0], k1[1], k1[2], k1[3], n1 + 1);
                nx1 = true;
            }
        }
    }
    int64_t e0 = d0, e1 = d1;
    if constexpr (SNAP) {
        // key(i + 1) of each boundary's block (block S, the end of the
        // sequence, is never moved)
        const int64_t n0 = k0nx;
        const int64_t n1 = k1nx;
        const int64_t slack = D >> 2;
        auto snap = [&](int64_t d, int64_t i, int64_t klo, int64_t knext, int64_t &e, int64_t &ii, int64_t &kk)
            __attribute__((always_inline)) {
            e = d;
            ii = i;
            kk = klo;
            if (i >= S) return;
            if (d - klo <= slack && d - klo <= knext - d) {
                e = klo;
            } else if (knext - d <= slack) {
                e = knext;
                ii = i + 1;
                kk = knext;
            }
        };
        int64_t ii0, kk0, ii1, kk1;
        snap(d0, lo0, k0lo, n0, e0, ii0, kk0);
        snap(d1, lo1, k1lo, n1, e1, ii1, kk1);
        lo0 = ii0;
        k0lo = kk0;
        lo1 = ii1;
        k1lo = kk1;
    }
    // rows before each boundary; a weighted diagonal inside an end's weight
    // stops at the last row of that end's segment
    int64_t r0 = e0 - CW * lo0, r1 = e1 - CW * lo1;
    if constexpr (CW != 1) {
        // rows before end lo + 1 (read only when lo < S)
        const int64_t n0 = k0nx - CW * (lo0 + 1), n1 = k1nx - CW * (lo1 + 1);
        if (lo0 < S) r0 = min(r0, n0);
        if (lo1 < S) r1 = min(r1, n1);
    }
    // Everything here is the same in every lane; saying so lets the compiler
    // keep it in scalar registers (and build uniform buffer descriptors).
    Share sh;
    sh.cw = CW;
    sh.o0 = readfirst(o0);
    sh.D = readfirst(D);
    sh.i0 = readfirst(lo0);
    sh.j0 = readfirst(r0);
    sh.d0 = sh.i0 + sh.j0;
    sh.i1 = readfirst(lo1);
    sh.j1 = readfirst(r1);
    sh.d1 = sh.i1 + sh.j1;
    sh.first_row = readfirst(k0lo) - CW * sh.i0;  // offsets[i0] - o0
    sh.split_head = sh.i0 < sh.i1 && sh.first_row < sh.j0;
    sh.tail_row = readfirst(k1lo) - CW * sh.i1;  // offsets[i1] - o0
    sh.has_tail = sh.i1 < S && sh.tail_row < sh.j1;
    return sh;
}

}  // namespace segred
