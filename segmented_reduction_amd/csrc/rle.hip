// rle.hip -- run-length encoding of uint32 keys and the offsets of the runs
// (luma.gl "GPURunLengthEncode and GPUUnique": "What is run-length
// encoding?", "Why RLE matters for GPU grouping", "Contract").
//
// Position i starts a run iff i == 0 or keys[i] != keys[i-1].  Runs are
// numbered in position order; run r gets values[r] = keys[start],
// offsets[r] = start, lengths[r] = next start - start, offsets[count] = n.
//
// Three launches, no atomics: (1) each tile of 4096 keys counts its run
// starts, notes its first one and stores its start bits (one 64-bit ballot
// per wave and step, 512 bytes per tile); (2) one workgroup scans the tile
// counts (run index of each tile's first start) and the first starts from
// the right (the start that follows each tile); (3) each tile ranks its
// starts in position order from the stored bits (the keys are not read
// again) and writes values, offsets and lengths with consecutive lanes on
// consecutive runs, loading a key only where a run starts.
//
// The same three launches serve two relatives, chosen by a mode: the
// distinct adjacent values alone (same page, "GPUUnique": RLE's equality and
// order, values only, so no lengths, offsets or right-to-left scan), and
// offsets from segment-start flags (luma.gl "GPUSegmentedReduction",
// "Composition": position i starts a segment iff flags[i] != 0; offsets
// only, closed by n).
#include <algorithm>

#include "internal.hpp"
#include "scan.hpp"
#include "wave.hpp"

namespace segred {

constexpr int kRleThreads = 256;
constexpr int kRleKeysPerThread = 16;
constexpr int kRleTile = kRleThreads * kRleKeysPerThread;
constexpr int kScanThreads = 1024;

enum { MODE_RLE = 0, MODE_UNIQUE = 1, MODE_FLAGS = 2 };
// Unique and flags inputs: the tile count stays below 2^31 workgroups.
constexpr int64_t kMaxPositions = int64_t(1) << 40;

// Keys of one tile: thread (wave w, lane l) holds positions
// tile_start + u * 256 + w * 64 + l, u = 0..15, and whether each starts a run.
struct TileKeys {
    uint32_t k[kRleKeysPerThread];
    bool head[kRleKeysPerThread];
};

// The tile's keys arrive as 16-byte buffer loads (four per thread, all
// issued together, through a descriptor limited to the keys that exist:
// reads past n return 0) and go through LDS into the per-step layout above.
// A position's left neighbour is the key of the lane before (a DPP wave
// shift); lane 0 takes the previous wave's last key of the same step from
// LDS, and the tile's first position the key before the tile, the one
// global load besides the tile's own (its descriptor is empty for the first
// tile, whose position 0 starts a run anyway).  Sixteen 4-byte loads per
// thread and a load of the neighbour key per step took 16-17.5 us for 16M
// keys; the loads were the issue bottleneck.
template <int MODE>
__device__ __forceinline__ void load_tile(const uint32_t *keys, int64_t n, int64_t start, int tid, TileKeys &t,
                                          uint32_t *s_keys /* LDS [kRleTile] */) {
    const int lane = tid & 63, wid = tid >> 6;
    const int64_t avail = min((int64_t)kRleTile, n - start);
    const auto rs = make_rsrc(keys + start, (uint32_t)(avail * 4));
    constexpr int Q = kRleTile / (kRleThreads * 4);
    uint4 q[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) q[i] = ld128(rs, (uint32_t)((i * kRleThreads * 4 + tid * 4) * 4));
    uint32_t before = 0;
    if constexpr (MODE != MODE_FLAGS) {
        const auto rp = make_rsrc(keys + start - (start > 0 ? 1 : 0), start > 0 ? 4u : 0u);
        before = ld32(rp, 0);
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) *reinterpret_cast<uint4 *>(&s_keys[i * kRleThreads * 4 + tid * 4]) = q[i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) t.k[u] = s_keys[u * kRleThreads + tid];
    // Positions are taken relative to the tile (32-bit): those at or past
    // `lim` lie past n (only in the last tile), and position 0 of the first
    // tile starts a run whatever its key (`zero` is 0 there and no position
    // elsewhere).
    const uint32_t lim = (uint32_t)avail;
    if constexpr (MODE == MODE_FLAGS) {
        // a start is a nonzero flag: no neighbour is needed
#pragma unroll
        for (int u = 0; u < kRleKeysPerThread; ++u)
            t.head[u] = (uint32_t)(u * kRleThreads + tid) < lim && t.k[u] != 0u;
        return;
    }
    const uint32_t zero = start == 0 ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) {
        const int p0 = u * kRleThreads + wid * 64;  // the wave's first position in the tile at this step
        const uint32_t wave_prev = p0 > 0 ? s_keys[p0 > 0 ? p0 - 1 : 0] : before;
        const uint32_t prev = dpp_move<kDppWaveShr1>(wave_prev, t.k[u]);  // lane 0 keeps wave_prev
        const uint32_t p = (uint32_t)(p0 + lane);
        t.head[u] = p < lim && (t.k[u] != prev || p == zero);
    }
}

// Start bits of a tile: word (u, w) = the ballot of wave w at step u
// (bit l: position tile_start + u * 256 + w * 64 + l starts a run).
__device__ __forceinline__ int64_t mask_word(int64_t tile, int u, int w) {
    return (tile * kRleKeysPerThread + u) * 4 + w;
}

template <int MODE>
__global__ __launch_bounds__(kRleThreads) void rle_count(const uint32_t *keys, int64_t n, int64_t *tile_count,
                                                         int64_t *tile_first, uint64_t *tile_mask) {
    __shared__ int64_t s_cnt[4];
    __shared__ int64_t s_first[4];
    __shared__ __attribute__((aligned(16))) uint32_t s_keys[kRleTile];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t start = (int64_t)blockIdx.x * kRleTile;
    TileKeys t;
    load_tile<MODE>(keys, n, start, tid, t, s_keys);
    int64_t cnt = 0;
    uint64_t mine = 0;  // lane u keeps step u's ballot
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) {
        const uint64_t m = ballot(t.head[u]);
        cnt += popc64(m);
        if (lane == u) mine = m;
    }
    // the wave's first start: the lowest lane of the lowest step that has one
    const uint64_t steps = ballot(mine != 0ull);
    int64_t first = INT64_MAX;
    if (steps) {
        const int u0 = (int)__builtin_ctzll(steps);
        const uint64_t m0 = (uint64_t)readlane64((int64_t)mine, u0);
        first = start + u0 * kRleThreads + wid * 64 + (int)__builtin_ctzll(m0);
    }
    if (lane < kRleKeysPerThread) tile_mask[mask_word(blockIdx.x, lane, wid)] = mine;
    if (lane == 0) {
        s_cnt[wid] = cnt;
        s_first[wid] = first;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t c = 0, f = INT64_MAX;
        for (int w = 0; w < 4; ++w) {
            c += s_cnt[w];
            f = s_first[w] < f ? s_first[w] : f;
        }
        tile_count[blockIdx.x] = c;
        if (MODE == MODE_RLE) tile_first[blockIdx.x] = f;
    }
}

// One workgroup: run index of each tile's first start (exclusive scan of the
// tile counts) and the first start after each tile (exclusive minimum of the
// tiles' first starts, from the right).  Each thread takes K consecutive
// tiles of a batch of 1024 * K, so a batch costs one round of loads issued
// together, a short serial pass per thread and one block-wide scan.
// Only the RLE needs the right-to-left pass (it bounds the last run of a
// tile); the flags mode writes offsets[count] = n as the RLE does.
constexpr int kScanPer = 4;
template <int MODE>
__global__ __launch_bounds__(kScanThreads) void rle_scan(int64_t tiles, int64_t n, const int64_t *tile_count,
                                                         const int64_t *tile_first, int64_t *tile_base,
                                                         int64_t *tile_next, int64_t *count, int64_t *offsets) {
    constexpr int K = kScanPer;
    constexpr int64_t kBatch = (int64_t)kScanThreads * K;
    __shared__ int64_t s_tmp[2 * (kScanThreads / 64)];
    const int tid = threadIdx.x;

    // Left to right: run index of each tile's first start.
    int64_t running = 0;
    for (int64_t b = 0; b < tiles; b += kBatch) {
        int64_t v[K], in[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = b + (int64_t)tid * K + j;
            v[j] = tile_count[t < tiles ? t : 0];
            if (t >= tiles) v[j] = 0;
        }
        int64_t acc = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            in[j] = acc;
            acc += v[j];
        }
        int64_t total;
        const int64_t ex = block_inclusive_scan<kScanThreads, false>(acc, s_tmp, total) - acc;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = b + (int64_t)tid * K + j;
            if (t < tiles) tile_base[t] = running + ex + in[j];
        }
        running += total;
    }

    if (MODE != MODE_RLE) {
        if (tid == 0) {
            *count = running;
            if (MODE == MODE_FLAGS) offsets[running] = n;
        }
        return;
    }

    // Right to left: thread order runs from the last tile down (reversed
    // position r = tiles - 1 - t), so the exclusive minimum over reversed
    // positions before r, joined with the tiles further right, is the first
    // run start after tile t.
    int64_t right = n;
    for (int64_t b = 0; b < tiles; b += kBatch) {
        int64_t w[K], in[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = tiles - 1 - (b + (int64_t)tid * K + j);
            w[j] = tile_first[t >= 0 ? t : 0];
            if (t < 0) w[j] = INT64_MAX;
        }
        int64_t m = INT64_MAX;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            in[j] = m;
            m = w[j] < m ? w[j] : m;
        }
        int64_t total;
        const int64_t incl = block_inclusive_scan<kScanThreads, true>(m, s_tmp, total);
        // exclusive over the threads before this one: lane - 1 of this wave,
        // or for lane 0 the running minimum of the earlier waves (still in
        // s_tmp after the block scan)
        int64_t ex = lane_get(incl, ((tid & 63) - 1) & 63);
        if ((tid & 63) == 0) ex = tid == 0 ? INT64_MAX : s_tmp[kScanThreads / 64 + (tid >> 6) - 1];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t t = tiles - 1 - (b + (int64_t)tid * K + j);
            int64_t e = in[j] < ex ? in[j] : ex;
            e = e < right ? e : right;
            if (t >= 0) tile_next[t] = e < n ? e : n;
        }
        __syncthreads();
        right = total < right ? total : right;
    }
    if (tid == 0) {
        *count = running;
        offsets[running] = n;
    }
}

template <int MODE>
__global__ __launch_bounds__(kRleThreads) void rle_materialize(const uint32_t *keys, int64_t n,
                                                               const int64_t *tile_base, const int64_t *tile_next,
                                                               const uint64_t *tile_mask, uint32_t *values,
                                                               uint32_t *lengths, int64_t *offsets) {
    __shared__ uint32_t s_pos[kRleTile];
    __shared__ int s_wc[kRleKeysPerThread][4];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t start = (int64_t)blockIdx.x * kRleTile;
    // the tile's run index and following start, loaded with its start bits
    const int64_t rb = tile_base[blockIdx.x];
    const int64_t next = MODE == MODE_RLE ? tile_next[blockIdx.x] : 0;
    uint64_t m[kRleKeysPerThread];
    bool head[kRleKeysPerThread];
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) m[u] = tile_mask[mask_word(blockIdx.x, u, wid)];
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) {
        head[u] = (m[u] >> lane) & 1ull;
        if (lane == 0) s_wc[u][wid] = popc64(m[u]);
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
#pragma unroll
    for (int u = 0; u < kRleKeysPerThread; ++u) {
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wid ? s_wc[u][w] : 0;
            all += s_wc[u][w];
        }
        if (head[u]) {
            const int rank = base + before + popc64(m[u] & below);
            s_pos[rank] = (uint32_t)(u * kRleThreads + tid);
        }
        base += all;
    }
    __syncthreads();
    const int cnt = base;
    // Runs in batches of B per thread: every key load of a batch is issued
    // before its stores (through a descriptor over the tile's keys; runs past
    // cnt load the tile's first key and store nothing), so a tile of up to
    // 4,096 runs costs two round trips instead of one per 256 runs.
    constexpr int B = 8;
    const auto rk = make_rsrc(keys + start, (uint32_t)(min((int64_t)kRleTile, n - start) * 4));
    for (int q0 = 0; q0 < cnt; q0 += B * kRleThreads) {
        uint32_t p[B], v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int q = q0 + i * kRleThreads + tid;
            p[i] = q < cnt ? s_pos[q] : 0u;
        }
        if constexpr (MODE != MODE_FLAGS) {
#pragma unroll
            for (int i = 0; i < B; ++i) v[i] = ld32(rk, p[i] * 4u);
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int q = q0 + i * kRleThreads + tid;
            if (q < cnt) {
                const int64_t pos = start + p[i];
                if (MODE != MODE_FLAGS) values[rb + q] = v[i];
                if (MODE != MODE_UNIQUE) offsets[rb + q] = pos;
                if (MODE == MODE_RLE) {
                    const int64_t npos = q + 1 < cnt ? start + s_pos[q + 1] : next;
                    lengths[rb + q] = (uint32_t)(npos - pos);
                }
            }
        }
    }
}

}  // namespace segred

using namespace segred;

namespace segred {

// The three launches of one mode; scratch holds the per-tile records.
template <int MODE>
int rle_launch(const uint32_t *keys, int64_t n, uint32_t *values, uint32_t *lengths, int64_t *offsets,
               int64_t *count, hipStream_t stream) {
    const int64_t tiles = (n + kRleTile - 1) / kRleTile;
    ScratchLease scratch;
    const size_t words = (size_t)std::max<int64_t>(tiles, 1) * (4 + kRleKeysPerThread * 4);
    int rc = scratch_acquire(scratch, words * sizeof(int64_t), stream);
    if (rc != SEGRED_OK) return rc;
    int64_t *tcount = static_cast<int64_t *>(scratch.ptr);
    int64_t *tfirst = tcount + tiles;
    int64_t *tbase = tfirst + tiles;
    int64_t *tnext = tbase + tiles;
    uint64_t *tmask = reinterpret_cast<uint64_t *>(tnext + tiles);  // [tiles][16][4] start bits

    if (tiles > 0)
        timed_launch_ggl(true, rle_count<MODE>, dim3((unsigned)tiles), dim3(kRleThreads), 0, stream, keys, n, tcount,
                         tfirst, tmask);
    timed_launch_ggl(false, rle_scan<MODE>, dim3(1), dim3(kScanThreads), 0, stream, tiles, n,
                     (const int64_t *)tcount, (const int64_t *)tfirst, tbase, tnext, count, offsets);
    if (tiles > 0)
        timed_launch_ggl(true, rle_materialize<MODE>, dim3((unsigned)tiles), dim3(kRleThreads), 0, stream, keys, n,
                         (const int64_t *)tbase, (const int64_t *)tnext, (const uint64_t *)tmask, values, lengths,
                         offsets);
    return hipGetLastError() == hipSuccess ? SEGRED_OK : SEGRED_ERR_HIP;
}

}  // namespace segred

extern "C" int segred_offsets_from_rle(const uint32_t *sorted_keys, int64_t n, uint32_t *values,
                                       uint32_t *lengths, int64_t *offsets, int64_t *count,
                                       hipStream_t stream) {
    if (n < 0 || n > (int64_t)UINT32_MAX) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!values || !lengths || !offsets || !count || (n > 0 && !sorted_keys)) return SEGRED_ERR_INVALID_ARGUMENT;
    if ((sorted_keys && !aligned(sorted_keys, 4)) || !aligned(values, 4) || !aligned(lengths, 4) ||
        !aligned(offsets, 8) || !aligned(count, 8))
        return SEGRED_ERR_INVALID_ARGUMENT;
    return rle_launch<MODE_RLE>(sorted_keys, n, values, lengths, offsets, count, stream);
}

extern "C" int segred_unique(const uint32_t *keys, int64_t n, uint32_t *values, int64_t *count,
                             hipStream_t stream) {
    if (n < 0 || n > kMaxPositions) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!values || !count || (n > 0 && !keys)) return SEGRED_ERR_INVALID_ARGUMENT;
    if ((keys && !aligned(keys, 4)) || !aligned(values, 4) || !aligned(count, 8)) return SEGRED_ERR_INVALID_ARGUMENT;
    return rle_launch<MODE_UNIQUE>(keys, n, values, nullptr, nullptr, count, stream);
}

extern "C" int segred_offsets_from_flags(const uint32_t *flags, int64_t n, int64_t *offsets, int64_t *count,
                                         hipStream_t stream) {
    if (n < 0 || n > kMaxPositions) return SEGRED_ERR_INVALID_ARGUMENT;
    if (!offsets || !count || (n > 0 && !flags)) return SEGRED_ERR_INVALID_ARGUMENT;
    if ((flags && !aligned(flags, 4)) || !aligned(offsets, 8) || !aligned(count, 8)) return SEGRED_ERR_INVALID_ARGUMENT;
    return rle_launch<MODE_FLAGS>(flags, n, nullptr, nullptr, offsets, count, stream);
}
