// wave.hpp -- wave64 helpers for gfx950 (CDNA4): lane queries, ballots and
// cross-lane moves for 32- and 64-bit values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segred {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Value of lane `src` (any lane may ask for any lane).
__device__ __forceinline__ uint32_t lane_get(uint32_t v, int src) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}
__device__ __forceinline__ uint64_t lane_get(uint64_t v, int src) {
    uint32_t lo = lane_get((uint32_t)v, src), hi = lane_get((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int64_t lane_get(int64_t v, int src) {
    return (int64_t)lane_get((uint64_t)v, src);
}
__device__ __forceinline__ double lane_get(double v, int src) {
    return __longlong_as_double((long long)lane_get((uint64_t)__double_as_longlong(v), src));
}
__device__ __forceinline__ float lane_get(float v, int src) {
    return __uint_as_float(lane_get(__float_as_uint(v), src));
}
__device__ __forceinline__ bool lane_get(bool v, int src) {
    return lane_get((uint32_t)v, src) != 0u;
}

// DPP moves (data-parallel primitives of the gfx9 family): a VALU operand
// taken from another lane of the same 16-lane row, or broadcast from the
// last lane of a row, in the instruction itself -- no LDS round trip as for
// ds_bpermute.  Lanes without a source (or in rows the row mask leaves out)
// receive `old`.
enum : int {
    kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118,
    kDppWaveShr1 = 0x138, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143
};
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float old, float v) {
    return __uint_as_float(dpp32<CTRL, ROW_MASK>(__float_as_uint(old), __float_as_uint(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_move(uint32_t old, uint32_t v) {
    return dpp32<CTRL, ROW_MASK>(old, v);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_move(uint64_t old, uint64_t v) {
    const uint32_t lo = dpp32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)v);
    const uint32_t hi = dpp32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_move(double old, double v) {
    return __longlong_as_double((long long)dpp_move<CTRL, ROW_MASK>((uint64_t)__double_as_longlong(old),
                                                                     (uint64_t)__double_as_longlong(v)));
}

// Segmented inclusive scan across the 64 lanes: on return lane l holds
// comb over the values of lanes k..l in lane order, k the last lane <= l
// whose flag was set (0 if none), and its flag is the OR of flags 0..l.
// comb(a, b) joins an earlier part a and a later part b; `id` is its
// identity.  Four in-row steps (shifts by 1, 2, 4, 8), then the rows' last
// lanes are broadcast into the next row (rows 1, 3) and lane 31 into rows 2
// and 3: six steps, all DPP.
template <typename T, typename Comb>
__device__ __forceinline__ void seg_scan_wave(T &x, bool &f, T id, Comb comb) {
#define SEGRED_SCAN_STEP(CTRL, RM)                                     \
    {                                                                  \
        const T px = dpp_move<CTRL, RM>(id, x);                        \
        const uint32_t pf = dpp32<CTRL, RM>(0u, f ? 1u : 0u);          \
        if (!f) x = comb(px, x);                                       \
        f = f || pf != 0u;                                             \
    }
    SEGRED_SCAN_STEP(kDppRowShr1, 0xF)
    SEGRED_SCAN_STEP(kDppRowShr2, 0xF)
    SEGRED_SCAN_STEP(kDppRowShr4, 0xF)
    SEGRED_SCAN_STEP(kDppRowShr8, 0xF)
    SEGRED_SCAN_STEP(kDppRowBcast15, 0xA)
    SEGRED_SCAN_STEP(kDppRowBcast31, 0xC)
#undef SEGRED_SCAN_STEP
}

// Make LDS writes of this wave visible to the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
    return v;  // values that are wave-uniform by construction
}

// The 64-bit value of lane idx (idx wave-uniform).  readlane returns a
// signed 32-bit int, so each half is taken as an unsigned word before it is
// widened: a low half with bit 31 set must not fill the upper half with ones.
__device__ __forceinline__ int64_t readlane64(int64_t v, int idx) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, idx);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), idx);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t readfirst(int64_t v) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Raw buffer access: a descriptor over [base, base + bytes).  A load whose
// lane offset (the VGPR offset plus the instruction's immediate offset) is at
// or past `bytes` returns 0 without touching memory, so a descriptor limited
// to the valid part of an array makes clamping unnecessary.  The scalar
// offset field (soffset) is added to the address but is not part of that
// range check on raw (stride 0) buffers, so every step through an array is
// put into the lane offset and soffset is always 0.  Descriptor word 3 is the
// gfx9-family raw 32-bit layout.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the streaming loads: non-temporal (nt).  Every element is
// read once, so nothing is gained by keeping it in the caches; with the hint
// a plain streaming read of 2 GiB ran at 6.7-7.0 TB/s on MI355X against
// 5.6-6.1 TB/s without it, for dword and dwordx4 loads alike.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, kStreamPolicy);
}

__device__ __forceinline__ uint2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    // Range checking is per dword, as for ld128.
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, kStreamPolicy);
    return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    // Range checking is per dword: a 16-byte unit cut by the limit returns its
    // in-range dwords and zeros for the rest.
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kStreamPolicy);
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// Bit t of m, sign-extended (all ones when set, else 0), as one v_bfe_i32.
// Written as an instruction so that the compiler keeps the AND with it
// instead of turning every use into a compare and a select (which costs an
// extra instruction and a 64-bit mask register per bit).
__device__ __forceinline__ uint32_t sbit(uint32_t m, int t) {
    uint32_t r;
    asm volatile("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(m), "n"(t));
    return r;
}

// Bitwise OR into a word of this wave's LDS (ds_or_b32).  It only sets flag
// bits, so the result does not depend on the order in which lanes arrive.
// (The segmented reduction, RLE and scan kernels use no other atomic; the
// scatter kernels and the search's validation word use global atomics.)
__device__ __forceinline__ void lds_or(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

}  // namespace segred
