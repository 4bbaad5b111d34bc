// keys.hpp -- element types, operations and the monotone order key shared
// by the library's kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace segred {

enum { DT_U32 = 0, DT_I32 = 1, DT_F32 = 2 };
enum { OP_SUM = 0, OP_MIN = 1, OP_MAX = 2, OP_MEAN = 3 };

// Monotone order key: u32 as is, i32 with the sign flipped, f32 with all bits
// flipped when negative and the sign set otherwise (graph-reduce, "Method").
template <int DT>
__device__ __forceinline__ uint32_t okey(uint32_t b) {
    if constexpr (DT == DT_U32) return b;
    else if constexpr (DT == DT_I32) return b ^ 0x80000000u;
    else return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);  // ~b if negative, else b | sign
}
template <int DT>
__device__ __forceinline__ uint32_t okey_inv(uint32_t k) {
    if constexpr (DT == DT_U32) return k;
    else if constexpr (DT == DT_I32) return k ^ 0x80000000u;
    else return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}

}  // namespace segred
