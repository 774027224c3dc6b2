// Row-wide reductions over groups of 1, 2, 4, 8 or 16 consecutive lanes
// through DPP lane moves (no LDS traffic).
#pragma once

#include "common.hpp"

namespace ea {

// Row-wide (N consecutive lanes, N in {1, 2, 4, 8, 16}) all-reduce through
// DPP lane moves (no LDS traffic).  Every lane of the group ends with a
// bitwise-identical result (operands are combined commutatively in pairs).
template <int N, typename Op>
__device__ __forceinline__ float dpp_allreduce(float v, Op op) {
    if constexpr (N >= 2) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    if constexpr (N >= 4) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    if constexpr (N >= 8) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    if constexpr (N >= 16) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
    static_assert(N <= 16, "row groups of at most 16 lanes");
    return v;
}
template <int N>
__device__ __forceinline__ float row_sum(float v) {
    return dpp_allreduce<N>(v, [](float a, float b) { return a + b; });
}
template <int N>
__device__ __forceinline__ float row_max(float v) {
    return dpp_allreduce<N>(v, [](float a, float b) { return fmaxf(a, b); });
}

}  // namespace ea
