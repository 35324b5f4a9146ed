// vla_reduce.h -- cross-lane sums over a row of adjacent lanes and over a wave
// (DPP: quad_perm, row_half_mirror, row_mirror, row_bcast), for kernels that
// hold one matrix row per TPR adjacent lanes.
#pragma once
#include "vla_chunk_parts.h"

namespace vla {
namespace chunk {

// sum over a row's TPR (4, 8 or 16) adjacent lanes, the same value in each
template <int TPR>
__device__ __forceinline__ float row_sum(float x)
{
    static_assert(TPR == 4 || TPR == 8 || TPR == 16, "rows of 4, 8 or 16 lanes");
    x += dpp<0xB1>(x);                               // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                               // quad_perm [2,3,0,1]
    if constexpr (TPR >= 8) x += dpp<0x141>(x);      // row_half_mirror
    if constexpr (TPR >= 16) x += dpp<0x140>(x);     // row_mirror
    return x;
}

// sum over the wave's 64 lanes (all active), as a wave-uniform value: row sums,
// then row 1 += row 0 and row 3 += row 2 (row_bcast:15), row 3 += row 1
// (row_bcast:31), and lane 63 read out
__device__ __forceinline__ float wave_sum(float x)
{
    x = row_sum<16>(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

}  // namespace chunk
}  // namespace vla
