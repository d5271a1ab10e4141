// Transposing lane-pair reductions with the gfx950 permlane swaps, shared by the
// LeapQuant refit and the packed-state kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace rsu {

// Sums (maxima) of x and y over lane pairs (l, l^16) (pair16) or (l, l^32) (pair32) with one
// lane swap: lanes whose bit 4 (bit 5) is clear get the result for x, the others for y.
// (v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the even rows
// of its second; v_permlane32_swap the upper half of the first with the lower half of the
// second; both layouts checked on gfx950.)
__device__ __forceinline__ float add_pair16(float x, float y) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned p0 = p[0], p1 = p[1];
    return __uint_as_float(p0) + __uint_as_float(p1);
}
__device__ __forceinline__ float add_pair32(float x, float y) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned p0 = p[0], p1 = p[1];
    return __uint_as_float(p0) + __uint_as_float(p1);
}
__device__ __forceinline__ float max_pair16(float x, float y) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned p0 = p[0], p1 = p[1];
    return fmaxf(__uint_as_float(p0), __uint_as_float(p1));
}
__device__ __forceinline__ float max_pair32(float x, float y) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned p0 = p[0], p1 = p[1];
    return fmaxf(__uint_as_float(p0), __uint_as_float(p1));
}

}  // namespace rsu
