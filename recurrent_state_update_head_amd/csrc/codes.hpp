// Packing of quantized codes, shared by the int8 and LeapQuant requantizers.
#pragma once

#include <cstdint>

namespace rsu {

// The low bytes of a, b, c, d as one word (a in byte 0): two byte permutes and an or.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

// A row (or column) whose maximum m is below 2^-64 is quantized after scaling it, and m, by
// 2^64: exact for every value, and qmax / m no longer overflows fp32 (a subnormal m would
// otherwise give an infinite scale and saturate every code). The factor for a maximum m:
constexpr float kTinyMax = 0x1p-64f, kTinyScale = 0x1p64f;
__device__ __forceinline__ float tiny_factor(float m) { return m < kTinyMax ? kTinyScale : 1.f; }

}  // namespace rsu
