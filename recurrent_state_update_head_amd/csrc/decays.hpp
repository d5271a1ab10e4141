// Per-key window decays of the record gates (LeapQuant, sec. 3.2: the cumulative decay
// Gamma_{j+1:l} of record j is the product of the gates of the records after it).
#pragma once
#include "rsu_device.hpp"

namespace rsu {

// In place over the staged gates G [n][128]: column thread c (< 128) replaces row i < n of
// column c with the product of the gates of rows i+1 .. n-1 (1 for the last row), multiplied
// from the newest row down, and returns the product of all n gates of the column. The column's
// gates are loaded together (one LDS round trip), so the scan is a chain of multiplies, not of
// dependent loads. The caller publishes the result with a barrier.
template <int kMax>
__device__ __forceinline__ float column_suffix_products(float* G, int n, int c) {
    float g[kMax];
#pragma unroll
    for (int i = 0; i < kMax; ++i) g[i] = i < n ? G[i * kD + c] : 1.f;
    float s = 1.f;
#pragma unroll
    for (int i = kMax - 1; i >= 0; --i) {
        if (i < n) G[i * kD + c] = s;
        s *= g[i];
    }
    return s;
}

}  // namespace rsu
