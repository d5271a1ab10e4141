// rsu_device.hpp -- device-side helpers shared by the gfx950 decode-step kernels.
//
// Thread layout used by every fp32-state kernel (one 256-thread workgroup per
// head, four wave64s):
//   wave w owns value columns [32w, 32w+32); lane l owns the 4 columns
//   32w + 4(l & 7) .. +3 and the key rows 8*it + (l >> 3), it = 0..15.
//   One wave-wide 128-bit load therefore covers 8 rows x 128 contiguous bytes,
//   and every column sum over the 128 key rows stays inside one wave: a thread
//   sums its 16 rows, then lanes l, l^8, l^16, l^32 combine (3 butterfly steps).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace rsu {

constexpr int kD = 128;            // d_k = d_v
constexpr int kThreads = 256;      // 4 x wave64 per head
constexpr int kRowsPerThread = 16; // fp32-state layout: 16 rows x 4 columns per thread

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

using bf16_t = uint16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Element loads of q / k / v in their storage type.
__device__ __forceinline__ float load_in(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }

// Four consecutive elements starting at a 4-element-aligned index.
__device__ __forceinline__ f32x4 load4_in(const float* p, size_t i) {
    return *reinterpret_cast<const f32x4*>(p + i);
}
__device__ __forceinline__ f32x4 load4_in(const bf16_t* p, size_t i) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + i);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}

// Two consecutive elements starting at an even index.
__device__ __forceinline__ f32x2 load2_in(const float* p, size_t i) {
    return *reinterpret_cast<const f32x2*>(p + i);
}
__device__ __forceinline__ f32x2 load2_in(const bf16_t* p, size_t i) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}

// ---- cooperative staging of a head's small arrays (records, log entries) into LDS
// as fp32. Every load of the block is issued before any LDS write, so staging costs
// one memory round trip. n (elements) must be a multiple of 8; at most
// kMaxElems elements.
template <typename T, int kMaxElems>
struct Stager {
    static constexpr int kPer = 16 / sizeof(T);                             // elements per 16 B
    static constexpr int kSlots = (kMaxElems / kPer + kThreads - 1) / kThreads;
    uint4 buf[kSlots];
    int n;
    __device__ __forceinline__ void load(const T* __restrict__ src, int n_elems, int tid) {
        n = n_elems;
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int c = tid + i * kThreads;
            // clamp the index instead of branching so the slot stays in registers
            const int cc = c * kPer < n ? c : 0;
            buf[i] = n > 0 ? *reinterpret_cast<const uint4*>(src + cc * kPer) : uint4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(float* __restrict__ dst, int tid) const {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int c = tid + i * kThreads;
            if (c * kPer >= n) continue;
            if constexpr (sizeof(T) == 4) {
                *reinterpret_cast<uint4*>(dst + c * kPer) = buf[i];
            } else {
                const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
                f32x4 lo = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                            __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
                f32x4 hi = {__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                            __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u)};
                *reinterpret_cast<f32x4*>(dst + c * kPer) = lo;
                *reinterpret_cast<f32x4*>(dst + c * kPer + 4) = hi;
            }
        }
    }
};

// Orders this wave's LDS writes before its later LDS reads of other lanes' data
// (no workgroup barrier: the four waves of a head never exchange data).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store of one element in the stored-key type (bf16 keys are copied bit-exactly).
__device__ __forceinline__ void store_in(float* p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_in(bf16_t* p, size_t i, float x) {
    p[i] = static_cast<bf16_t>(__float_as_uint(x) >> 16);
}

// Four consecutive elements at a 4-element-aligned index (bf16: values that came from
// bf16 inputs, copied bit-exactly).
__device__ __forceinline__ void store4_in(float* p, size_t i, f32x4 x) {
    *reinterpret_cast<f32x4*>(p + i) = x;
}
__device__ __forceinline__ void store4_in(bf16_t* p, size_t i, f32x4 x) {
    const uint2 w = {(__float_as_uint(x.x) >> 16) | (__float_as_uint(x.y) & 0xffff0000u),
                     (__float_as_uint(x.z) >> 16) | (__float_as_uint(x.w) & 0xffff0000u)};
    *reinterpret_cast<uint2*>(p + i) = w;
}

// State streaming: the state is touched once per step, so bypass cache retention.
__device__ __forceinline__ f32x4 stream_load(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void stream_store(float* p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

// Head processed by workgroup `bid` of a grid of `nblk`. Workgroups are dispatched
// round-robin over the 8 XCDs (bid % 8). Heads are regrouped so that each XCD
// streams runs of kXcdRun consecutive heads (256 KiB of fp32 state) instead of
// every 8th head: measured on MI355X, this raises the read+write HBM rate of the
// dense step by ~11%. Within each block of 8 * kXcdRun heads the map is a
// permutation; a ragged tail keeps the identity.
constexpr int kXcds = 8;
constexpr int kXcdRun = 4;
__device__ __forceinline__ int head_of_block(int bid, int nblk) {
    constexpr int grp = kXcds * kXcdRun;
    if (bid >= nblk / grp * grp) return bid;
    return bid / grp * grp + (bid % kXcds) * kXcdRun + (bid / kXcds) % kXcdRun;
}

// Row block (8 key rows, 4 KiB of fp32 state) that a wave of the fp32-state layout
// visits at iteration it: the four waves of a head start at row blocks 0, 4, 8 and 12,
// so the first loads of a workgroup cover four 4 KiB regions of the head instead of one.
// Measured on MI355X: the dense step 1% faster than with every wave starting at row 0.
__device__ __forceinline__ int row_block(int it, int wave) { return (it + 4 * wave) & 15; }

// ---- cross-lane reductions on the VALU (DPP and permlane swaps; no LDS round trip)
// Lane layouts checked on gfx950: quad_perm 0xB1 / 0x4E exchange lanes i^1 / i^2,
// row_ror:8 exchanges i^8 inside each row of 16 lanes, row_ror:4 rotates a row by
// 4, row_half_mirror reverses each group of 8 lanes (lane i reads lane i^7), and the
// two results of permlane16_swap(x, x) / permlane32_swap(x, x) hold x of lane i and
// of lane i^16 / i^32.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                                 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128, kDppHalfMirror = 0x141;

// The two results are copied to scalars before any bit cast: with this toolchain,
// __builtin_bit_cast of an element of the returned vector reads element 0.
__device__ __forceinline__ void swap16(float x, float& lo, float& hi) {
    const unsigned b = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    const unsigned p0 = p[0], p1 = p[1];
    lo = __uint_as_float(p0);
    hi = __uint_as_float(p1);
}
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
    const unsigned b = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const unsigned p0 = p[0], p1 = p[1];
    lo = __uint_as_float(p0);
    hi = __uint_as_float(p1);
}
__device__ __forceinline__ float add_xor16(float x) {
    float a, b;
    swap16(x, a, b);
    return a + b;
}
__device__ __forceinline__ float add_xor32(float x) {
    float a, b;
    swap32(x, a, b);
    return a + b;
}
__device__ __forceinline__ float max_xor16(float x) {
    float a, b;
    swap16(x, a, b);
    return fmaxf(a, b);
}

// Value of x in lane (src mod 64) of the same wave, for each lane's own src (a lane
// permute through the LDS crossbar; no LDS memory is used). The permute reads nothing
// from lanes that are switched off, so it must run with the whole wave active: it is
// never placed under a lane-dependent condition.
__device__ __forceinline__ float lane_gather(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// Value of x in lane i (a wave-uniform index) of the same wave.
__device__ __forceinline__ float lane_value(float x, int i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), i));
}

// Suffix products over lanes 0..kN-1 of a wave (kN a power of two, at most 32): lane
// l < kN gets x_l x_{l+1} ... x_{kN-1}; lanes past kN keep x. Every permute runs with the
// whole wave; the range check selects the factor after it.
template <int kN>
__device__ __forceinline__ float suffix_prod(float x, int lane) {
#pragma unroll
    for (int d = 1; d < kN; d <<= 1) {
        const float o = lane_gather(x, lane + d);
        x *= lane + d < kN ? o : 1.f;
    }
    return x;
}

// Exclusive suffix products of the same: lane l < kN gets x_{l+1} ... x_{kN-1} (1 for
// l = kN - 1), from the inclusive ones.
template <int kN>
__device__ __forceinline__ float suffix_prod_excl(float incl, int lane) {
    const float o = lane_gather(incl, lane + 1);
    return lane + 1 < kN ? o : 1.f;
}

// Sum over the 16 lanes of each DPP row (result in every lane of the row).
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppRor8>(x);
    x += dpp<kDppRor4>(x);
    return x;
}
// Max over the 32 lanes of each half-wave.
__device__ __forceinline__ float half_wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppRor8>(x));
    x = fmaxf(x, dpp<kDppRor4>(x));
    return max_xor16(x);
}
// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Sum over all 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float x) { return add_xor32(add_xor16(row16_sum(x))); }

// Sum over the lanes that differ only in lane bits 3..5 (the 8 row lanes of a
// column group in the fp32-state layout).
__device__ __forceinline__ float sum_row_lanes(float x) {
    x += dpp<kDppRor8>(x);
    return add_xor32(add_xor16(x));
}
__device__ __forceinline__ f32x4 sum_row_lanes(f32x4 x) {
    return f32x4{sum_row_lanes(x.x), sum_row_lanes(x.y), sum_row_lanes(x.z), sum_row_lanes(x.w)};
}

}  // namespace rsu
