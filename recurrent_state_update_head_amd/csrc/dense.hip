// dense.hip -- one eager decode step on the dense fp32 state (GDN and KDA).
//
// Recurrence (LeapQuant, App. A, the GDN and KDA expansions, with beta carried
// by the correction): with g the gate (alpha repeated over the key rows for
// GDN, the per-key vector d for KDA),
//   p = S^T (g * k),  u = beta (v - p),  S <- Diag(g) S + k u^T,  y = S^T q.
// The readout is taken from the updated state; it is evaluated in the same pass
// as p through the identity S_new^T q = S^T (g * q) + u (k . q), so the state
// is loaded once, reduced once (two column sums at the same time), updated in
// registers and stored once: 64 KiB in and 64 KiB out per head per step.
#include "kernels.hpp"
#include "rsu_device.hpp"

namespace rsu {

template <bool kPerKey, typename T>
__global__ __launch_bounds__(kThreads) void dense_step_kernel(
    float* __restrict__ S, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ gate, const float* __restrict__ beta,
    float* __restrict__ y) {
    // per key row: (g*k, g*q, k, g)
    __shared__ f32x4 row_vec[kD];
    __shared__ float kq_part[2];

    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ro = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;

    // key-side inputs (small) first, then the whole state tile
    float kr = 0.f, qr = 0.f, gr = 0.f;
    if (tid < kD) {
        kr = load_in(k, vec_off + tid);
        qr = load_in(q, vec_off + tid);
        gr = kPerKey ? gate[vec_off + tid] : gate[h];
    }
    const f32x4 vv = load4_in(v, vec_off + col);
    const float b = beta[h];
    const float alpha = kPerKey ? 1.f : gate[h];

    float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        s[it] = stream_load(Sh + (it * 8 + ro) * kD + col);

    if (tid < kD) {
        row_vec[tid] = f32x4{gr * kr, gr * qr, kr, gr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    __syncthreads();
    const float kq = kq_part[0] + kq_part[1];

    // column sums over this thread's 16 rows, then over the 8 row lanes
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[it * 8 + ro];
        p += s[it] * rv.x;
        r += s[it] * rv.y;
    }
    p = sum_row_lanes(p);
    r = sum_row_lanes(r);

    const f32x4 u = b * (vv - p);
    if (ro == 0) *reinterpret_cast<f32x4*>(y + vec_off + col) = r + u * kq;

#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[it * 8 + ro];
        const float g = kPerKey ? rv.w : alpha;
        stream_store(Sh + (it * 8 + ro) * kD + col, s[it] * g + rv.z * u);
    }
}

// Read+write copy with the same access pattern, for the practical HBM ceiling.
__global__ __launch_bounds__(kThreads) void copy_kernel(const float* __restrict__ src,
                                                        float* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kD * kD;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int off = (lane >> 3) * kD + wave * 32 + (lane & 7) * 4;
    if (base + kD * kD <= n) {
        f32x4 s[kRowsPerThread];
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) s[it] = stream_load(src + base + it * 8 * kD + off);
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) stream_store(dst + base + it * 8 * kD + off, s[it]);
    } else {
        for (int it = 0; it < kRowsPerThread; ++it) {
            const int64_t i = base + it * 8 * kD + off;
            if (i + 4 <= n) stream_store(dst + i, stream_load(src + i));
        }
    }
}

template <bool kPerKey, typename T>
static hipError_t launch_dense_t(const StepArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dense_step_kernel<kPerKey, T>), dim3(a.heads), dim3(kThreads), 0, stream,
                       a.S, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

hipError_t launch_dense(const StepArgs& a, bool per_key, bool bf16, hipStream_t stream) {
    if (per_key) return bf16 ? launch_dense_t<true, bf16_t>(a, stream) : launch_dense_t<true, float>(a, stream);
    return bf16 ? launch_dense_t<false, bf16_t>(a, stream) : launch_dense_t<false, float>(a, stream);
}

hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + kD * kD - 1) / (kD * kD);
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       src, dst, n);
    return hipGetLastError();
}

}  // namespace rsu
