// dense.hip -- one eager decode step on the dense fp32 state (GDN, KDA, RWKV6, RWKV7).
//
// Recurrence (LeapQuant, App. A, the GDN and KDA expansions, with beta carried
// by the correction): with g the gate (alpha repeated over the key rows for
// GDN, the per-key vector d for KDA),
//   p = S^T (g * k),  u = beta (v - p),  S <- Diag(g) S + k u^T,  y = S^T q.
// RWKV6 (DeltaLog, Table 1; App. A eq. 1 with read vector 0) has no delta read:
// u = v, with the per-key decay w as g.
// The readout is taken from the updated state; it is evaluated in the same pass
// as p through the identity S_new^T q = S^T (g * q) + u (k . q), so the state
// is loaded once, reduced once (two column sums at the same time), updated in
// registers and stored once: 64 KiB in and 64 KiB out per head per step.
// Non-temporal 128-bit loads and stores and the XCD-grouped head order
// (head_of_block) were chosen by measurement on MI355X.
#include "kernels.hpp"
#include "rsu_device.hpp"

namespace rsu {

template <bool kPerKey, bool kDelta, typename T>
__global__ __launch_bounds__(kThreads) void dense_step_kernel(
    float* __restrict__ S, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ gate, const float* __restrict__ beta,
    float* __restrict__ y) {
    // per wave, per key row: (g*k, g*q, k, g); each wave stages its own copy, so the
    // four waves of a head run without a workgroup barrier
    __shared__ f32x4 row_vec[kThreads / 64][kD];

    const int h = head_of_block(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ro = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;

    // key-side inputs (lane -> key rows 2*lane, 2*lane + 1), then the whole state tile
    const f32x2 k2 = load2_in(k, vec_off + 2 * lane);
    const f32x2 q2 = load2_in(q, vec_off + 2 * lane);
    const float alpha = kPerKey ? 1.f : gate[h];
    const f32x2 g2 = kPerKey ? *reinterpret_cast<const f32x2*>(gate + vec_off + 2 * lane) : f32x2{alpha, alpha};
    const f32x4 vv = load4_in(v, vec_off + col);
    const float b = kDelta ? beta[h] : 1.f;

    float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        s[it] = stream_load(Sh + (row_block(it, wave) * 8 + ro) * kD + col);

    row_vec[wave][2 * lane] = f32x4{g2.x * k2.x, g2.x * q2.x, k2.x, g2.x};
    row_vec[wave][2 * lane + 1] = f32x4{g2.y * k2.y, g2.y * q2.y, k2.y, g2.y};
    const float kq = wave_sum(k2.x * q2.x + k2.y * q2.y);
    wave_lds_sync();

    // column sums over this thread's 16 rows, then over the 8 row lanes
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[wave][row_block(it, wave) * 8 + ro];
        if constexpr (kDelta) p += s[it] * rv.x;
        r += s[it] * rv.y;
    }
    if constexpr (kDelta) p = sum_row_lanes(p);
    r = sum_row_lanes(r);

    const f32x4 u = kDelta ? b * (vv - p) : vv;
    if (ro == 0) *reinterpret_cast<f32x4*>(y + vec_off + col) = r + u * kq;

#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[wave][row_block(it, wave) * 8 + ro];
        const float g = kPerKey ? rv.w : alpha;
        stream_store(Sh + (row_block(it, wave) * 8 + ro) * kD + col, s[it] * g + rv.z * u);
    }
}

// RWKV7 (LeapQuant, App. A, models with a separate erase direction): the erase sub-step
// reads S along a * kappa and the output reads the result along q; both reads come
// from the old state, so one sweep gives p = S^T (a * kappa) and r = S^T (w * q), and
//   u = 0 - p,  S <- Diag(w) S + kappa u^T + k v^T,  y = r + u (kappa . q) + v (k . q):
// the state crosses HBM once in and once out, as in the single-record step.
template <typename T>
__global__ __launch_bounds__(kThreads) void rwkv7_step_kernel(
    float* __restrict__ S, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ kappa, const float* __restrict__ w, const float* __restrict__ a,
    float* __restrict__ y) {
    // per wave, per key row: (a * kappa, w * q, kappa, w) and k
    __shared__ f32x4 row_vec[kThreads / 64][kD];
    __shared__ float krow[kThreads / 64][kD];

    const int h = head_of_block(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ro = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;

    const f32x2 k2 = load2_in(k, vec_off + 2 * lane);
    const f32x2 q2 = load2_in(q, vec_off + 2 * lane);
    const f32x2 c2 = load2_in(kappa, vec_off + 2 * lane);
    const f32x2 w2 = *reinterpret_cast<const f32x2*>(w + vec_off + 2 * lane);
    const f32x2 a2 = *reinterpret_cast<const f32x2*>(a + vec_off + 2 * lane);
    const f32x4 vv = load4_in(v, vec_off + col);

    float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        s[it] = stream_load(Sh + (row_block(it, wave) * 8 + ro) * kD + col);

    row_vec[wave][2 * lane] = f32x4{a2.x * c2.x, w2.x * q2.x, c2.x, w2.x};
    row_vec[wave][2 * lane + 1] = f32x4{a2.y * c2.y, w2.y * q2.y, c2.y, w2.y};
    krow[wave][2 * lane] = k2.x;
    krow[wave][2 * lane + 1] = k2.y;
    const float cq = wave_sum(c2.x * q2.x + c2.y * q2.y);
    const float kq = wave_sum(k2.x * q2.x + k2.y * q2.y);
    wave_lds_sync();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[wave][row_block(it, wave) * 8 + ro];
        p += s[it] * rv.x;
        r += s[it] * rv.y;
    }
    p = sum_row_lanes(p);
    r = sum_row_lanes(r);

    const f32x4 u = 0.f - p;
    if (ro == 0) *reinterpret_cast<f32x4*>(y + vec_off + col) = r + u * cq + vv * kq;

#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[wave][row_block(it, wave) * 8 + ro];
        stream_store(Sh + (row_block(it, wave) * 8 + ro) * kD + col, s[it] * rv.w + rv.z * u + krow[wave][row_block(it, wave) * 8 + ro] * vv);
    }
}

// DeltaProduct (LeapQuant, App. A, Table 4: n delta-rule sub-steps of eq. 1 per token),
// each sub-step with its own key k_i, value v_i and strength beta_i, the scalar gate alpha
// decaying the state once, in the first. Every read of the token comes from the old state:
// with P_i = S^T k_i and R = S^T q,
//   u_i = beta_i (v_i - alpha P_i - sum_{m<i} u_m (k_m . k_i)),
//   S <- alpha S + sum_i k_i u_i^T,   y = alpha R + sum_i u_i (k_i . q),
// so the state is swept once for kN + 1 column sums and crosses HBM once in and once out.
template <int kN, typename T>
__global__ __launch_bounds__(kThreads) void deltaproduct_step_kernel(
    float* __restrict__ S, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ y) {
    // per wave, per key row: the kN keys and q (each wave stages its own copy)
    __shared__ float rowk[kThreads / 64][kN + 1][kD];

    const int h = head_of_block(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ro = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t key_off = static_cast<size_t>(h) * kN * kD;

    f32x2 kk[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) kk[i] = load2_in(k, key_off + i * kD + 2 * lane);
    const f32x2 q2 = load2_in(q, vec_off + 2 * lane);
    const float al = alpha[h];

    float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        s[it] = stream_load(Sh + (row_block(it, wave) * 8 + ro) * kD + col);

#pragma unroll
    for (int i = 0; i < kN; ++i) {
        rowk[wave][i][2 * lane] = kk[i].x;
        rowk[wave][i][2 * lane + 1] = kk[i].y;
    }
    rowk[wave][kN][2 * lane] = q2.x;
    rowk[wave][kN][2 * lane + 1] = q2.y;
    // the key-key and key-query dot products, wave-uniform (kept in scalar registers)
    float kq[kN], kkd[kN][kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        kq[i] = uniform(wave_sum(kk[i].x * q2.x + kk[i].y * q2.y));
#pragma unroll
        for (int m = 0; m < i; ++m) kkd[m][i] = uniform(wave_sum(kk[m].x * kk[i].x + kk[m].y * kk[i].y));
    }
    wave_lds_sync();

    // kN + 1 column sums over this thread's 16 rows, then over the 8 row lanes
    f32x4 P[kN + 1];
#pragma unroll
    for (int i = 0; i <= kN; ++i) P[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const int row = row_block(it, wave) * 8 + ro;
#pragma unroll
        for (int i = 0; i <= kN; ++i) P[i] += s[it] * rowk[wave][i][row];
    }
#pragma unroll
    for (int i = 0; i <= kN; ++i) P[i] = sum_row_lanes(P[i]);

    // the sub-steps' corrections, in order (values and strengths loaded only now: held
    // through the sweep they would take 5 kN more registers)
    __builtin_amdgcn_sched_barrier(0);
    f32x4 vv[kN];
    float bt[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        vv[i] = load4_in(v, key_off + i * kD + col);
        bt[i] = beta[static_cast<size_t>(h) * kN + i];
    }
    f32x4 u[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        f32x4 p = al * P[i];
#pragma unroll
        for (int m = 0; m < i; ++m) p += u[m] * kkd[m][i];
        u[i] = bt[i] * (vv[i] - p);
    }
    if (ro == 0) {
        f32x4 o = al * P[kN];
#pragma unroll
        for (int i = 0; i < kN; ++i) o += u[i] * kq[i];
        *reinterpret_cast<f32x4*>(y + vec_off + col) = o;
    }

#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const int row = row_block(it, wave) * 8 + ro;
        f32x4 x = s[it] * al;
#pragma unroll
        for (int i = 0; i < kN; ++i) x += rowk[wave][i][row] * u[i];
        stream_store(Sh + row * kD + col, x);
    }
}

// Read+write copy with the same access pattern, for the practical HBM ceiling.
__global__ __launch_bounds__(kThreads) void copy_kernel(const float* __restrict__ src,
                                                        float* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(head_of_block(blockIdx.x, gridDim.x)) * kD * kD;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int off = (lane >> 3) * kD + wave * 32 + (lane & 7) * 4;
    if (base + kD * kD <= n) {
        f32x4 s[kRowsPerThread];
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) s[it] = stream_load(src + base + row_block(it, wave) * 8 * kD + off);
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) stream_store(dst + base + row_block(it, wave) * 8 * kD + off, s[it]);
    } else {
        for (int it = 0; it < kRowsPerThread; ++it) {
            const int64_t i = base + it * 8 * kD + off;
            if (i + 4 <= n) stream_store(dst + i, stream_load(src + i));
        }
    }
}

// Read-only and write-only streams over whole 128 x 128 fp32 tiles, with the dense step's
// tile pattern, head order and cache policy: the HBM read and write rates that bound a step
// which reads every tile once and writes it once. The read probe writes each tile's 128
// column sums (512 B per 64 KiB read) so that its loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const float* __restrict__ src,
                                                              float* __restrict__ sums) {
    const int64_t tile = head_of_block(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = wave * 32 + (lane & 7) * 4;
    const float* t = src + tile * kD * kD + (lane >> 3) * kD + col;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) s[it] = stream_load(t + row_block(it, wave) * 8 * kD);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) acc += s[it];
    acc = sum_row_lanes(acc);
    if ((lane >> 3) == 0) *reinterpret_cast<f32x4*>(sums + tile * kD + col) = acc;
}

__global__ __launch_bounds__(kThreads) void write_probe_kernel(float* __restrict__ dst, float value) {
    const int64_t tile = head_of_block(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    float* t = dst + tile * kD * kD + (lane >> 3) * kD + wave * 32 + (lane & 7) * 4;
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        stream_store(t + row_block(it, wave) * 8 * kD, f32x4{value, value, value, value});
}

template <bool kPerKey, bool kDelta, typename T>
static hipError_t launch_dense_t(const StepArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dense_step_kernel<kPerKey, kDelta, T>), dim3(a.heads), dim3(kThreads), 0, stream,
                       a.S, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

hipError_t launch_dense(const StepArgs& a, bool per_key, bool bf16, hipStream_t stream) {
    if (per_key)
        return bf16 ? launch_dense_t<true, true, bf16_t>(a, stream) : launch_dense_t<true, true, float>(a, stream);
    return bf16 ? launch_dense_t<false, true, bf16_t>(a, stream) : launch_dense_t<false, true, float>(a, stream);
}

hipError_t launch_rwkv6(const StepArgs& a, bool bf16, hipStream_t stream) {
    return bf16 ? launch_dense_t<true, false, bf16_t>(a, stream) : launch_dense_t<true, false, float>(a, stream);
}

hipError_t launch_rwkv7(const StepArgs& a, const void* kappa, const float* erase_rate, bool bf16,
                        hipStream_t stream) {
    if (bf16)
        hipLaunchKernelGGL(rwkv7_step_kernel<bf16_t>, dim3(a.heads), dim3(kThreads), 0, stream, a.S,
                           static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                           static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(kappa), a.gate, erase_rate,
                           a.y);
    else
        hipLaunchKernelGGL(rwkv7_step_kernel<float>, dim3(a.heads), dim3(kThreads), 0, stream, a.S,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), static_cast<const float*>(kappa), a.gate, erase_rate,
                           a.y);
    return hipGetLastError();
}

template <int kN, typename T>
static hipError_t launch_dp_t(const StepArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((deltaproduct_step_kernel<kN, T>), dim3(a.heads), dim3(kThreads), 0, stream, a.S,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dp_n(const StepArgs& a, int n, hipStream_t stream) {
    switch (n) {
        case 1: return launch_dp_t<1, T>(a, stream);
        case 2: return launch_dp_t<2, T>(a, stream);
        case 3: return launch_dp_t<3, T>(a, stream);
        default: return launch_dp_t<4, T>(a, stream);
    }
}

hipError_t launch_deltaproduct(const StepArgs& a, int n, bool bf16, hipStream_t stream) {
    return bf16 ? launch_dp_n<bf16_t>(a, n, stream) : launch_dp_n<float>(a, n, stream);
}

hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + kD * kD - 1) / (kD * kD);
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       src, dst, n);
    return hipGetLastError();
}

hipError_t launch_read_probe(const float* src, float* sums, int tiles, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(tiles), dim3(kThreads), 0, stream, src, sums);
    return hipGetLastError();
}

hipError_t launch_write_probe(float* dst, float value, int tiles, hipStream_t stream) {
    hipLaunchKernelGGL(write_probe_kernel, dim3(tiles), dim3(kThreads), 0, stream, dst, value);
    return hipGetLastError();
}

}  // namespace rsu
