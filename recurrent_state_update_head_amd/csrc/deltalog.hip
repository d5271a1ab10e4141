// deltalog.hip -- dense fp32 base plus a bounded log of (a, b) factor pairs.
//
// DeltaLog, sec. 3.1 (Algorithm 1, eqs. 4-7): the state of a head is
//   S = D(lbar) Sbar + sum_{m<L} D(lbar - Lam_m) K_m U_m^T,   D(l) = diag(exp l),
// with lbar the log-decay accumulated since the last merge and Lam_m the value
// of lbar when entry m was appended. One decode step with gate g (lambda = ln g):
//   lbar' = lbar + lambda
//   p = (D(lambda) S)^T k = Sbar^T (e^{lbar'} k) + sum_m U_m (K_m . e^{lbar'-Lam_m} k)
//   b = beta (v - p),  a = k
//   y = S'^T q = Sbar^T (e^{lbar'} q) + sum_m U_m (K_m . e^{lbar'-Lam_m} q) + b (k . q)
// then either the pair is appended (eq. 5: K_L = a, U_L = b, Lam_L = lbar')
// or, when the log is full, the represented state plus a b^T is written back
// into Sbar (eq. 6) and lbar is reset.
//
// The base is swept once per step for both read vectors (same fp32 layout as
// the dense step); the key-side replay coefficients K_m . (...) are computed
// once per head in the preparation phase and shared by all value columns.
// Append steps only read the 64 KiB base; merge steps also write it. With
// per-slot live lengths (sec. 4 keeps the live length per request slot, so
// requests admitted at different times are at different points of their cycle),
// one call serves a mixed batch: an append pass, then a merge pass.
//
// RWKV6 (DeltaLog Table 1 and sec. 3.4: per-key decay, update pair (k, v)) takes the
// same steps without the delta read: b = v, and its value-side factors are stored in
// the input dtype (both factors bf16 for bf16 inputs, as the page's RWKV6 log keeps them).
#include <type_traits>

#include "kernels.hpp"
#include "rsu_device.hpp"

namespace rsu {

// Log entries are staged through registers into LDS in chunks of kChunk entries; the
// first chunk is issued before the base tile, so short logs cost one round trip.
constexpr int kChunk = 16;

// Metadata write counts (DeltaLog sec. 3.3: one writer per head commits K_log[L],
// Lam_log[L], lbar and L). A build with RSU_CHECK_METADATA defined adds one to a per-head
// counter for every element of those it writes (and of U_log[L]), so a test can check
// that each is written exactly once per step; the ordinary build counts nothing.
#ifdef RSU_CHECK_METADATA
__device__ unsigned meta_writes[kMetaCheckHeads * kMetaKinds];
__device__ __forceinline__ void meta_count(int h, int kind, unsigned n) {
    if (h < kMetaCheckHeads) atomicAdd(&meta_writes[h * kMetaKinds + kind], n);
}

hipError_t read_metadata_counts(unsigned* host, int64_t heads, hipStream_t stream) {
    void* dev = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&dev, HIP_SYMBOL(meta_writes))) return e;
    if (hipError_t e = hipStreamSynchronize(stream)) return e;
    const size_t bytes = sizeof(unsigned) * kMetaKinds * static_cast<size_t>(heads);
    if (hipError_t e = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost)) return e;
    return hipMemset(dev, 0, sizeof(unsigned) * kMetaKinds * kMetaCheckHeads);
}
#else
__device__ __forceinline__ void meta_count(int, int, unsigned) {}

hipError_t read_metadata_counts(unsigned*, int64_t, hipStream_t) { return hipErrorNotSupported; }
#endif

// Dynamic LDS of a step, in 32-bit words, for n staged entries (n = L for the
// batch-uniform calls, n = C for the per-slot call): Ek[n][128] (K_m, turned in
// place into exp(lbar' - Lam_m) K_m), Us[n][128] (U_m), Ls[n][128] (KDA) or Ls[n]
// rounded up to 4 (GDN), and for steps that may merge kd[128][Cp] (the transpose of
// Ek, Cp = C rounded up to 4).
__host__ __device__ constexpr int log_lds_floats(int n, int Cp, bool per_key, bool may_merge) {
    return 2 * n * kD + (per_key ? n * kD : ((n + 3) & ~3)) + (may_merge ? kD * Cp : 0);
}

enum LogMode { kAppendMode = 0, kMergeMode = 1, kSlotAppend = 2, kSlotMerge = 3 };

// kMode: append (batch-uniform L < C), merge (L == C), or one of the two passes of a
// per-slot step, where every head reads its own live length from Lslot[h] (clamped to
// [0, C]). The append pass serves the heads with L < C and leaves the others alone;
// the merge pass, launched after it, serves the heads with L == C and advances every
// Lslot[h]. Two passes keep the appends at the append kernel's register budget (the
// merge path holds the whole base tile through its update).
// kDelta: the delta rule's correction b = beta (v - p) (GDN, KDA); without it b = v
// (RWKV6). UT: the stored type of the value-side factors.
template <bool kPerKey, bool kDelta, int kMode, typename T, typename UT>
__global__ __launch_bounds__(kThreads) void log_step_kernel(
    int C, int L_uniform, int* __restrict__ Lslot, float* __restrict__ Sbase,
    float* __restrict__ lbar, T* __restrict__ Klog, UT* __restrict__ Ulog,
    float* __restrict__ Lam, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ gate, const float* __restrict__ beta,
    float* __restrict__ y) {
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ f32x4 row_vec[kD];              // (E k, E q, k, E), E = exp(lbar') per key row
    __shared__ f32x2 kq_row[kD];               // (k_r, q_r)
    __shared__ f32x2 coef[kMaxC];              // per entry (Ek_m . k, Ek_m . q)
    __shared__ float kq_part[2];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ro = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t ent0 = static_cast<size_t>(h) * C * kD;

    constexpr bool kSlots = kMode == kSlotAppend || kMode == kSlotMerge;
    constexpr bool merge = kMode == kMergeMode || kMode == kSlotMerge;
    int L = L_uniform;
    if constexpr (kSlots) {
        // One thread reads the live length and the workgroup takes it from LDS: Lslot[h]
        // is advanced below by thread 0, so no other thread may read it from memory
        // after that write (the barrier orders the one read before the one write).
        __shared__ int L_head;
        if (tid == 0) L_head = min(max(Lslot[h], 0), C);
        __syncthreads();
        L = L_head;
        if (kMode == kSlotAppend && L == C) return;  // merged by the second pass
        if (kMode == kSlotMerge && L < C) {          // appended by the first pass
            if (tid == 0) {
                Lslot[h] = L + 1;
                meta_count(h, kMetaL, 1);
            }
            return;
        }
    }
    const int n_lds = kSlots ? C : L;
    const int Cp = (C + 3) & ~3;
    float* Ek = dyn_lds;
    float* Us = Ek + n_lds * kD;
    float* Ls = Us + n_lds * kD;
    float* kd = Ls + (kPerKey ? n_lds * kD : ((n_lds + 3) & ~3));

    // ---- loads: the first chunk of log entries, inputs, the base tile, then the rest
    Stager<T, kChunk * kD> sk;
    Stager<UT, kChunk * kD> su;
    Stager<float, kPerKey ? kChunk * kD : 8> sl;
    auto issue = [&](int m0) {
        const int n = min(kChunk, L - m0) * kD;
        sk.load(Klog + ent0 + static_cast<size_t>(m0) * kD, n, tid);
        su.load(Ulog + ent0 + static_cast<size_t>(m0) * kD, n, tid);
        if constexpr (kPerKey) sl.load(Lam + ent0 + static_cast<size_t>(m0) * kD, n, tid);
    };
    auto land = [&](int m0) {
        sk.store(Ek + m0 * kD, tid);
        su.store(Us + m0 * kD, tid);
        if constexpr (kPerKey) sl.store(Ls + m0 * kD, tid);
    };
    issue(0);
    float lam_s = 0.f;
    if constexpr (!kPerKey)
        if (tid < L) lam_s = Lam[static_cast<size_t>(h) * C + tid];
    const f32x4 vv = load4_in(v, vec_off + col);
    const float bt = kDelta ? beta[h] : 1.f;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = kPerKey ? gate[vec_off + r] : gate[h];
    const float lb_old = kPerKey ? lbar[vec_off + r] : lbar[h];
    // loads complete in order: the preparation below waits for the first chunk and the
    // inputs while the base tile is still in flight
    float* Sh = Sbase + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) s[it] = stream_load(Sh + (row_block(it, wave) * 8 + ro) * kD + col);

    land(0);
    for (int m0 = kChunk; m0 < L; m0 += kChunk) {
        issue(m0);
        land(m0);
    }
    if constexpr (!kPerKey)
        if (tid < L) Ls[tid] = lam_s;
    __syncthreads();

    // ---- key-side preparation: thread r < 128 owns key row r
    const float lb_new = lb_old + logf(gr);
    if (first) {
        for (int m = 0; m < L; ++m) {
            const float lam = kPerKey ? Ls[m * kD + r] : Ls[m];
            const float e = expf(lb_new - lam) * Ek[m * kD + r];
            Ek[m * kD + r] = e;  // in place: row r belongs to this thread
            if (merge) kd[r * Cp + m] = e;
        }
        if (merge)
            for (int m = L; m < Cp; ++m) kd[r * Cp + m] = 0.f;
        const float E = expf(lb_new);
        row_vec[r] = f32x4{E * kr, E * qr, kr, E};
        kq_row[r] = f32x2{kr, qr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    __syncthreads();

    // ---- replay coefficients: the 16 lanes of a DPP row reduce one entry (8 rows each)
    {
        const int chunk = tid & 15;
        for (int m0 = 0; m0 < L; m0 += kThreads / 16) {
            const int m = m0 + (tid >> 4);
            f32x2 c = {0.f, 0.f};
            if (m < L) {
                const f32x4 e0 = *reinterpret_cast<const f32x4*>(Ek + m * kD + 8 * chunk);
                const f32x4 e1 = *reinterpret_cast<const f32x4*>(Ek + m * kD + 8 * chunk + 4);
                const f32x2* kqr = kq_row + 8 * chunk;
                c = e0.x * kqr[0] + e0.y * kqr[1] + e0.z * kqr[2] + e0.w * kqr[3] +
                    e1.x * kqr[4] + e1.y * kqr[5] + e1.z * kqr[6] + e1.w * kqr[7];
            }
            c.x = row16_sum(c.x);
            c.y = row16_sum(c.y);
            if (chunk == 0 && m < L) coef[m] = c;
        }
    }
    __syncthreads();

    // metadata: one writer per element (all reads of lbar / Lam / Lslot are done)
    if (first) {
        if (merge) {
            if (kPerKey || r == 0) {
                lbar[kPerKey ? vec_off + r : h] = 0.f;
                meta_count(h, kMetaLbar, 1);
            }
        } else {
            const size_t ent = static_cast<size_t>(h) * C + L;
            store_in(Klog, ent * kD + r, kr);
            meta_count(h, kMetaK, 1);
            if (kPerKey || r == 0) {
                Lam[kPerKey ? ent * kD + r : ent] = lb_new;
                lbar[kPerKey ? vec_off + r : h] = lb_new;
                meta_count(h, kMetaLam, 1);
                meta_count(h, kMetaLbar, 1);
            }
        }
        if (kMode == kSlotMerge && tid == 0) {
            Lslot[h] = 0;
            meta_count(h, kMetaL, 1);
        }
    }

    // ---- sweep of the base for both read vectors, plus the log entries
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[row_block(it, wave) * 8 + ro];
        if constexpr (kDelta) p1 += s[it] * rv.x;
        p2 += s[it] * rv.y;
    }
    for (int m = ro; m < L; m += 8) {
        const f32x2 c = coef[m];
        const f32x4 u = *reinterpret_cast<const f32x4*>(Us + m * kD + col);
        if constexpr (kDelta) p1 += u * c.x;
        p2 += u * c.y;
    }
    if constexpr (kDelta) p1 = sum_row_lanes(p1);
    p2 = sum_row_lanes(p2);
    const float kq = kq_part[0] + kq_part[1];
    const f32x4 b = kDelta ? bt * (vv - p1) : vv;
    if (ro == 0) {
        *reinterpret_cast<f32x4*>(y + vec_off + col) = p2 + b * kq;
        if (!merge) {
            store4_in(Ulog, ent0 + static_cast<size_t>(L) * kD + col, b);
            meta_count(h, kMetaU, 4);
        }
    }
    if (!merge) return;

    // ---- merge (eq. 6): Sbar <- D(lbar') Sbar + sum_m D(lbar'-Lam_m) K_m U_m^T + k b^T
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x4 rv = row_vec[row_block(it, wave) * 8 + ro];
        s[it] = s[it] * rv.w + rv.z * b;
    }
    for (int m0 = 0; m0 < L; m0 += 4) {
        f32x4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = (m0 + i < L) ? *reinterpret_cast<const f32x4*>(Us + (m0 + i) * kD + col)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(kd + (row_block(it, wave) * 8 + ro) * Cp + m0);
            s[it] += u[0] * e.x + u[1] * e.y + u[2] * e.z + u[3] * e.w;
        }
    }
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) stream_store(Sh + (row_block(it, wave) * 8 + ro) * kD + col, s[it]);
}

template <bool kPerKey, bool kDelta, int kMode, typename T>
static hipError_t launch_log_t(const StepArgs& a, const LogArgs& l, hipStream_t stream) {
    using UT = std::conditional_t<kDelta, float, T>;
    constexpr auto kernel = log_step_kernel<kPerKey, kDelta, kMode, T, UT>;
    constexpr bool may_merge = kMode == kMergeMode || kMode == kSlotMerge;
    const int n = (kMode == kSlotAppend || kMode == kSlotMerge) ? l.C : l.L;
    const size_t lds = sizeof(float) * log_lds_floats(n, (l.C + 3) & ~3, kPerKey, may_merge);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(float) * log_lds_floats(kMaxC, (kMaxC + 3) & ~3, kPerKey, may_merge)));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kernel, dim3(a.heads), dim3(kThreads), lds, stream,
                       l.C, l.L, l.Lslot, a.S, l.lbar, static_cast<T*>(l.Klog), static_cast<UT*>(l.Ulog), l.Lam,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <bool kPerKey, bool kDelta, typename T>
static hipError_t launch_log_m(const StepArgs& a, const LogArgs& l, int mode, hipStream_t stream) {
    if (mode == 2) {  // per-slot step: the append pass, then the merge pass on the same stream
        if (hipError_t e = launch_log_t<kPerKey, kDelta, kSlotAppend, T>(a, l, stream)) return e;
        return launch_log_t<kPerKey, kDelta, kSlotMerge, T>(a, l, stream);
    }
    return mode == kMergeMode ? launch_log_t<kPerKey, kDelta, kMergeMode, T>(a, l, stream)
                              : launch_log_t<kPerKey, kDelta, kAppendMode, T>(a, l, stream);
}

hipError_t launch_log(const StepArgs& a, const LogArgs& l, int mode, bool per_key, bool bf16,
                      hipStream_t stream) {
    if (per_key)
        return bf16 ? launch_log_m<true, true, bf16_t>(a, l, mode, stream)
                    : launch_log_m<true, true, float>(a, l, mode, stream);
    return bf16 ? launch_log_m<false, true, bf16_t>(a, l, mode, stream)
                : launch_log_m<false, true, float>(a, l, mode, stream);
}

hipError_t launch_rwkv6_log(const StepArgs& a, const LogArgs& l, int mode, bool bf16, hipStream_t stream) {
    return bf16 ? launch_log_m<true, false, bf16_t>(a, l, mode, stream)
                : launch_log_m<true, false, float>(a, l, mode, stream);
}

}  // namespace rsu
