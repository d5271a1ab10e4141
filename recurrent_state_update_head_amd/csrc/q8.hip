// q8.hip -- int8 state with per-key-row absmax scales, quantized once per window.
//
// Per-window quantization (LeapQuant, sec. 3.2, eqs. 3-4; App. B.2, eq. 9):
// the quantized window-start state S^_0 = (Z, a) stays fixed while the window's
// records (g_j, k_j, u_j) are buffered in higher precision. Step l of the
// window (0-based pos = l - 1) reads, for x = g_l * k_l (the delta read from
// the decayed state) and for x = q (the readout of the updated state),
//   S_{l-1}^T x = S^_0^T Gamma_{1:l-1} x + sum_{j<l} u_j (k_j . Gamma_{j+1:l-1} x)
// and S_l^T q = S_{l-1}^T (g_l q) + u_l (k_l . q). The int8 tile is swept once
// for both read vectors, with the row scale a_i / 127 and the cumulative decay
// folded into the read vectors, so dequantization costs one conversion per code.
// At l = W the full state S_W of eq. 4 is formed in registers, its per-row
// absmax taken and the tile requantized in place.
//
// Thread layout of the int8 tile (one 256-thread workgroup per head): lane l
// of wave w owns columns 4(l & 31) .. +3 and rows 8*it + 2w + (l >> 5),
// it = 0..15, i.e. one 32-bit word of codes per row; one wave-wide load covers
// two full rows (256 contiguous bytes).
#include "kernels.hpp"
#include "rsu_device.hpp"

namespace rsu {

__device__ __forceinline__ f32x4 unpack_i8x4(uint32_t w) {
    return f32x4{static_cast<float>(static_cast<int8_t>(w & 0xffu)),
                 static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu)),
                 static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu)),
                 static_cast<float>(static_cast<int8_t>(w >> 24))};
}

__device__ __forceinline__ uint32_t quant_code(float x, float scale) {
    float z = __builtin_rintf(x * scale);  // round to nearest, ties to even
    z = fminf(fmaxf(z, -127.f), 127.f);
    return static_cast<uint32_t>(static_cast<int32_t>(z)) & 0xffu;
}

__device__ __forceinline__ int q8_row(int it, int wave, int ro) { return 8 * it + 2 * wave + ro; }

// Requantize a head's fp32 tile held in registers (int8 layout) into Zh / Ah:
// a_i = max_j |S_ij|, scale = 127 / a_i (one correctly rounded fp32 division),
// z = clamp(rne(S * scale), -127, 127); a zero row gets a_i = 0 and z = 0.
// Every thread of the workgroup must call it (it contains a barrier).
__device__ __forceinline__ void requantize_tile(const f32x4 (&s)[kRowsPerThread], uint32_t* Zh,
                                                float* Ah, float* scale_s, int wave, int lane) {
    const int c4 = lane & 31, ro = lane >> 5;
    float amax[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const float m = fmaxf(fmaxf(fabsf(s[it].x), fabsf(s[it].y)), fmaxf(fabsf(s[it].z), fabsf(s[it].w)));
        amax[it] = half_wave_max(m);  // the 32 lanes of a half-wave hold one row
    }
    // lane c4 (< 16) of each half-wave publishes the scale of row (c4, wave, ro)
    float mine = 0.f;
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) mine = (c4 == it) ? amax[it] : mine;
    if (c4 < kRowsPerThread) {
        const int r = q8_row(c4, wave, ro);
        scale_s[r] = mine > 0.f ? __fdiv_rn(127.f, mine) : 0.f;
        Ah[r] = mine;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const int r = q8_row(it, wave, ro);
        const float sc = scale_s[r];
        const uint32_t w = quant_code(s[it].x, sc) | (quant_code(s[it].y, sc) << 8) |
                           (quant_code(s[it].z, sc) << 16) | (quant_code(s[it].w, sc) << 24);
        __builtin_nontemporal_store(w, Zh + r * (kD / 4) + c4);
    }
}

__global__ __launch_bounds__(kThreads) void q8_quantize_kernel(const float* __restrict__ S,
                                                               int8_t* __restrict__ Z,
                                                               float* __restrict__ A) {
    __shared__ float scale_s[kD];
    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        s[it] = stream_load(Sh + q8_row(it, wave, ro) * kD + 4 * c4);
    requantize_tile(s, reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD),
                    A + static_cast<size_t>(h) * kD, scale_s, wave, lane);
}

// Dynamic LDS of a window step, in 32-bit words: KE[Wp][128] (record keys, turned in
// place into the decayed keys E), Us[Wp][128] (record corrections), Gs[Wp][128]
// (record gates, KDA only) and, at the boundary, Zs[128][kZsStride] (the old codes
// re-laid out for the MFMA tiles; the padded row stride spreads the LDS banks).
constexpr int kZsStride = kD / 4 + 1;
__host__ __device__ constexpr int window_lds_floats(int Wp, bool per_key, bool boundary) {
    return (2 + (per_key ? 1 : 0)) * Wp * kD + (boundary ? kD * kZsStride : 0);
}

// Round-half-to-even of |w| <= 2^22 to an integer with one fp32 add: the sum's
// low mantissa bits are the integer. The code byte is the low byte of the sum's
// bits after clamping those bits to the codes of -127 .. 127.
__device__ __forceinline__ uint32_t code_byte(float w) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const int bits = __float_as_int(w + kMagic);
    const int lo = 0x4B400000 - 127, hi = 0x4B400000 + 127;
    return static_cast<uint32_t>(min(max(bits, lo), hi)) & 0xffu;
}

template <bool kPerKey, bool kBoundary, typename T>
__global__ __launch_bounds__(kThreads) void q8_window_kernel(
    int W, int pos, int8_t* __restrict__ Z, float* __restrict__ A, T* __restrict__ Kbuf,
    float* __restrict__ Ubuf, float* __restrict__ Gbuf, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ float dyn_lds[];
    __shared__ float gs_scalar[kMaxW];    // GDN: the records' gates
    __shared__ f32x2 rowv[kD];            // a_r/127 Gamma_{1:l} (k_r, q_r)
    __shared__ f32x2 kq_row[kD];          // (k_r, q_r)
    __shared__ f32x2 coef[kMaxW];         // per record (E_j . k, E_j . q)
    __shared__ f32x2 red[4][kD];          // per-wave column partials
    __shared__ float kq_part[2];
    __shared__ float zcoef[kBoundary ? kD : 1];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const int Wp = (W + 3) & ~3;
    float* KE = dyn_lds;
    float* Us = KE + Wp * kD;
    float* Gs = Us + Wp * kD;
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Gs + (kPerKey ? Wp * kD : 0));

    // ---- every load of the step is issued here: records and inputs first, then the
    // codes, so that the key-side preparation below only waits for the former while
    // the codes are still in flight (loads complete in order)
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    Stager<T, kMaxW * kD> sk;
    Stager<float, kMaxW * kD> su;
    sk.load(Kbuf + rec0, pos * kD, tid);
    su.load(Ubuf + rec0, pos * kD, tid);
    Stager<float, kPerKey ? kMaxW * kD : 8> sg;
    float g_rec = 1.f;
    if constexpr (kPerKey) sg.load(Gbuf + rec0, pos * kD, tid);
    else if (tid < pos) g_rec = Gbuf[static_cast<size_t>(h) * W + tid];
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = kPerKey ? gate[vec_off + r] : gate[h];
    const float ar = A[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    sk.store(KE, tid);
    su.store(Us, tid);
    if constexpr (kPerKey) sg.store(Gs, tid);
    else if (tid < pos) gs_scalar[tid] = g_rec;
    if (kBoundary)  // rows W..Wp-1 of Us meet zero coefficients at the boundary; keep them finite
        for (int i = W * kD + tid; i < Wp * kD; i += kThreads) Us[i] = 0.f;
    __syncthreads();

    // ---- key-side preparation: thread r < 128 walks the records of key row r backwards
    if (first) {
        float G = 1.f;  // product of the gates of the records after j (and before l)
        for (int j = pos - 1; j >= 0; --j) {
            KE[j * kD + r] *= G * gr;  // Gamma_{j+1:l} k_j at row r; row r belongs to this thread
            G *= kPerKey ? Gs[j * kD + r] : gs_scalar[j];
        }
        const float c0 = ar / 127.f * G * gr;  // a_r/127 Gamma_{1:l} at row r
        rowv[r] = f32x2{c0 * kr, c0 * qr};
        kq_row[r] = f32x2{kr, qr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
        if (kBoundary) {
            zcoef[r] = c0;
            KE[pos * kD + r] = kr;  // the current record: no decay after it
            for (int j = pos + 1; j < Wp; ++j) KE[j * kD + r] = 0.f;
        }
    }
    __syncthreads();

    // ---- record coefficients: the 16 lanes of a DPP row reduce one record (8 rows each)
    {
        const int chunk = tid & 15;
        for (int j0 = 0; j0 < pos; j0 += kThreads / 16) {
            const int j = j0 + (tid >> 4);
            f32x2 c = {0.f, 0.f};
            if (j < pos) {
                const f32x4 e0 = *reinterpret_cast<const f32x4*>(KE + j * kD + 8 * chunk);
                const f32x4 e1 = *reinterpret_cast<const f32x4*>(KE + j * kD + 8 * chunk + 4);
                const f32x2* kqr = kq_row + 8 * chunk;
                c = e0.x * kqr[0] + e0.y * kqr[1] + e0.z * kqr[2] + e0.w * kqr[3] +
                    e1.x * kqr[4] + e1.y * kqr[5] + e1.z * kqr[6] + e1.w * kqr[7];
            }
            c.x = row16_sum(c.x);
            c.y = row16_sum(c.y);
            if (chunk == 0 && j < pos) coef[j] = c;
        }
    }
    __syncthreads();

    // ---- one sweep of the int8 tile for both read vectors, plus the records
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x2 rv = rowv[q8_row(it, wave, ro)];
        const f32x4 zf = unpack_i8x4(zw[it]);
        p1 += zf * rv.x;
        p2 += zf * rv.y;
    }
    for (int j = 2 * wave + ro; j < pos; j += 8) {
        const f32x2 c = coef[j];
        const f32x4 u = *reinterpret_cast<const f32x4*>(Us + j * kD + 4 * c4);
        p1 += u * c.x;
        p2 += u * c.y;
    }
    p1 = f32x4{add_xor32(p1.x), add_xor32(p1.y), add_xor32(p1.z), add_xor32(p1.w)};
    p2 = f32x4{add_xor32(p2.x), add_xor32(p2.y), add_xor32(p2.z), add_xor32(p2.w)};
    if (ro == 0) {
        red[wave][4 * c4 + 0] = f32x2{p1.x, p2.x};
        red[wave][4 * c4 + 1] = f32x2{p1.y, p2.y};
        red[wave][4 * c4 + 2] = f32x2{p1.z, p2.z};
        red[wave][4 * c4 + 3] = f32x2{p1.w, p2.w};
    }
    __syncthreads();

    // ---- correction, output, and the record of this step (thread -> value column c == r)
    if (first) {
        const int c = tid;
        const f32x2 acc = red[0][c] + red[1][c] + red[2][c] + red[3][c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        if (kBoundary) {
            Us[pos * kD + c] = u;
        } else {
            const size_t rec = rec0 + static_cast<size_t>(pos) * kD;
            Ubuf[rec + c] = u;
            store_in(Kbuf, rec + c, kr);
            if (kPerKey) Gbuf[rec + c] = gr;
            else if (c == 0) Gbuf[static_cast<size_t>(h) * W + pos] = gr;
        }
    }
    if (!kBoundary) return;

    // ---- window boundary: S_W = Gamma_{1:W} S^_0 + sum_j Gamma_{j+1:W} k_j u_j^T, requantize.
    // The record sum is a [128 x Wp] . [Wp x 128] contraction per head, done on the
    // matrix cores as its transpose with v_mfma_f32_16x16x4f32 (A from lane l is
    // A[l%16][l/16], B is B[l/16][l%16], result i of lane l is D[4(l/16)+i][l%16]).
    // Tiles: wave w owns key rows 16*rt + (l%16), rt = 2w, 2w+1, and in value-column
    // tile ct the 4 columns 16*ct + 4(l/16) .. +3 -- one 32-bit word of codes.
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) Zs[q8_row(it, wave, ro) * kZsStride + c4] = zw[it];
    __syncthreads();
    const int lr = lane & 15, lq = lane >> 4;
    for (int a = 0; a < 2; ++a) {  // one 16-row tile band at a time: 8 accumulators live
        const int row = 16 * (2 * wave + a) + lr;
        const float zc = zcoef[row];
        f32x4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct] = unpack_i8x4(Zs[row * kZsStride + 4 * ct + lq]) * zc;
        for (int k0 = 0; k0 < Wp; k0 += 4) {
            const float bv = KE[(k0 + lq) * kD + row];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const float av = Us[(k0 + lq) * kD + 16 * ct + lr];
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[ct], 0, 0, 0);
            }
        }
        // per-row absmax: 32 values in this lane, then the 4 lanes l, l^16, l^32, l^48
        float m = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(acc[ct].x), fabsf(acc[ct].y)),
                               fmaxf(fabsf(acc[ct].z), fabsf(acc[ct].w))));
        m = max_xor16(m);
        float m0, m1;
        swap32(m, m0, m1);
        m = fmaxf(m0, m1);
        const float sc = m > 0.f ? __fdiv_rn(127.f, m) : 0.f;
        if (lq == 0) A[vec_off + row] = m;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const uint32_t w = code_byte(acc[ct].x * sc) | (code_byte(acc[ct].y * sc) << 8) |
                               (code_byte(acc[ct].z * sc) << 16) | (code_byte(acc[ct].w * sc) << 24);
            __builtin_nontemporal_store(w, Zh + row * (kD / 4) + 4 * ct + lq);
        }
    }
}

hipError_t launch_q8_quantize(int heads, const float* S, int8_t* Z, float* A, hipStream_t stream) {
    hipLaunchKernelGGL(q8_quantize_kernel, dim3(heads), dim3(kThreads), 0, stream, S, Z, A);
    return hipGetLastError();
}

template <bool kPerKey, bool kBoundary, typename T>
static hipError_t launch_window_kernel(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    const int Wp = (w.W + 3) & ~3;
    const size_t lds = sizeof(float) * window_lds_floats(Wp, kPerKey, kBoundary);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(q8_window_kernel<kPerKey, kBoundary, T>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(float) * window_lds_floats(kMaxW, kPerKey, kBoundary)));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((q8_window_kernel<kPerKey, kBoundary, T>), dim3(a.heads), dim3(kThreads), lds,
                       stream, w.W, w.pos, w.Z, w.A, static_cast<T*>(w.Kbuf), w.Ubuf, w.Gbuf,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <bool kPerKey, typename T>
static hipError_t launch_window_t(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    return w.pos == w.W - 1 ? launch_window_kernel<kPerKey, true, T>(a, w, stream)
                            : launch_window_kernel<kPerKey, false, T>(a, w, stream);
}

hipError_t launch_q8_window(const StepArgs& a, const WindowArgs& w, bool per_key, bool bf16,
                            hipStream_t stream) {
    if (per_key) return bf16 ? launch_window_t<true, bf16_t>(a, w, stream) : launch_window_t<true, float>(a, w, stream);
    return bf16 ? launch_window_t<false, bf16_t>(a, w, stream) : launch_window_t<false, float>(a, w, stream);
}

}  // namespace rsu
