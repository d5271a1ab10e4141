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
#include "codes.hpp"
#include "decays.hpp"

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
// a_i = max_j |S_ij|, scale = 127 / (a_i f_i) (one correctly rounded fp32 division, f_i =
// tiny_factor(a_i)), z = clamp(rne((S f_i) * scale), -127, 127); a zero row gets a_i = 0 and
// z = 0. scale_s receives (scale, f_i) per row. Every thread of the workgroup must call it (it
// contains a barrier).
__device__ __forceinline__ void requantize_tile(const f32x4 (&s)[kRowsPerThread], uint32_t* Zh,
                                                float* Ah, f32x2* scale_s, int wave, int lane) {
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
        const float f = tiny_factor(mine);
        scale_s[r] = f32x2{mine > 0.f ? __fdiv_rn(127.f, mine * f) : 0.f, f};
        Ah[r] = mine;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const int r = q8_row(it, wave, ro);
        const f32x2 sf = scale_s[r];
        const float sc = sf.x;
        const f32x4 x = s[it] * sf.y;  // exact
        const uint32_t w = quant_code(x.x, sc) | (quant_code(x.y, sc) << 8) |
                           (quant_code(x.z, sc) << 16) | (quant_code(x.w, sc) << 24);
        __builtin_nontemporal_store(w, Zh + r * (kD / 4) + c4);
    }
}

__global__ __launch_bounds__(kThreads) void q8_quantize_kernel(const float* __restrict__ S,
                                                               int8_t* __restrict__ Z,
                                                               float* __restrict__ A) {
    __shared__ f32x2 scale_s[kD];
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

// Eight consecutive elements of a key-side vector in their storage type, kept packed
// in registers until used (bf16: one 16-byte load; fp32: two).
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16_t> {
    uint32_t w[4];
    __device__ __forceinline__ void load(const bf16_t* p) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    }
    __device__ __forceinline__ float operator[](int e) const {
        return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    }
};
template <>
struct Raw8<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void load(const float* p) {
        lo = *reinterpret_cast<const f32x4*>(p);
        hi = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

// Per-key decays of a window's staged record keys, over all 256 threads of the workgroup:
// thread t takes key row t >> 1 and the records of one half, j = (t & 1) kHalf + e, so the
// two halves of a row sit in neighbouring lanes. load() issues the loads of the half's gates
// (records j >= n count as 1); apply() turns KE[j][row] into extra * (the product of the
// row's gates of the records after j) * KE[j][row] for every record j < n and returns the
// product of the gates of all n records at the row (in both lanes of the row).
template <int kHalf>
struct KeyDecays {
    float g[kHalf];
    __device__ __forceinline__ void load(const float* __restrict__ G, int n, int tid) {
        const int row = tid >> 1, j0 = (tid & 1) * kHalf;
#pragma unroll
        for (int e = 0; e < kHalf; ++e) {
            const int j = j0 + e;
            const float gj = G[static_cast<size_t>(j < n ? j : 0) * kD + row];  // slot clamped: in bounds
            g[e] = j < n ? gj : 1.f;
        }
    }
    __device__ __forceinline__ float apply(float* KE, int n, float extra, int tid) const {
        const int row = tid >> 1, upper = tid & 1, j0 = upper * kHalf;
        float mine = 1.f;
#pragma unroll
        for (int e = 0; e < kHalf; ++e) mine *= g[e];
        const float other = dpp<kDppXor1>(mine);      // the partner lane's half
        float s = extra * (upper ? 1.f : other);     // decay from the records after this half
#pragma unroll
        for (int e = kHalf - 1; e >= 0; --e) {
            const int j = j0 + e;
            if (j < n) KE[j * kD + row] *= s;
            s *= g[e];
        }
        return mine * other;
    }
};

// ---- one step inside the window (pos < W - 1): read S_{l-1} in both directions and
// append this step's record. The records never pass through LDS: the 16 lanes of a
// DPP row hold 8 keys each of one record and reduce its coefficients
// (Gamma_{j+1:l} k_j) . k and (Gamma_{j+1:l} k_j) . q in place, and the record
// corrections u_j are loaded straight into the registers of the row-owners that
// add c_j u_j to their column partials. Scalar gates (GDN) are multiplied from
// register copies (lane i of every wave holds g_i), so the step needs two
// workgroup barriers; per-key gates (KDA) are staged in LDS first and turned there into
// their suffix products per key column (two more).
template <bool kPerKey, int kWmax, typename T>
__global__ __launch_bounds__(kThreads) void q8_step_kernel(
    int W, int pos, const int8_t* __restrict__ Z, const float* __restrict__ A, T* __restrict__ Kbuf,
    float* __restrict__ Ubuf, float* __restrict__ Gbuf, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ __align__(16) float gs_lds[];     // KDA: the records' gates [pos][128]
    __shared__ f32x2 rowv[kD];            // a_r/127 Gamma_{1:l} (k_r, q_r)
    __shared__ f32x2 coef[kMaxW];         // per record (E_j . k, E_j . q)
    __shared__ f32x2 red[4][kD];          // per-wave column partials
    __shared__ float kq_part[2];
    constexpr int kKSlots = kWmax / 16;   // records per 16-lane group
    constexpr int kUSlots = kWmax / 8;    // records per row-owner

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5, owner = 2 * wave + ro;
    const int grp = tid >> 4, ch = tid & 15;  // record-key layout: group = record, 8 keys per lane
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;

    // ---- every load is issued first: record keys and corrections, gates, inputs, codes
    Raw8<T> kc[kKSlots];
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        const int j = grp + 16 * s;
        // unconditional, so that no branch makes the compiler wait for it (a branch around a
        // load ends in a wait for every load before it): a lane past the last record reads
        // slot 0, a slot group with no record at all reads this lane's own input keys (loaded
        // anyway, so no extra traffic); such keys are never used
        kc[s].load(16 * s < pos ? Kbuf + rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + 8 * ch : k + vec_off + 8 * ch);
    }
    f32x4 ur[kUSlots];
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        const int j = owner + 8 * m;
        // unconditional as the keys (a slot group with no record reads the lane's scales); a
        // clamped slot's values meet a zero coefficient
        ur[m] = *reinterpret_cast<const f32x4*>(8 * m < pos ? Ubuf + rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + 4 * c4
                                                           : A + vec_off + 4 * c4);
    }
    float g_lane = 1.f;  // GDN: lane i holds the gate of record i
    Stager<float, kPerKey ? kWmax * kD : 8> sg;
    if constexpr (kPerKey) sg.load(Gbuf + rec0, pos * kD, tid);
    else if (lane < pos) g_lane = Gbuf[static_cast<size_t>(h) * W + lane];
    Raw8<T> kch, qch;
    kch.load(k + vec_off + 8 * ch);
    qch.load(q + vec_off + 8 * ch);
    f32x4 gch_lo = {1.f, 1.f, 1.f, 1.f}, gch_hi = {1.f, 1.f, 1.f, 1.f};  // KDA: current gates of the 8 keys
    if constexpr (kPerKey) {
        gch_lo = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch);
        gch_hi = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch + 4);
    }
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = kPerKey ? gate[vec_off + r] : gate[h];
    const float ar = A[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    const uint32_t* Zh = reinterpret_cast<const uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    // ---- decays: G_s = prod of the record gates after record grp + 16 s (from the
    // newest down), Gall = prod of all record gates; the current gate comes on top
    float Gs[kKSlots][kPerKey ? 8 : 1];
    float Gall = 1.f;
    if constexpr (kPerKey) {  // the gates' suffix products per key column, in place
        sg.store(gs_lds, tid);
        __syncthreads();
        if (first) Gall = column_suffix_products<kWmax>(gs_lds, pos, r);
        __syncthreads();
    }
    if constexpr (!kPerKey) {
        // suffix scan over the record lanes (g = 1 from record pos on): the product of the
        // gates after each record, gathered for the records of this lane's groups
        const float Sfx = suffix_prod<kWmax>(g_lane, lane);
        const float E = suffix_prod_excl<kWmax>(Sfx, lane);
#pragma unroll
        for (int s = 0; s < kKSlots; ++s) Gs[s][0] = lane_gather(E, grp + 16 * s);
        Gall = lane_value(Sfx, 0);
    } else {
#pragma unroll
        for (int s = 0; s < kKSlots; ++s) {
            const int j = grp + 16 * s;
#pragma unroll
            for (int e = 0; e < 8; ++e) Gs[s][e] = 1.f;
            if (j >= pos) continue;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(gs_lds + j * kD + 8 * ch);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(gs_lds + j * kD + 8 * ch + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Gs[s][e] = lo[e];
                Gs[s][e + 4] = hi[e];
            }
        }
    }

    // ---- record coefficients, reduced over the 16 lanes of each group
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        if (16 * s >= pos) continue;
        const int j = grp + 16 * s;
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ge = kPerKey ? (e < 4 ? gch_lo[e] : gch_hi[e - 4]) : gr;
            const float ej = kc[s][e] * (Gs[s][kPerKey ? e : 0] * ge);  // Gamma_{j+1:l} k_j
            ck += ej * kch[e];
            cq += ej * qch[e];
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && j < pos) coef[j] = f32x2{ck, cq};
    }
    if (first) {
        const float c0 = ar * (1.f / 127.f) * Gall * gr;  // a_r/127 Gamma_{1:l} at row r
        rowv[r] = f32x2{c0 * kr, c0 * qr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
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
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        if (8 * m >= pos) continue;
        const int j = owner + 8 * m;
        const f32x2 c = j < pos ? coef[j] : f32x2{0.f, 0.f};
        p1 += ur[m] * c.x;
        p2 += ur[m] * c.y;
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
        const size_t rec = rec0 + static_cast<size_t>(pos) * kD;
        Ubuf[rec + c] = u;
        store_in(Kbuf, rec + c, kr);
        if (kPerKey) Gbuf[rec + c] = gr;
        else if (c == 0) Gbuf[static_cast<size_t>(h) * W + pos] = gr;
    }
}

// Dynamic LDS of the boundary step, in 32-bit words, for windows of up to kWmax records:
// KE[kWmax][128] (record keys, turned in place into the decayed keys E; zero after the
// last record), Us[kWmax][128] (record corrections; zero after the last) and
// Zs[128][kZsStride] (the codes re-laid out for the MFMA tiles, then the new codes on
// their way out; the padded row stride spreads the LDS banks). Per-key record gates are
// not staged: each key row's gates go from HBM straight into the registers of the thread
// that walks that row.
constexpr int kZsStride = kD / 4 + 1;
__host__ __device__ constexpr int boundary_lds_floats(int wmax) { return 2 * wmax * kD + kD * kZsStride; }

// Codes without a clamp, for the products w = x * fp32(127 / (m f)) of a row whose absmax is m,
// with f = tiny_factor(m) (1, or 2^64 for m below 2^-64): the code of w f, rounded half to even
// by the magic add inside one fma (|w f| <= 2^22: the sum's low mantissa bits are the integer,
// its low byte the code's two's complement). The product w is rounded to fp32 first, as the
// quantizer of a plain state decides it. w f is exact wherever w is normal (f is a power of
// two) and then equals fp32((x f) * fp32(127 / (m f))), the product for the scaled row; a
// subnormal w gives |w f| < 2^-62, code 0 either way. |x| <= m bounds |w f| by 127 (1 + 2^-24),
// which rounds to at most 127, so the integer is already a code (m = 0 gives w = 0).
// Non-finite rows give unspecified codes.
__device__ __forceinline__ uint32_t code_bits_in_range(float w, float f) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    return static_cast<uint32_t>(__float_as_int(__builtin_fmaf(w, f, kMagic)));
}
__device__ __forceinline__ uint32_t code_word_in_range(f32x4 w, float f) {
    return pack_low_bytes(code_bits_in_range(w.x, f), code_bits_in_range(w.y, f), code_bits_in_range(w.z, f),
                          code_bits_in_range(w.w, f));
}

// A raw buffer resource over n bytes at p (no stride, 32-bit data format word): loads through
// it take a scalar and a lane byte offset, and an offset past n reads zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_buffer(const void* p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}
// max(m, |a|, |b|) with NaN-propagating maxima (v_maximum3_f32, whose inputs need no
// canonicalizing; a NaN leaves the row's codes unspecified, as for any non-finite row).
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(a)), __builtin_fabsf(b));
}

// S_W of eq. 4 from the staged window, requantized in place: the record sum is a
// [128 x kWmax] . [kWmax x 128] contraction per head, done on the matrix cores as its
// transpose with v_mfma_f32_16x16x4f32 (A from lane l is A[l%16][l/16], B is B[l/16][l%16],
// result i of lane l is D[4(l/16)+i][l%16]). Wave w owns key rows 32w .. 32w+31 as two bands
// of 16 (B = decayed keys KE, one row per lane l%16); value-column tile ct (A = corrections
// Us) takes the columns col_base(m) + ct, m = 0..15, col_base(4g + i) = 64 (i / 2) + 16g +
// 8 (i % 2), so that lane l reads the corrections of 8 consecutive columns with two 128-bit
// LDS loads, and result i of tile ct is column col_base(4(l/16) + i) + ct: lane l ends up with
// the code words 4(l/16) .. +3 and 16 + 4(l/16) .. +3 of its row, so that each of its two
// 16-byte stores fills 64 contiguous bytes of the row with its 3 neighbours. All operands
// of a band are loaded before its MFMAs. Rows of KE / Us past the last record are zero;
// zcoef[r] = a_r / 127 Gamma_{1:W, r}; old_codes(a, zo) gives the lane's 8 old code words of
// band a (row 16 (2 wave + a) + l%16, words 4(l/16) .. +3 in zo[0..3] and 16 + 4(l/16) .. +3 in
// zo[4..7]); the new codes of those 32 columns leave straight from the lane's registers.
__device__ __forceinline__ int col_base(int m) { return 64 * ((m & 3) >> 1) + 16 * (m >> 2) + 8 * (m & 1); }
template <int kWmax, typename OldCodes>
__device__ __forceinline__ void form_and_requantize(const float* KE, const float* Us, OldCodes old_codes,
                                                    const float* zcoef, float* __restrict__ Ah,
                                                    uint32_t* __restrict__ Zh, int wave, int lane) {
    constexpr int kSteps = kWmax / 4;
    const int lr = lane & 15, lq = lane >> 4;
    auto band = [&](int a) {  // one 16-row band at a time: 8 accumulators live
        const int row = 16 * (2 * wave + a) + lr;
        float eb[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            eb[s] = KE[(4 * s + lq) * kD + row];
        // old codes: word d (d = 2i + hh) holds columns col_base(4 lq + i) + 4hh .. +3
        uint32_t zo[8];
        old_codes(a, zo);
        const float zc = zcoef[row];
        f32x4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[ct][i] = static_cast<float>(static_cast<int8_t>((zo[2 * i + ct / 4] >> (8 * (ct % 4))) & 0xffu)) * zc;
        // the corrections of four records at a time (loaded again for the second band: holding
        // them across both bands would take 16 kWmax registers)
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const float* src = Us + (4 * s + lq) * kD + col_base(lr);
            const f32x4 ua[2] = {*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 4)};
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[ct / 4][ct % 4], eb[s], acc[ct], 0, 0, 0);
            if (s % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
        // per-row absmax: 32 values in this lane, then the 4 lanes l, l^16, l^32, l^48
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ct += 2) {
            m0 = max3_abs(m0, acc[ct].x, acc[ct].y);
            m1 = max3_abs(m1, acc[ct].z, acc[ct].w);
            m0 = max3_abs(m0, acc[ct + 1].x, acc[ct + 1].y);
            m1 = max3_abs(m1, acc[ct + 1].z, acc[ct + 1].w);
        }
        float m = max_xor16(fmaxf(m0, m1));
        swap32(m, m0, m1);
        m = fmaxf(m0, m1);
        // a row maximum below 2^-64 is decided as the row scaled by f = 2^64 (no branch: the
        // factor enters the rounding fma)
        const float f = tiny_factor(m);
        const float q = __fdiv_rn(127.f, m * f);  // (unconditional: a branch would split the block)
        const float sc = m > 0.f ? q : 0.f;
        if (lq == 0) Ah[row] = m;
        // word 2i + hh of the lane's 8 holds columns col_base(4 lq + i) + 4hh .. +3
        uint32_t cw[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                cw[2 * i + hh] = code_word_in_range(f32x4{acc[4 * hh + 0][i], acc[4 * hh + 1][i], acc[4 * hh + 2][i],
                                                          acc[4 * hh + 3][i]} * sc, f);
        uint32_t* out = Zh + row * (kD / 4) + 4 * lq;
        __builtin_nontemporal_store((u32x4{cw[0], cw[1], cw[2], cw[3]}), reinterpret_cast<u32x4*>(out));
        __builtin_nontemporal_store((u32x4{cw[4], cw[5], cw[6], cw[7]}), reinterpret_cast<u32x4*>(out + 16));
    };
    band(0);
    band(1);
}

// ---- the last step of the window (pos = W - 1): the step itself, then S_W of eq. 4
// formed from the codes and all W records, and requantized in place.
template <bool kPerKey, int kWmax, typename T>
__global__ __launch_bounds__(kThreads) void q8_boundary_kernel(
    int W, int pos, int8_t* __restrict__ Z, float* __restrict__ A, const T* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ float gsuf[kMaxW + 1];     // GDN: gate products after each record; [kMaxW]: all
    __shared__ float gtot[kPerKey ? kD : 1];  // KDA: the product of all record gates per key row
    __shared__ f32x2 rowv[kD];            // a_r/127 Gamma_{1:l} (k_r, q_r)
    __shared__ f32x2 kq_row[kD];          // (k_r, q_r)
    __shared__ f32x2 coef[kMaxW];         // per record (E_j . k, E_j . q)
    __shared__ f32x2 red[4][kD];          // per-wave column partials
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    float* KE = dyn_lds;
    float* Us = KE + kWmax * kD;
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Us + kWmax * kD);

    // ---- every load of the step is issued here: records and inputs first, then the
    // codes, so that the key-side preparation below only waits for the former while
    // the codes are still in flight (loads complete in order)
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    Stager<T, kMaxW * kD> sk;
    Stager<float, kMaxW * kD> su;
    sk.load(Kbuf + rec0, pos * kD, tid);
    su.load(Ubuf + rec0, pos * kD, tid);
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    float g_rec = 1.f;
    KeyDecays<kPerKey ? kWmax / 2 : 1> kdec;   // per-key gates: row tid >> 1, half tid & 1
    float g_half_row = 1.f;                      // the current gate at that row
    if constexpr (kPerKey) {
        kdec.load(Gbuf + rec0, pos, tid);
        g_half_row = gate[vec_off + (tid >> 1)];
    } else if (tid < pos) {
        g_rec = Gbuf[static_cast<size_t>(h) * W + tid];
    }
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = kPerKey ? gate[vec_off + r] : gate[h];
    const float ar = A[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    if constexpr (!kPerKey) {
        // wave 0: lane j gets the product of the gates of records j+1 .. pos-1 (newest first)
        if (wave == 0) {
            float G = 1.f, Gall = 1.f;
            for (int i = pos - 1; i >= 0; --i) {
                const float gi = lane_value(g_rec, i);
                G = i > lane ? G * gi : G;
                Gall *= gi;
            }
            if (lane < pos) gsuf[lane] = G;
            if (lane == 0) gsuf[kMaxW] = Gall;
        }
    }
    sk.store(KE, tid);
    su.store(Us, tid);
    for (int i = W * kD + tid; i < kWmax * kD; i += kThreads) Us[i] = 0.f;  // rows after the last record
    __syncthreads();

    // ---- decayed keys E_j = Gamma_{j+1:l} k_j in place; the current key is row pos
    if constexpr (!kPerKey) {
        for (int i = tid; i < pos * kD; i += kThreads) KE[i] *= gsuf[i >> 7] * gr;
    } else {
        // both halves of each key row's records at once; gtot: the product of the row's gates
        const float G = kdec.apply(KE, pos, g_half_row, tid);
        if ((tid & 1) == 0) gtot[tid >> 1] = G;
    }
    if (first) {
        kq_row[r] = f32x2{kr, qr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
        KE[pos * kD + r] = kr;  // the current record: no decay after it
        for (int j = pos + 1; j < kWmax; ++j) KE[j * kD + r] = 0.f;
    }
    __syncthreads();
    if (first) {
        const float G = kPerKey ? gtot[r] : gsuf[kMaxW];  // product of all record gates at row r
        const float c0 = ar * (1.f / 127.f) * G * gr;   // a_r/127 Gamma_{1:l} at row r
        rowv[r] = f32x2{c0 * kr, c0 * qr};
        zcoef[r] = c0;
    }

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
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) Zs[q8_row(it, wave, ro) * kZsStride + c4] = zw[it];
    __syncthreads();

    // ---- correction and output; u of this step becomes row pos of Us
    if (first) {
        const int c = tid;
        const f32x2 acc = red[0][c] + red[1][c] + red[2][c] + red[3][c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        Us[pos * kD + c] = u;
    }
    __syncthreads();

    // ---- S_W = Gamma_{1:W} S^_0 + sum_j Gamma_{j+1:W} k_j u_j^T, requantized.
    const int lr = lane & 15, lq = lane >> 4;
    auto old_codes = [&](int a, uint32_t(&zo)[8]) {
        const uint32_t* src = Zs + (16 * (2 * wave + a) + lr) * kZsStride + 4 * lq;
#pragma unroll
        for (int d = 0; d < 8; ++d) zo[d] = src[d < 4 ? d : 12 + d];
    };
    form_and_requantize<kWmax>(KE, Us, old_codes, zcoef, A + vec_off, Zh, wave, lane);
}

// ---- RWKV7 on the per-window int8 state, two records per token (LeapQuant, App. A: an
// erase sub-step with gate w, key kappa and read vector a * kappa, then a write with gate 1
// and key k). Record 2t = (w_t, kappa_t, u_e = 0 - S_{t-1}^T (a_t * kappa_t)), record 2t+1 =
// (1, k_t, v_t). Token t reads S_{t-1} (eq. 4 over its 2t records) along a_t * kappa_t and,
// for the output, along w_t * q_t:  y = S_{t-1}^T (w_t q_t) + u_e (kappa_t . q_t) + v_t (k_t . q_t).
// Both reads are one sweep with the per-key step's layout (records in registers, 16-lane
// groups for their coefficients, row-owners for their corrections); a record's decay is the
// product of the later records' gates (the read vectors carry the token's own factors).
// Every token, the last one too, appends its two records; at the end of the window a
// second launch requantizes S_W from all 2W records.
constexpr int kRwkv7Rec = 32;  // records per window: two per token, W <= 16
// Dynamic LDS of the requantizer: decayed keys and corrections of up to kRwkv7Rec records.
__host__ __device__ constexpr int requant_lds_floats() { return 2 * kRwkv7Rec * kD; }

template <typename T>
__global__ __launch_bounds__(kThreads) void rwkv7_q8_step_kernel(
    int W, int pos, const int8_t* __restrict__ Z, const float* __restrict__ A, T* __restrict__ Kbuf,
    float* __restrict__ Ubuf, float* __restrict__ Gbuf, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ kappa, const float* __restrict__ w,
    const float* __restrict__ erase, float* __restrict__ y) {
    extern __shared__ __align__(16) float gs_lds[];   // the records' gates [2 pos][128]
    __shared__ f32x2 rowv[kD];            // a_r/127 Gamma_{1:t-1} (a_r kappa_r, w_r q_r)
    __shared__ f32x2 coef[kRwkv7Rec];     // per record (E_j . a kappa, E_j . w q)
    __shared__ f32x2 red[4][kD];          // per-wave column partials
    __shared__ f32x2 kq_part[2];          // (kappa . q, k . q) of the two waves that hold rows
    constexpr int kKSlots = kRwkv7Rec / 16, kUSlots = kRwkv7Rec / 8;

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5, owner = 2 * wave + ro;
    const int grp = tid >> 4, ch = tid & 15;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * 2 * W * kD;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const int nrec = 2 * pos;

    // ---- loads: records, gates, inputs, then the codes
    Raw8<T> kc[kKSlots];
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        const int j = grp + 16 * s;
        // unconditional, so that no branch makes the compiler wait for it (a branch around a
        // load ends in a wait for every load before it): a lane past the last record reads
        // slot 0, a slot group with no record at all reads this lane's own input keys (loaded
        // anyway, so no extra traffic); such keys are never used
        kc[s].load(16 * s < nrec ? Kbuf + rec0 + static_cast<size_t>(j < nrec ? j : 0) * kD + 8 * ch : k + vec_off + 8 * ch);
    }
    f32x4 ur[kUSlots];
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        const int j = owner + 8 * m;
        // unconditional as the keys (a slot group with no record reads the lane's scales); a
        // clamped slot's values meet a zero coefficient
        ur[m] = *reinterpret_cast<const f32x4*>(8 * m < nrec ? Ubuf + rec0 + static_cast<size_t>(j < nrec ? j : 0) * kD + 4 * c4
                                                              : A + vec_off + 4 * c4);
    }
    Stager<float, kRwkv7Rec * kD> sg;
    sg.load(Gbuf + rec0, nrec * kD, tid);
    Raw8<T> cch, qch;  // kappa and q of the lane's 8 keys
    cch.load(kappa + vec_off + 8 * ch);
    qch.load(q + vec_off + 8 * ch);
    const f32x4 w_lo = *reinterpret_cast<const f32x4*>(w + vec_off + 8 * ch);
    const f32x4 w_hi = *reinterpret_cast<const f32x4*>(w + vec_off + 8 * ch + 4);
    const f32x4 e_lo = *reinterpret_cast<const f32x4*>(erase + vec_off + 8 * ch);
    const f32x4 e_hi = *reinterpret_cast<const f32x4*>(erase + vec_off + 8 * ch + 4);
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r), cr = load_in(kappa, vec_off + r);
    const float wr = w[vec_off + r], er = erase[vec_off + r];
    const float ar = A[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const uint32_t* Zh = reinterpret_cast<const uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    // ---- decays: Gs = product of the gates of the records after record grp + 16 s, per key of
    // the lane's 8; Gall = product of all record gates at row r (suffix products per key
    // column, in place)
    sg.store(gs_lds, tid);
    __syncthreads();
    float Gall = 1.f;
    if (first) Gall = column_suffix_products<kRwkv7Rec>(gs_lds, nrec, r);
    __syncthreads();
    float Gs[kKSlots][8];
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        const int j = grp + 16 * s;
#pragma unroll
        for (int e = 0; e < 8; ++e) Gs[s][e] = 1.f;
        if (j >= nrec) continue;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(gs_lds + j * kD + 8 * ch);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(gs_lds + j * kD + 8 * ch + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Gs[s][e] = lo[e];
            Gs[s][e + 4] = hi[e];
        }
    }

    // ---- record coefficients against both read vectors, over the 16 lanes of each group
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        if (16 * s >= nrec) continue;
        const int j = grp + 16 * s;
        float c1 = 0.f, c2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = kc[s][e] * Gs[s][e];
            const float x1 = (e < 4 ? e_lo[e] : e_hi[e - 4]) * cch[e];
            const float x2 = (e < 4 ? w_lo[e] : w_hi[e - 4]) * qch[e];
            c1 += ej * x1;
            c2 += ej * x2;
        }
        c1 = row16_sum(c1);
        c2 = row16_sum(c2);
        if (ch == 0 && j < nrec) coef[j] = f32x2{c1, c2};
    }
    if (first) {
        const float c0 = ar * (1.f / 127.f) * Gall;  // a_r/127 Gamma_{1:t-1} at row r
        rowv[r] = f32x2{c0 * (er * cr), c0 * (wr * qr)};
        const float cq = wave_sum(cr * qr);
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = f32x2{cq, kq};
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
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        if (8 * m >= nrec) continue;
        const int j = owner + 8 * m;
        const f32x2 c = j < nrec ? coef[j] : f32x2{0.f, 0.f};
        p1 += ur[m] * c.x;
        p2 += ur[m] * c.y;
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

    // ---- the erase value, the output, and the token's two records (thread -> column c == r)
    if (first) {
        const int c = tid;
        const f32x2 acc = red[0][c] + red[1][c] + red[2][c] + red[3][c];
        const f32x2 kq = kq_part[0] + kq_part[1];
        const float ue = 0.f - acc.x;
        y[vec_off + c] = acc.y + ue * kq.x + vr * kq.y;
        const size_t re = rec0 + static_cast<size_t>(nrec) * kD, rw = re + kD;
        store_in(Kbuf, re + c, cr);
        Ubuf[re + c] = ue;
        Gbuf[re + c] = wr;
        store_in(Kbuf, rw + c, kr);
        Ubuf[rw + c] = vr;
        Gbuf[rw + c] = 1.f;
    }
}

// ---- DeltaProduct on the per-window int8 state (LeapQuant, sec. 3.2 with App. A: each of a
// token's kN delta-rule sub-steps is one buffered record; gate alpha for the first, 1 for the
// others; key k_i; correction u_i). Token pos reads S_{t-1} (eq. 4 over the kN pos earlier
// records) along its kN keys and along q, all in one sweep; with P_i = S_{t-1}^T k_i and
// R = S_{t-1}^T q,
//   u_i = beta_i (v_i - alpha P_i - sum_{m<i} u_m (k_m . k_i)),   y = alpha R + sum_i u_i (k_i . q),
// then appends its kN records; at the end of the window a second launch requantizes S_W from
// all kN W records. The records' gates are scalars, so their decays come from a suffix scan
// across the record lanes. Layouts as in the RWKV7 step: record keys in 16-lane groups for
// their coefficients, record corrections in the registers of the row-owners.
template <int kN, typename T>
__global__ __launch_bounds__(kThreads) void dp_q8_step_kernel(
    int W, int pos, const int8_t* __restrict__ Z, const float* __restrict__ A, T* __restrict__ Kbuf,
    float* __restrict__ Ubuf, float* __restrict__ Gbuf, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ y) {
    constexpr int kRec = kRwkv7Rec;       // record slots (kN W <= 32)
    constexpr int kX = kN + 1;            // read vectors: the kN keys, then q
    constexpr int kKSlots = kRec / 16, kUSlots = kRec / 8;
    __shared__ float rowv[kX][kD];        // a_r/127 Gamma_{1:t-1} x_r
    __shared__ float coef[kRec][kX];      // per record, (Gamma_{j+1:t-1} k_j) . x
    __shared__ float red[4][kX][kD];      // per-wave column partials
    __shared__ float dots[2][kX][kX];     // [wave][m][i]: partial k_m . x_i, m < i, of the two row waves

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5, owner = 2 * wave + ro;
    const int grp = tid >> 4, ch = tid & 15;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t key_off = static_cast<size_t>(h) * kN * kD;
    const int R = kN * W;                          // record slots per head
    const size_t rec0 = static_cast<size_t>(h) * R * kD;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const int nrec = kN * pos;

    // ---- loads: records, gates, inputs, then the codes
    Raw8<T> kc[kKSlots];
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        const int j = grp + 16 * s;
        // unconditional, so that no branch makes the compiler wait for it (a branch around a
        // load ends in a wait for every load before it): a lane past the last record reads
        // slot 0, a slot group with no record at all reads this lane's own input keys (loaded
        // anyway, so no extra traffic); such keys are never used
        kc[s].load(16 * s < nrec ? Kbuf + rec0 + static_cast<size_t>(j < nrec ? j : 0) * kD + 8 * ch : k + key_off + 8 * ch);
    }
    f32x4 ur[kUSlots];
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        const int j = owner + 8 * m;
        // unconditional as the keys (a slot group with no record reads the lane's scales); a
        // clamped slot's values meet a zero coefficient
        ur[m] = *reinterpret_cast<const f32x4*>(8 * m < nrec ? Ubuf + rec0 + static_cast<size_t>(j < nrec ? j : 0) * kD + 4 * c4
                                                              : A + vec_off + 4 * c4);
    }
    const float g_lane = lane < nrec ? Gbuf[static_cast<size_t>(h) * R + lane] : 1.f;
    Raw8<T> xch[kX];  // the lane's 8 key rows of every read vector
#pragma unroll
    for (int i = 0; i < kN; ++i) xch[i].load(k + key_off + i * kD + 8 * ch);
    xch[kN].load(q + vec_off + 8 * ch);
    float xr[kX];     // key row r of every read vector
#pragma unroll
    for (int i = 0; i < kN; ++i) xr[i] = load_in(k, key_off + i * kD + r);
    xr[kN] = load_in(q, vec_off + r);
    const float ar = A[vec_off + r];
    const float al = alpha[h];
    const uint32_t* Zh = reinterpret_cast<const uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    // ---- decays: products of the gates after each record (g = 1 from record nrec on)
    const float Sfx = suffix_prod<kRec>(g_lane, lane);
    const float E = suffix_prod_excl<kRec>(Sfx, lane);
    float Gs[kKSlots];
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) Gs[s] = lane_gather(E, grp + 16 * s);
    const float Gall = lane_value(Sfx, 0);

    // ---- record coefficients against every read vector, over the 16 lanes of each group
#pragma unroll
    for (int s = 0; s < kKSlots; ++s) {
        if (16 * s >= nrec) continue;
        const int j = grp + 16 * s;
        float c[kX];
#pragma unroll
        for (int i = 0; i < kX; ++i) c[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = kc[s][e] * Gs[s];
#pragma unroll
            for (int i = 0; i < kX; ++i) c[i] += ej * xch[i][e];
        }
#pragma unroll
        for (int i = 0; i < kX; ++i) c[i] = row16_sum(c[i]);
        if (ch == 0 && j < nrec)
#pragma unroll
            for (int i = 0; i < kX; ++i) coef[j][i] = c[i];
    }
    if (first) {
        const float c0 = ar * (1.f / 127.f) * Gall;  // a_r/127 Gamma_{1:t-1} at row r
#pragma unroll
        for (int i = 0; i < kX; ++i) rowv[i][r] = c0 * xr[i];
#pragma unroll
        for (int m = 0; m < kN; ++m)
#pragma unroll
            for (int i = m + 1; i < kX; ++i) {
                const float d = wave_sum(xr[m] * xr[i]);
                if (lane == 0) dots[wave][m][i] = d;
            }
    }
    __syncthreads();

    // ---- one sweep of the int8 tile for every read vector, plus the records
    f32x4 P[kX];
#pragma unroll
    for (int i = 0; i < kX; ++i) P[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const int row = q8_row(it, wave, ro);
        const f32x4 zf = unpack_i8x4(zw[it]);
#pragma unroll
        for (int i = 0; i < kX; ++i) P[i] += zf * rowv[i][row];
        if ((it & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // decode a few words at a time
    }
#pragma unroll
    for (int m = 0; m < kUSlots; ++m) {
        if (8 * m >= nrec) continue;
        const int j = owner + 8 * m;
        if (j < nrec)
#pragma unroll
            for (int i = 0; i < kX; ++i) P[i] += ur[m] * coef[j][i];
    }
#pragma unroll
    for (int i = 0; i < kX; ++i) {
        P[i] = f32x4{add_xor32(P[i].x), add_xor32(P[i].y), add_xor32(P[i].z), add_xor32(P[i].w)};
        if (ro == 0) *reinterpret_cast<f32x4*>(&red[wave][i][4 * c4]) = P[i];
    }
    __syncthreads();

    // ---- the sub-steps' corrections in order, the output, and the token's records
    // (thread -> value column c == key row r)
    if (first) {
        const int c = tid;
        float Pc[kX];
#pragma unroll
        for (int i = 0; i < kX; ++i) Pc[i] = red[0][i][c] + red[1][i][c] + red[2][i][c] + red[3][i][c];
        float u[kN];
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            float p = al * Pc[i];
#pragma unroll
            for (int m = 0; m < i; ++m) p += u[m] * (dots[0][m][i] + dots[1][m][i]);
            u[i] = beta[static_cast<size_t>(h) * kN + i] * (load_in(v, key_off + i * kD + c) - p);
        }
        float o = al * Pc[kN];
#pragma unroll
        for (int i = 0; i < kN; ++i) o += u[i] * (dots[0][i][kN] + dots[1][i][kN]);
        y[vec_off + c] = o;
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            const size_t rec = rec0 + static_cast<size_t>(nrec + i) * kD;
            Ubuf[rec + c] = u[i];
            store_in(Kbuf, rec + c, xr[i]);
        }
        if (c < kN) Gbuf[static_cast<size_t>(h) * R + nrec + c] = c == 0 ? al : 1.f;
    }
}


// ---- requantization of S_W = Gamma_{1:W} S^_0 + sum_j Gamma_{j+1:W} k_j u_j^T from nrec
// buffered records and no current step (the window's last records are already appended).
// kPerKey: per-key record gates Gbuf [heads, rec_stride, 128] (RWKV7), else one scalar gate per
// record, Gbuf [heads, rec_stride] (DeltaProduct sub-steps).
template <bool kPerKey, typename T>
__global__ __launch_bounds__(kThreads) void q8_requant_kernel(int nrec, int rec_stride, int8_t* __restrict__ Z,
                                                              float* __restrict__ A, const T* __restrict__ Kbuf,
                                                              const float* __restrict__ Ubuf,
                                                              const float* __restrict__ Gbuf) {
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ float zcoef[kD];
    float* KE = dyn_lds;
    float* Us = KE + kRwkv7Rec * kD;

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * rec_stride * kD;
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);

    Stager<T, kRwkv7Rec * kD> sk;
    Stager<float, kRwkv7Rec * kD> su;
    sk.load(Kbuf + rec0, nrec * kD, tid);
    su.load(Ubuf + rec0, nrec * kD, tid);
    KeyDecays<kPerKey ? kRwkv7Rec / 2 : 1> kdec;  // per-key gates of key row tid >> 1, half tid & 1
    float g_lane = 1.f;                             // scalar gates: lane j holds the gate of record j
    if constexpr (kPerKey) kdec.load(Gbuf + rec0, nrec, tid);
    else if (lane < nrec) g_lane = Gbuf[static_cast<size_t>(h) * rec_stride + lane];
    const float ar_half_row = A[vec_off + (tid >> 1)];
    const float ar = A[vec_off + r];
    (void)ar_half_row;
    (void)ar;
    // the old codes go straight into the layout of the MFMA results (no sweep needs them
    // first): band a, row 16 (2 wave + a) + lr, words 4 lq .. +3 and 16 + 4 lq .. +3
    uint32_t zr[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 w = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(Zh + (16 * (2 * wave + a) + lr) * (kD / 4) + 4 * lq + 16 * hh));
            zr[a][4 * hh + 0] = w.x;
            zr[a][4 * hh + 1] = w.y;
            zr[a][4 * hh + 2] = w.z;
            zr[a][4 * hh + 3] = w.w;
        }
    sk.store(KE, tid);
    su.store(Us, tid);
    for (int i = nrec * kD + tid; i < kRwkv7Rec * kD; i += kThreads) Us[i] = 0.f;
    __syncthreads();
    if constexpr (kPerKey) {  // both halves of each key row's records at once
        const float G = kdec.apply(KE, nrec, 1.f, tid);
        if ((tid & 1) == 0) zcoef[tid >> 1] = ar_half_row * (1.f / 127.f) * G;
    } else {                  // the scalar decays from a suffix scan over the record lanes
        const float Sfx = suffix_prod<kRwkv7Rec>(g_lane, lane);
        const float E = suffix_prod_excl<kRwkv7Rec>(Sfx, lane);
        for (int i = tid; i < nrec * kD; i += kThreads) KE[i] *= lane_gather(E, i >> 7);
        if (first) zcoef[r] = ar * (1.f / 127.f) * lane_value(Sfx, 0);
    }
    if (first)
        for (int j = nrec; j < kRwkv7Rec; ++j) KE[j * kD + r] = 0.f;
    __syncthreads();
    auto old_codes = [&](int a, uint32_t(&zo)[8]) {
#pragma unroll
        for (int d = 0; d < 8; ++d) zo[d] = zr[a][d];
    };
    form_and_requantize<kRwkv7Rec>(KE, Us, old_codes, zcoef, A + vec_off, Zh, wave, lane);
}

// Three bf16 parts of an fp32 value: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid).
// Both differences are exact in fp32, so hi + mid + lo equals x to about 2^-27 |x|.
__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const __bf16 h = static_cast<__bf16>(x);
    const float r1 = x - static_cast<float>(h);
    const __bf16 m = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(m);
    const __bf16 l = static_cast<__bf16>(r2);
    hi = __builtin_bit_cast(uint16_t, h);
    mid = __builtin_bit_cast(uint16_t, m);
    lo = __builtin_bit_cast(uint16_t, l);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16(x0) | bf16(x1) << 16, both rounded to nearest even (one conversion instruction).
__device__ __forceinline__ uint32_t pk_bf16(float x0, float x1) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x0, x1}), bf16x2));
}
// split3_bf16 of two values at once, each part as a packed pair (x0 in the low half).
__device__ __forceinline__ void split3_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = pk_bf16(x0, x1);
    const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xffff0000u);
    mid = pk_bf16(r0, r1);
    const float s0 = r0 - __uint_as_float(mid << 16), s1 = r1 - __uint_as_float(mid & 0xffff0000u);
    lo = pk_bf16(s0, s1);
}

// Word w of code row r in the LDS copy of a head's codes (32 words a row, no padding): the
// 16-byte chunk index is XORed with (r / 2) % 8, so that 16 consecutive rows read at the
// same chunk hit 16 different bank groups, and a row's 32 words stay in one bank sweep.
__device__ __forceinline__ int zs_word(int r, int w) { return r * (kD / 4) + (w ^ (4 * ((r >> 1) & 7))); }
// Slot of value column c in the staged corrections: tile ct, A row m = 4g + i takes the code
// word 4g + ct (ct < 4) or 16 + 4g + ct - 4 (ct >= 4), column 4 word + i, stored at 16ct + m.
__device__ __forceinline__ int ut_slot(int c) {
    const int w = c >> 2;
    return 16 * ((w & 3) + 4 * (w >> 4)) + 4 * ((w >> 2) & 3) + (c & 3);
}

// ---- the last step of the window for scalar gates (GDN), bf16 keys and W <= 16.
// The decay of record j is a scalar, so it moves onto the correction:
// S_W = Gamma_{1:W} S^_0 + sum_j k_j (Gamma_{j+1:W} u_j)^T. The keys are exact in
// bf16; each scaled correction is split into three bf16 parts, and the contraction
// runs as two v_mfma_f32_16x16x32_bf16 per 16x16 tile (hi and mid parts against the
// keys, then the lo part): the products are exact and accumulate in fp32, so the
// result matches an fp32 contraction up to rounding order, at a quarter of the
// matrix-core time of v_mfma_f32_16x16x4f32. Operand layout (checked on gfx950):
// lane l supplies A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16], e = 0..7. (A
// v_mfma_f32_16x16x16_bf16 for the lo parts alone would skip the zero half of the
// second product, but chained onto the same accumulator after the x32 product it
// gave wrong sums with this toolchain.)
// Records are staged transposed, as 16-byte words of 8 consecutive records:
// Kt[b][row] (keys of records 8b .. 8b+7 at a key row) and Ut[part][b][ut_slot(column)].
__global__ __launch_bounds__(kThreads) void q8_boundary_bf16_kernel(
    int W, int pos, int8_t* __restrict__ Z, float* __restrict__ A, const bf16_t* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    constexpr int kRec = 16;              // record slots
    __shared__ f32x2 rowv[kD];            // a_r/127 Gamma_{1:l} (k_r, q_r)
    __shared__ f32x2 coef[kRec];          // per record (E_j . k, E_j . q)
    __shared__ f32x2 red[4][kD];          // per-wave column partials of the code sweep
    __shared__ f32x2 recp[kD];            // record terms of records 8 .. 15 per column
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];
    __shared__ float gam[kRec];           // Gamma_{j+1:W}; 1 for the current record
    __shared__ u32x4 Kt[2][kD];
    __shared__ u32x4 Ut[3][2][kD];
    __shared__ __align__(16) uint32_t Zs[kD * kD / 4];  // codes, row-major, 16-byte chunks swizzled (zs_word)

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const int grp = tid >> 4, ch = tid & 15;         // coefficient layout: record grp, keys 8ch .. +7
    const int cc = tid & (kD - 1), half = tid >> 7;  // column layout: column / key row cc, records 8 half .. +7
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const bool first = tid < kD;

    // ---- every load is issued first: records (two layouts), gates, inputs, then codes
    Raw8<bf16_t> kc;
    if (0 < pos) kc.load(Kbuf + rec0 + static_cast<size_t>(grp < pos ? grp : 0) * kD + 8 * ch);
    float ucol[8];
    uint32_t kcol[4];  // keys of records 8 half + e at key row cc, two bf16 per word
    // the record slot of each load is the same in the whole wave: one buffer resource per
    // record array of the head, the slot in the scalar offset, the column in the lane offset
    const int half_w = __builtin_amdgcn_readfirstlane(half);
    const auto urs = head_buffer(Ubuf + rec0, W * kD * sizeof(float));
    const auto krs = head_buffer(Kbuf + rec0, W * kD * sizeof(bf16_t));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half_w + e;
        const int slot = j < pos ? j : 0;  // clamped to slot 0 (in bounds), the value dropped for j >= pos
        const float ul = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(urs, cc * sizeof(float), slot * kD * sizeof(float), 0));
        const uint32_t kl =
            __builtin_amdgcn_raw_buffer_load_b16(krs, cc * sizeof(bf16_t), slot * kD * sizeof(bf16_t), 0);
        ucol[e] = j < pos ? ul : 0.f;
        const uint32_t kb = j < pos ? kl : 0u;
        kcol[e >> 1] = (e & 1) ? (kcol[e >> 1] | (kb << 16)) : kb;
    }
    const float g_lane = lane < pos ? Gbuf[static_cast<size_t>(h) * W + lane] : 1.f;
    Raw8<bf16_t> kch, qch;
    kch.load(k + vec_off + 8 * ch);
    qch.load(q + vec_off + 8 * ch);
    const float kr = load_in(k, vec_off + cc), qr = load_in(q, vec_off + cc);
    const float gr = gate[h];
    const float ar = A[vec_off + cc];
    const float vr = load_in(v, vec_off + cc);
    const float bt = beta[h];
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    // ---- gate products by a suffix scan over the record lanes (g = 1 past the last
    // record): Gl = the product of the gates after record `lane`, Gg the same for record
    // grp, Gall the product of all record gates
    const float Sfx = suffix_prod<kRec>(g_lane, lane);
    const float Gl = suffix_prod_excl<kRec>(Sfx, lane);
    const float Gg = lane_gather(Gl, grp);
    const float Gall = lane_value(Sfx, 0);
    if (wave == 0 && lane < kRec) gam[lane] = lane < pos ? Gl * gr : 1.f;
    if (0 < pos) {
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = kc[e] * (Gg * gr);  // Gamma_{j+1:l} k_j
            ck += ej * kch[e];
            cq += ej * qch[e];
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < pos) coef[grp] = f32x2{ck, cq};
    }
    if (first) {
        const float c0 = ar * (1.f / 127.f) * Gall * gr;  // a_r/127 Gamma_{1:l} at row r
        rowv[cc] = f32x2{c0 * kr, c0 * qr};
        zcoef[cc] = c0;
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    Kt[half][cc] = u32x4{kcol[0], kcol[1], kcol[2], kcol[3]};
    __syncthreads();

    // ---- code sweep for both read vectors; record terms per column; scaled records staged
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x2 rv = rowv[q8_row(it, wave, ro)];
        const f32x4 zf = unpack_i8x4(zw[it]);
        p1 += zf * rv.x;
        p2 += zf * rv.y;
        // decode a few words at a time: decoding all 64 codes ahead of their products
        // would hold them in 64 registers
        if ((it & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    f32x2 rp = {0.f, 0.f};
    u32x4 part[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const f32x2 c = j < pos ? coef[j] : f32x2{0.f, 0.f};
        rp += c * ucol[e];
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const int j = 8 * half + e;
        uint32_t hi, mid, lo;
        split3_bf16x2(gam[j] * ucol[e], gam[j + 1] * ucol[e + 1], hi, mid, lo);
        part[0][e >> 1] = hi;
        part[1][e >> 1] = mid;
        part[2][e >> 1] = lo;
    }
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) Ut[pp][half][ut_slot(cc)] = part[pp];
    p1 = f32x4{add_xor32(p1.x), add_xor32(p1.y), add_xor32(p1.z), add_xor32(p1.w)};
    p2 = f32x4{add_xor32(p2.x), add_xor32(p2.y), add_xor32(p2.z), add_xor32(p2.w)};
    if (ro == 0) {
        red[wave][4 * c4 + 0] = f32x2{p1.x, p2.x};
        red[wave][4 * c4 + 1] = f32x2{p1.y, p2.y};
        red[wave][4 * c4 + 2] = f32x2{p1.z, p2.z};
        red[wave][4 * c4 + 3] = f32x2{p1.w, p2.w};
    }
    if (half == 1) recp[cc] = rp;
    {  // zs_word of row 8 it + 2 wave + ro: the chunk swizzle is wave + 4 (it % 2)
        const int w_even = (2 * wave + ro) * (kD / 4) + (c4 ^ (4 * wave));
        const int w_odd = (2 * wave + ro) * (kD / 4) + (c4 ^ (4 * wave + 16));
#pragma unroll
        for (int it = 0; it < kRowsPerThread; ++it) Zs[((it & 1) ? w_odd : w_even) + 8 * (kD / 4) * it] = zw[it];
    }
    __syncthreads();

    // ---- correction and output; the current record (no decay after it) joins the operands
    if (first) {
        const int c = cc;
        const f32x2 acc = red[0][c] + red[1][c] + red[2][c] + red[3][c] + rp + recp[c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        uint32_t uh, um, ul;
        split3_bf16(u, uh, um, ul);
        const int cs = ut_slot(c);
        reinterpret_cast<uint16_t*>(&Ut[0][pos >> 3][cs])[pos & 7] = static_cast<uint16_t>(uh);
        reinterpret_cast<uint16_t*>(&Ut[1][pos >> 3][cs])[pos & 7] = static_cast<uint16_t>(um);
        reinterpret_cast<uint16_t*>(&Ut[2][pos >> 3][cs])[pos & 7] = static_cast<uint16_t>(ul);
        reinterpret_cast<uint16_t*>(&Kt[pos >> 3][c])[pos & 7] = static_cast<uint16_t>(__float_as_uint(kr) >> 16);
    }
    __syncthreads();

    // ---- S_W on the matrix cores. Wave w owns key rows 32w .. 32w+31 as two bands of
    // 16 (B = keys, key row 16 band + l%16). Tile ct takes, for A row m = 4g + i (A = scaled
    // corrections, row m from lane m of each lane group), the value column 4 word + i with
    // word 4g + ct (ct < 4) or 16 + 4g + ct - 4 (ct >= 4); ut_slot stores it at 16ct + m.
    // Result i of lane l is then in code word 4(l/16) + ct or 16 + 4(l/16) + ct - 4: lane l
    // holds words 4(l/16) .. +3 and 16 + 4(l/16) .. +3 of its row, and each of its two 16-byte
    // stores fills 64 contiguous bytes of the row with its 3 neighbours.
    const int lr = lane & 15, lq = lane >> 4, blk = lq & 1;
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, Kt[blk][row]);
        // the lo parts fill only half of the second product's depth: the lanes of the other
        // half (lq >= 2) supply zero keys, so whatever they read as corrections drops out
        const bf16x8 bv_lo = lq < 2 ? bv : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        const float zc = zcoef[row];
        const u32x4 zlo = *reinterpret_cast<const u32x4*>(&Zs[zs_word(row, 4 * lq)]);
        const u32x4 zhi = *reinterpret_cast<const u32x4*>(&Zs[zs_word(row, 16 + 4 * lq)]);
        f32x4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            acc[ct] = unpack_i8x4(zlo[ct]) * zc;
            acc[ct + 4] = unpack_i8x4(zhi[ct]) * zc;
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, Ut[lq < 2 ? 0 : 1][blk][16 * ct + lr]);
            const bf16x8 a2 = __builtin_bit_cast(bf16x8, Ut[2][blk][16 * ct + lr]);
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv, acc[ct], 0, 0, 0);
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, bv_lo, acc[ct], 0, 0, 0);
        }
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ct += 2) {
            m0 = max3_abs(m0, acc[ct].x, acc[ct].y);
            m1 = max3_abs(m1, acc[ct].z, acc[ct].w);
            m0 = max3_abs(m0, acc[ct + 1].x, acc[ct + 1].y);
            m1 = max3_abs(m1, acc[ct + 1].z, acc[ct + 1].w);
        }
        float m = max_xor16(fmaxf(m0, m1));
        swap32(m, m0, m1);
        m = fmaxf(m0, m1);
        // a row maximum below 2^-64 is decided as the row scaled by f = 2^64 (no branch: the
        // factor enters the rounding fma)
        const float f = tiny_factor(m);
        const float q = __fdiv_rn(127.f, m * f);  // (unconditional: a branch would split the block)
        const float sc = m > 0.f ? q : 0.f;
        if (lq == 0) A[vec_off + row] = m;
        uint32_t cw[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            cw[ct] = code_word_in_range(acc[ct] * sc, f);
        uint32_t* out = Zh + row * (kD / 4) + 4 * lq;
        __builtin_nontemporal_store((u32x4{cw[0], cw[1], cw[2], cw[3]}), reinterpret_cast<u32x4*>(out));
        __builtin_nontemporal_store((u32x4{cw[4], cw[5], cw[6], cw[7]}), reinterpret_cast<u32x4*>(out + 16));
    }
}

// ---- requantization from up to 32 records with scalar gates and bf16 keys (the DeltaProduct
// window's end): as the GDN bf16 boundary, the decay after record j moves onto its correction,
// S_W = Gamma_{1:W} S^_0 + sum_j k_j (Gamma_{j+1:W} u_j)^T, the keys are exact bf16 operands and
// each scaled correction is split into three bf16 parts, so the record contraction is three
// v_mfma_f32_16x16x32_bf16 per 16 x 16 tile (hi, mid, lo parts, the 32 records along the depth)
// with exact products and fp32 sums, instead of eight fp32 MFMAs. Thread cc + 128 half stages
// column / key row cc of records 16 half .. 16 half + 15.
__global__ __launch_bounds__(kThreads) void q8_requant_bf16_kernel(int nrec, int rec_stride, int8_t* __restrict__ Z,
                                                                   float* __restrict__ A,
                                                                   const bf16_t* __restrict__ Kbuf,
                                                                   const float* __restrict__ Ubuf,
                                                                   const float* __restrict__ Gbuf) {
    constexpr int kRec = 32;
    __shared__ u32x4 Kt[kRec / 8][kD];        // keys of records 8b .. 8b+7 at each key row
    __shared__ u32x4 Ut[3][kRec / 8][kD];     // scaled corrections, three bf16 parts, per column
    __shared__ uint32_t Zs[kD * kZsStride];
    __shared__ float zcoef[kD];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const int cc = tid & (kD - 1), half = tid >> 7;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * rec_stride * kD;
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);

    // ---- loads: the records of this thread's column / key row, the gates, then the codes
    float ucol[16];
    uint32_t kcol[8];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int j = 16 * half + e;
        const size_t at = rec0 + static_cast<size_t>(j < nrec ? j : 0) * kD + cc;  // slot clamped: in bounds
        const float ul = Ubuf[at];
        const uint32_t kl = static_cast<uint32_t>(Kbuf[at]);
        ucol[e] = j < nrec ? ul : 0.f;
        const uint32_t kb = j < nrec ? kl : 0u;
        kcol[e >> 1] = (e & 1) ? (kcol[e >> 1] | (kb << 16)) : kb;
    }
    const float g_lane = lane < nrec ? Gbuf[static_cast<size_t>(h) * rec_stride + lane] : 1.f;
    const float ar = A[vec_off + cc];
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + q8_row(it, wave, ro) * (kD / 4) + c4);

    // ---- the decay after each record (suffix scan over the record lanes; g = 1 past nrec),
    // the scaled corrections split into bf16 parts, the keys, and the codes staged
    const float Sfx = suffix_prod<kRec>(g_lane, lane);
    const float E = suffix_prod_excl<kRec>(Sfx, lane);
    const float gall = lane_value(Sfx, 0);
    float gam[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) gam[e] = lane_gather(E, 16 * half + e);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        u32x4 part[3];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            uint32_t hi, mid, lo;
            split3_bf16x2(gam[8 * b + e] * ucol[8 * b + e], gam[8 * b + e + 1] * ucol[8 * b + e + 1], hi, mid, lo);
            part[0][e >> 1] = hi;
            part[1][e >> 1] = mid;
            part[2][e >> 1] = lo;
        }
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) Ut[pp][2 * half + b][cc] = part[pp];
        Kt[2 * half + b][cc] = u32x4{kcol[4 * b], kcol[4 * b + 1], kcol[4 * b + 2], kcol[4 * b + 3]};
    }
    if (half == 0) zcoef[cc] = ar * (1.f / 127.f) * gall;
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) Zs[q8_row(it, wave, ro) * kZsStride + c4] = zw[it];
    __syncthreads();

    // ---- S_W on the matrix cores (wave w: key rows 32w .. 32w+31 as two bands; B = the keys of
    // the records 8(l/16) .. +7 at key row 16 band + l%16, A = their scaled corrections at column
    // 16ct + l%16; result i of lane l is column 16ct + 4(l/16) + i), then the row absmax and codes
    const int lr = lane & 15, lq = lane >> 4;
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, Kt[lq][row]);
        const float zc = zcoef[row];
        f32x4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct] = unpack_i8x4(Zs[row * kZsStride + 4 * ct + lq]) * zc;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int col = 16 * ct + lr;
#pragma unroll
            for (int pp = 0; pp < 3; ++pp)
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Ut[pp][lq][col]), bv,
                                                                  acc[ct], 0, 0, 0);
        }
        float m = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(acc[ct].x), fabsf(acc[ct].y)),
                               fmaxf(fabsf(acc[ct].z), fabsf(acc[ct].w))));
        m = max_xor16(m);
        float m0, m1;
        swap32(m, m0, m1);
        m = fmaxf(m0, m1);
        // a row maximum below 2^-64 is decided as the row scaled by f = 2^64 (no branch: the
        // factor enters the rounding fma)
        const float f = tiny_factor(m);
        const float q = __fdiv_rn(127.f, m * f);  // (unconditional: a branch would split the block)
        const float sc = m > 0.f ? q : 0.f;
        if (lq == 0) A[vec_off + row] = m;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            Zs[row * kZsStride + 4 * ct + lq] = code_word_in_range(acc[ct] * sc, f);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * wave + 8 * i + (lane >> 3), d0 = 4 * (lane & 7);
        const uint32_t* src = Zs + row * kZsStride + d0;
        const u32x4 w4 = {src[0], src[1], src[2], src[3]};
        __builtin_nontemporal_store(w4, reinterpret_cast<u32x4*>(Zh + row * (kD / 4) + d0));
    }
}

hipError_t launch_q8_quantize(int heads, const float* S, int8_t* Z, float* A, hipStream_t stream) {
    hipLaunchKernelGGL(q8_quantize_kernel, dim3(heads), dim3(kThreads), 0, stream, S, Z, A);
    return hipGetLastError();
}

template <bool kPerKey, int kWmax, typename T>
static hipError_t launch_step_kernel(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    const size_t lds = kPerKey ? sizeof(float) * w.pos * kD : 0;
    hipLaunchKernelGGL((q8_step_kernel<kPerKey, kWmax, T>), dim3(a.heads), dim3(kThreads), lds, stream,
                       w.W, w.pos, w.Z, w.A, static_cast<T*>(w.Kbuf), w.Ubuf, w.Gbuf,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <bool kPerKey, int kWmax, typename T>
static hipError_t launch_boundary_kernel(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    const size_t lds = sizeof(float) * boundary_lds_floats(kWmax);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(q8_boundary_kernel<kPerKey, kWmax, T>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(float) * boundary_lds_floats(kWmax)));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((q8_boundary_kernel<kPerKey, kWmax, T>), dim3(a.heads), dim3(kThreads), lds, stream,
                       w.W, w.pos, w.Z, w.A, static_cast<const T*>(w.Kbuf), w.Ubuf, w.Gbuf,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <bool kPerKey, typename T>
static hipError_t launch_window_t(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    if constexpr (!kPerKey && sizeof(T) == 2) {
        if (w.pos == w.W - 1 && w.W <= 16) {
            hipLaunchKernelGGL(q8_boundary_bf16_kernel, dim3(a.heads), dim3(kThreads), 0, stream, w.W, w.pos,
                               w.Z, w.A, static_cast<const bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf,
                               static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                               static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
            return hipGetLastError();
        }
    }
    if (w.pos == w.W - 1)
        return w.W <= 16 ? launch_boundary_kernel<kPerKey, 16, T>(a, w, stream)
                         : launch_boundary_kernel<kPerKey, kMaxW, T>(a, w, stream);
    return w.W <= 16 ? launch_step_kernel<kPerKey, 16, T>(a, w, stream)
                     : launch_step_kernel<kPerKey, kMaxW, T>(a, w, stream);
}

template <typename T>
static hipError_t launch_rwkv7_window_t(const StepArgs& a, const WindowArgs& w, const void* kappa,
                                        const float* erase, hipStream_t stream) {
    hipLaunchKernelGGL(rwkv7_q8_step_kernel<T>, dim3(a.heads), dim3(kThreads), sizeof(float) * 2 * w.pos * kD,
                       stream, w.W, w.pos, w.Z, w.A, static_cast<T*>(w.Kbuf), w.Ubuf, w.Gbuf,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<const T*>(kappa), a.gate, erase, a.y);
    if (hipError_t e = hipGetLastError()) return e;
    if (w.pos < w.W - 1) return hipSuccess;
    const int floats = requant_lds_floats();
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(q8_requant_kernel<true, T>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(sizeof(float) * floats));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((q8_requant_kernel<true, T>), dim3(a.heads), dim3(kThreads), sizeof(float) * floats, stream,
                       2 * w.W, 2 * w.W, w.Z, w.A, static_cast<const T*>(w.Kbuf), w.Ubuf, w.Gbuf);
    return hipGetLastError();
}

template <int kN, typename T>
static hipError_t launch_dp_window_t(const StepArgs& a, const WindowArgs& w, hipStream_t stream) {
    hipLaunchKernelGGL((dp_q8_step_kernel<kN, T>), dim3(a.heads), dim3(kThreads), 0, stream, w.W, w.pos, w.Z, w.A,
                       static_cast<T*>(w.Kbuf), w.Ubuf, w.Gbuf, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.gate, a.beta, a.y);
    if (hipError_t e = hipGetLastError()) return e;
    if (w.pos < w.W - 1) return hipSuccess;
    if constexpr (sizeof(T) == 2) {  // bf16 keys: the bf16-split requantizer
        hipLaunchKernelGGL(q8_requant_bf16_kernel, dim3(a.heads), dim3(kThreads), 0, stream, kN * w.W, kN * w.W,
                           w.Z, w.A, static_cast<const bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf);
        return hipGetLastError();
    }
    const int floats = requant_lds_floats();
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(q8_requant_kernel<false, T>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(sizeof(float) * floats));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((q8_requant_kernel<false, T>), dim3(a.heads), dim3(kThreads), sizeof(float) * floats, stream,
                       kN * w.W, kN * w.W, w.Z, w.A, static_cast<const T*>(w.Kbuf), w.Ubuf, w.Gbuf);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dp_window_n(const StepArgs& a, const WindowArgs& w, int n, hipStream_t stream) {
    switch (n) {
        case 1: return launch_dp_window_t<1, T>(a, w, stream);
        case 2: return launch_dp_window_t<2, T>(a, w, stream);
        case 3: return launch_dp_window_t<3, T>(a, w, stream);
        default: return launch_dp_window_t<4, T>(a, w, stream);
    }
}

hipError_t launch_dp_q8_window(const StepArgs& a, const WindowArgs& w, int n, bool bf16, hipStream_t stream) {
    return bf16 ? launch_dp_window_n<bf16_t>(a, w, n, stream) : launch_dp_window_n<float>(a, w, n, stream);
}

hipError_t launch_rwkv7_q8_window(const StepArgs& a, const WindowArgs& w, const void* kappa, const float* erase,
                                  bool bf16, hipStream_t stream) {
    return bf16 ? launch_rwkv7_window_t<bf16_t>(a, w, kappa, erase, stream)
                : launch_rwkv7_window_t<float>(a, w, kappa, erase, stream);
}

hipError_t launch_q8_window(const StepArgs& a, const WindowArgs& w, bool per_key, bool bf16,
                            hipStream_t stream) {
    if (per_key) return bf16 ? launch_window_t<true, bf16_t>(a, w, stream) : launch_window_t<true, float>(a, w, stream);
    return bf16 ? launch_window_t<false, bf16_t>(a, w, stream) : launch_window_t<false, float>(a, w, stream);
}

}  // namespace rsu
