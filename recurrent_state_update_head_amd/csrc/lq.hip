// lq.hip -- LeapQuant's window-boundary format for scalar gates (GDN) and bf16 keys.
//
// A window starts from (LeapQuant sec. 3.3 eqs. 5-6, sec. 3.4 eq. 7)
//   S_0 = C dequant(Z, B) + Kt Ut^T,  C = Diag(c),  dequant(Z, B)_ij = Z_ij B_j / 127,
// with r = 4 compensator tokens (Kt, Ut) in fp16, a per-key-row smoothing scale c and a
// per-value-channel int8 payload Z with fp32 absmax B. Inside the window the readout is
// eq. 10 (App. B.3):
//   S_l^T x = B Z^T/127 (C Gamma_{1:l} x) + Ut (Kt^T Gamma_{1:l} x) + sum_j u_j (k_j^T Gamma_{j+1:l} x),
// i.e. the int8 sweep with c and the decay folded into the read vector and B applied per
// value column to the swept partials, the token pairs as four more records decayed by
// every gate of the window, and the real records as in the per-row int8 path.
// At the window's last step the state S_W (eq. 7) is formed, the tokens are refitted to
// it by subspace iteration (V <- MGS(S^T S V) from the previous window's Ut, Kt = S V,
// Ut = V, both rounded to fp16), and the residual S_W - Kt Ut^T is smoothed
// (c_i = max(sqrt(mean_j |R_ij|), 1e-6)) and quantized per value channel.
#include "kernels.hpp"
#include "rsu_device.hpp"
#include "codes.hpp"
#include "decays.hpp"
#include "swaps.hpp"

namespace rsu {

constexpr int kTok = 4;                 // compensator tokens per head
constexpr float kSmoothFloor = 1e-6f;   // floor of the smoothing scale
typedef _Float16 half_t;

// Int8 tiles use the per-row int8 path's thread layout: lane l of wave w owns one 32-bit
// word of codes (4 columns) in each of the 16 rows 8 it + 2 w + (l >> 5).
__device__ __forceinline__ int lq_row(int it, int wave, int ro) { return 8 * it + 2 * wave + ro; }

__device__ __forceinline__ f32x4 unpack_codes(uint32_t w) {
    return f32x4{static_cast<float>(static_cast<int8_t>(w & 0xffu)),
                 static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu)),
                 static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu)),
                 static_cast<float>(static_cast<int8_t>(w >> 24))};
}


// ---------------------------------------------------------------- the refit
// Sizes of the fitted format: kT tokens (4 at 8 and 6 bits, 8 at 4 bits), codes of kBits bits,
// and the LDS staging of the code rows (whole rows leave the workgroup together).
template <int kT, int kBits>
struct RefitCfg {
    static_assert((kT == 4 || kT == 8) && (kBits == 8 || kBits == 6 || kBits == 4), "4 or 8 tokens, 8-, 6- or 4-bit codes");
    static constexpr int kC = kT / 4;                        // f32x4 chunks of a token vector
    static constexpr int kQmax = (1 << (kBits - 1)) - 1;     // largest code: 127, 31 or 7
    static constexpr int kRowWords = kD * kBits / 32;        // 32 (8-bit), 24 (6-bit) or 16 (4-bit) words per row
    // staged row stride: 16-byte rows, 8 rows span the banks
    static constexpr int kCodeStride = kBits == 8 ? 40 : kBits == 6 ? 28 : 20;
};

// y + a x and a x element by element, written without a splat of a: the refit's state
// is invariant across the fit's iterations, and splats of it would be hoisted out of the
// loop as four registers each.
__device__ __forceinline__ f32x4 axpy(float a, f32x4 x, f32x4 y) {
    return f32x4{fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w)};
}
__device__ __forceinline__ f32x4 scale(float a, f32x4 x) { return f32x4{a * x.x, a * x.y, a * x.z, a * x.w}; }

// Code of w = x * (qmax / B): round half to even with one fp32 add (the low mantissa bits
// of w + 1.5 * 2^23 are the integer), clamped to [-qmax, qmax]; the returned bits are
// 0x4B400000 + z, so the code's two's complement is in the low bits: the low byte (8-bit),
// the low nibble (4-bit), or the high part z >> 2 in bits 2..5 and the low part z & 3 in
// bits 0..1 (6-bit). The add is not contracted with the product that forms w: the code is
// decided on w rounded to fp32.
template <int kBits>
__device__ __forceinline__ uint32_t lq_code_t(float w) {
#pragma clang fp contract(off)
    constexpr float kMagic = 12582912.0f;
    constexpr int kQ = (1 << (kBits - 1)) - 1;
    const int bits = __float_as_int(w + kMagic);
    return static_cast<uint32_t>(min(max(bits, 0x4B400000 - kQ), 0x4B400000 + kQ));
}

// ---------------------------------------------------------------- in-window step
// Threads and loads as in the per-row int8 step (records in registers, 16-lane groups
// for the record coefficients, row-owners for the record corrections); the tokens are
// four more records: groups 0..3 reduce (Kt_t . k, Kt_t . q) and owners 0..3 add
// Ut_t c_t. The swept payload partials are scaled by B_j / 127 per column first.
// With per-key gates (KDA) Gamma is diagonal over the key rows: the records' gates are
// staged in LDS, each lane forms the decay products of its 8 keys (after its record
// for the record terms, over the whole window for the token terms), and the payload's
// read vector takes the decay of its own row.
template <bool kPerKey>
__global__ __launch_bounds__(kThreads) void lq_step_kernel(
    int W, int pos, const int8_t* __restrict__ Z, const float* __restrict__ Bcol,
    const float* __restrict__ Csm, const half_t* __restrict__ Kc, const half_t* __restrict__ Uc,
    bf16_t* __restrict__ Kbuf, float* __restrict__ Ubuf, float* __restrict__ Gbuf,
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ gate, const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ __align__(16) float gs_lds[];   // KDA: the records' gates [pos][128]
    __shared__ f32x2 rowv[kD];
    __shared__ f32x2 coef[16];
    __shared__ f32x2 ctok[kTok];
    __shared__ __align__(16) float gtot[kPerKey ? kD : 4];  // KDA: the product of all record gates per key
    __shared__ f32x2 red[4][kD];
    __shared__ float kq_part[2];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5, owner = 2 * wave + ro;
    const int grp = tid >> 4, ch = tid & 15;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kTok * kD;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;

    // ---- loads: records, tokens, gates, inputs, then the codes
    // (unconditional, so that no branch makes the compiler wait for them: slots and tokens
    // are clamped in bounds; what a clamped lane loads is never used or meets a zero coefficient)
    uint32_t kc[4];
    {  // (at pos 0 the lane's own input keys, loaded anyway)
        const uint4 x = *reinterpret_cast<const uint4*>(
            0 < pos ? Kbuf + rec0 + static_cast<size_t>(grp < pos ? grp : 0) * kD + 8 * ch : k + vec_off + 8 * ch);
        kc[0] = x.x; kc[1] = x.y; kc[2] = x.z; kc[3] = x.w;
    }
    f32x4 ur[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int j = owner + 8 * m;
        ur[m] = *reinterpret_cast<const f32x4*>(8 * m < pos ? Ubuf + rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + 4 * c4
                                                           : Bcol + vec_off + 4 * c4);  // (the lane's scales: loaded anyway)
    }
    // token keys (groups 0..3, 8 keys per lane) and token values (owners 0..3, 4 columns)
    const uint4 ktw = *reinterpret_cast<const uint4*>(Kc + tok0 + (grp < kTok ? grp : 0) * kD + 8 * ch);
    const uint2 utw = *reinterpret_cast<const uint2*>(Uc + tok0 + (owner < kTok ? owner : 0) * kD + 4 * c4);
    float g_lane = 1.f;  // GDN: lane i holds the gate of record i
    Stager<float, kPerKey ? 16 * kD : 8> sg;
    if constexpr (kPerKey) sg.load(Gbuf + rec0, pos * kD, tid);
    else if (lane < pos) g_lane = Gbuf[static_cast<size_t>(h) * W + lane];
    const uint4 kchw = *reinterpret_cast<const uint4*>(k + vec_off + 8 * ch);
    const uint4 qchw = *reinterpret_cast<const uint4*>(q + vec_off + 8 * ch);
    f32x4 gch_lo = {1.f, 1.f, 1.f, 1.f}, gch_hi = {1.f, 1.f, 1.f, 1.f};  // KDA: current gates of the 8 keys
    if constexpr (kPerKey) {
        gch_lo = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch);
        gch_hi = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch + 4);
    }
    const f32x4 bsc = *reinterpret_cast<const f32x4*>(Bcol + vec_off + 4 * c4) * (1.f / 127.f);
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = kPerKey ? gate[vec_off + r] : gate[h];
    const float cr = Csm[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    const uint32_t* Zh = reinterpret_cast<const uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + lq_row(it, wave, ro) * (kD / 4) + c4);

    // ---- decays (newest gate first): after record grp, and over the whole window so far.
    // Per key (KDA): Ge[e] after record grp and Gt[e] over the window for the lane's 8
    // keys, Gall for row r; the current gate comes on top of each.
    float Gg = 1.f, Gall = 1.f;
    float Ge[kPerKey ? 8 : 1], Gt[kPerKey ? 8 : 1];
    if constexpr (!kPerKey) {
        // suffix scan over the record lanes (g = 1 from record pos on): the product of the
        // gates after each record, gathered for this lane's record group
        const float Sfx = suffix_prod<16>(g_lane, lane);
        Gg = lane_gather(suffix_prod_excl<16>(Sfx, lane), grp);
        Gall = lane_value(Sfx, 0);
    } else {
        // the gates' suffix products per key column, in place; the column totals in gtot
        sg.store(gs_lds, tid);
        __syncthreads();
        if (first) {
            Gall = column_suffix_products<16>(gs_lds, pos, r);
            gtot[r] = Gall;
        }
        __syncthreads();
        const bool rec = grp < pos;
        const f32x4 lo = rec ? *reinterpret_cast<const f32x4*>(gs_lds + grp * kD + 8 * ch) : f32x4{1.f, 1.f, 1.f, 1.f};
        const f32x4 hi = rec ? *reinterpret_cast<const f32x4*>(gs_lds + grp * kD + 8 * ch + 4) : f32x4{1.f, 1.f, 1.f, 1.f};
        const f32x4 tlo = *reinterpret_cast<const f32x4*>(gtot + 8 * ch);
        const f32x4 thi = *reinterpret_cast<const f32x4*>(gtot + 8 * ch + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Ge[e] = lo[e];
            Ge[e + 4] = hi[e];
            Gt[e] = tlo[e];
            Gt[e + 4] = thi[e];
        }
    }
    auto gcur = [&](int e) { return e < 4 ? gch_lo[e] : gch_hi[e - 4]; };
    const uint32_t kcw[4] = {kchw.x, kchw.y, kchw.z, kchw.w};
    const uint32_t qcw[4] = {qchw.x, qchw.y, qchw.z, qchw.w};
    auto bfe = [](const uint32_t (&w)[4], int e) {
        return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    };
    if (0 < pos) {
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = bfe(kc, e) * (kPerKey ? Ge[e] * gcur(e) : Gg * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < pos) coef[grp] = f32x2{ck, cq};
    }
    if (wave == 0) {  // groups 0..3: token coefficients, decayed by every gate of the window
        const half_t* kt = reinterpret_cast<const half_t*>(&ktw);
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = static_cast<float>(kt[e]) * (kPerKey ? Gt[e] * gcur(e) : Gall * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0) ctok[grp] = f32x2{ck, cq};
    }
    if (first) {
        const float c0 = cr * Gall * gr;  // c_r Gamma_{1:l} at row r
        rowv[r] = f32x2{c0 * kr, c0 * qr};
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    __syncthreads();

    // ---- payload sweep, scaled per column; then token and record terms
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x2 rv = rowv[lq_row(it, wave, ro)];
        const f32x4 zf = unpack_codes(zw[it]);
        p1 += zf * rv.x;
        p2 += zf * rv.y;
    }
    p1 *= bsc;
    p2 *= bsc;
    if (owner < kTok) {
        const half_t* ut = reinterpret_cast<const half_t*>(&utw);
        const f32x4 u = {static_cast<float>(ut[0]), static_cast<float>(ut[1]), static_cast<float>(ut[2]),
                         static_cast<float>(ut[3])};
        const f32x2 c = ctok[owner];
        p1 += u * c.x;
        p2 += u * c.y;
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
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

// ---------------------------------------------------------------- the window's last step
// The step as in the per-row bf16 boundary (column-owner record terms, scaled records
// staged transposed for the bf16-split MFMA), with the payload terms scaled by B and c
// and the token pairs added; then S_W is formed on the matrix cores (payload init, the
// records' two bf16 MFMAs per tile, the tokens' one fp32 MFMA per tile), passed through
// LDS into the refit's register layout, and refitted. The first floats of dynamic LDS are
// one region used three times: the step and the contraction operands, then the state on
// its way between the two register layouts (half of it at a time), then the refit's arrays.
// After it lie W (the old Ut, the refit's start) and the old payload's B / 127. The region
// is sized to the largest of the three (44 KB of LDS in all), so that three workgroups
// share a CU.
constexpr int kZsStride = kD / 4 + 1;
// floats of the step-phase region: Kt (4 KB), Ut (12 KB), Zs, Ktok, Utok, red, recp
constexpr int kStepFloats = 2 * kD * 4 + 3 * 2 * kD * 4 + kD * kZsStride + 2 * kTok * kD + 4 * kD * 2 + kD * 2;
constexpr int cmax3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
constexpr int kTransitFloats = kD * kD / 2;  // half the state in LDS during S^T Y
constexpr int kLqRegionFloats = kStepFloats > kTransitFloats + 2 * 4 * kD ? kStepFloats : kTransitFloats + 2 * 4 * kD;
constexpr int kLqBoundaryFloats = kLqRegionFloats + 4 * kD + kD;
static_assert(kLqRegionFloats % 4 == 0, "W after the region must be 16-byte aligned");

// The half state in LDS during S^T Y: row r in 16-byte units, unit u stored at u ^ f(r) with
// f(r) = (r & 7) ^ ((r & 1) << 3), so that the tile-layout writes and the 16-row slice reads
// both spread over the banks.
__device__ __forceinline__ f32x4& state_unit(float* base, int r, int u) {
    return reinterpret_cast<f32x4*>(base + r * kD)[u ^ ((r & 7) ^ ((r & 1) << 3))];
}

// The writer of the tile layout: acc[a][ct] is row 16(2w + a) + (l & 15), columns
// 16ct + 4(l >> 4) .. +3; stores the wave's 32 rows as rows r0 .. r0+31 of the buffer.
struct TileRows {
    const f32x4 (&acc)[2][8];
    int lane;
    __device__ void operator()(float* base, int r0) const {
        const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) state_unit(base, r0 + 16 * a + lr, 4 * ct + lq) = acc[a][ct];
    }
};

// ---------------------------------------------------------------- the refit in the MFMA tile layout
// The boundaries form S_W on the matrix cores in a tile layout: lane l of wave w holds, in tile
// ct of band a, key row 16(2w + a) + (l & 15) and value columns 16ct + 4(l >> 4) .. +3. This refit
// keeps the state there (64 fp32 registers):
//  * S V (the fit's Y, and the new key tokens) on v_mfma_f32_4x4x1_16b_f32. A block of 4 lanes
//    (4b .. 4b+3) holds 4 consecutive rows of the same columns, so one state element per lane is
//    the block's A operand and V of that column, one token per lane, its B operand; register i of
//    lane 4b + j accumulates row i of the block, token j. The 4 lane groups (l >> 4) end with partial
//    sums over their columns, added by two transposing lane swaps.
//  * S^T Y sums over the rows, which lie along the 16 lanes of a DPP row here, so the state passes
//    through LDS in two halves of 32 KB into slices of 16 rows by 4 columns per lane, where a
//    column's rows sum over 8 lanes (as in the register layout of the plain-state conversion).
//  * The residual S - Kt Ut^T on v_mfma_f32_16x16x4f32, whose result layout is the tile layout: A
//    the negated value tokens of 16 columns, B the key tokens of 16 rows, 4 tokens per instruction.
//  * The smoothing sum of a row stays in the 4 lanes that hold it; the column absmax reduces over
//    the 16 lanes of a DPP row, then over the 4 waves through LDS.
// LDS (floats): part A (32 KB) holds the half state during S^T Y, then the staged code rows, the
// rounded tokens Kr, Ur [128][kT], the per-wave column maxima [4][128] and the code scales [128];
// then V^T [kT][128] and Y [128][kT] (also the new key tokens). W [128][kT] (the fit's start and
// the S^T Y result) lies outside the region.
template <int kT, int kBits>
struct TileRefitLds {
    using Cfg = RefitCfg<kT, kBits>;
    static constexpr int kA = kTransitFloats;
    static constexpr int kRegionFloats = kA + 2 * kT * kD;
    static constexpr int kWFloats = kT * kD;
    static_assert(kD * Cfg::kCodeStride + 2 * kT * kD + 4 * kD + kD <= kA, "part A holds the code rows and the small arrays");
    float* half;
    uint32_t* codes;
    float *Kr, *Ur, *cmax, *sc, *VT, *Y;
    f32x4* W;
    __device__ TileRefitLds(float* region, float* w_area)
        : half(region), codes(reinterpret_cast<uint32_t*>(region)), Kr(region + kD * Cfg::kCodeStride),
          Ur(Kr + kT * kD), cmax(Ur + kT * kD), sc(cmax + 4 * kD), VT(region + kA), Y(VT + kT * kD),
          W(reinterpret_cast<f32x4*>(w_area)) {}
};

// Max over the 16 lanes of each DPP row of non-negative floats, compared as their bit patterns
// (integer max takes the DPP operand directly; a float max would first quiet each operand).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t row16_max_bits(uint32_t x) {
    x = max(x, dpp_u<kDppXor1>(x));
    x = max(x, dpp_u<kDppXor2>(x));
    x = max(x, dpp_u<kDppRor8>(x));
    return max(x, dpp_u<kDppRor4>(x));
}

// W -> V^T: modified Gram-Schmidt over the kT columns of W in order (one wave, lane l holding
// rows 2l and 2l + 1; the wave rotates with the workgroup so that the serial work does not
// always fall on the same SIMD); a column with zero norm after the projections stays zero.
template <int kT>
__device__ __forceinline__ void tile_mgs(const f32x4* W, float* VT, int wave, int lane) {
    constexpr int kC = kT / 4;
    if (wave == static_cast<int>(blockIdx.x & 3)) {
        float a[kT], b[kT];
#pragma unroll
        for (int h = 0; h < kC; ++h) {
            const f32x4 wa = W[(2 * lane) * kC + h], wb = W[(2 * lane + 1) * kC + h];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[4 * h + e] = wa[e];
                b[4 * h + e] = wb[e];
            }
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) {
#pragma unroll
            for (int g = 0; g < t; ++g) {
                const float d = wave_sum(a[g] * a[t] + b[g] * b[t]);
                a[t] -= d * a[g];
                b[t] -= d * b[g];
            }
            const float n2 = wave_sum(a[t] * a[t] + b[t] * b[t]);
            const float inv = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
            a[t] *= inv;
            b[t] *= inv;
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x2*>(VT + t * kD + 2 * lane) = f32x2{a[t], b[t]};
    }
    __syncthreads();
}

// Y = S V into Y [128][kT] (the caller adds the barrier before Y is read).
template <int kT>
__device__ __forceinline__ void tile_sv(const f32x4 (&s)[2][8], const float* VT, float* Y, int wave, int lane) {
    const int lq = lane >> 4, j = lane & 3;
#pragma unroll
    for (int g = 0; g < kT / 4; ++g) {
        f32x4 d[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a) d[a][0] = d[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float* vrow = VT + (4 * g + j) * kD + 4 * lq;  // V of columns 16ct + 4lq + e, token 4g + j
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 vb = *reinterpret_cast<const f32x4*>(vrow + 16 * ct);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d[0][ct & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(s[0][ct][e], vb[e], d[0][ct & 1], 0, 0, 0);
                d[1][ct & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(s[1][ct][e], vb[e], d[1][ct & 1], 0, 0, 0);
            }
        }
        const f32x4 d0 = d[0][0] + d[0][1], d1 = d[1][0] + d[1][1];
        // register i of lane l: row 16(2w + a) + 4((l & 15) >> 2) + i, token 4g + (l & 3), summed over the
        // columns of lane group l >> 4; the swaps sum the 4 groups and leave each lane two of the 8 values
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = add_pair16(d0[i], d1[i]);   // bit 4 clear: band 0, set: band 1
        const float w0 = add_pair32(u[0], u[2]), w1 = add_pair32(u[1], u[3]);  // bit 5 clear: i = 0, 1; set: 2, 3
        const int row = 16 * (2 * wave + ((lane >> 4) & 1)) + 4 * ((lane & 15) >> 2) + 2 * (lane >> 5);
        Y[row * kT + 4 * g + j] = w0;
        Y[(row + 1) * kT + 4 * g + j] = w1;
        // the next token group's operand loads stay behind this group's (registers)
        if (kT == 8) __builtin_amdgcn_sched_barrier(0);
    }
}

// W = S^T Y: the tile state goes to LDS half by half (rows 0 .. 63 from waves 0 and 1, then
// 64 .. 127), each half is read back as slices of 16 rows by 4 columns (lane l of wave w: columns
// 4(8w + (l & 7)) .. +3, rows 8it + (l >> 3)) and multiplied by Y, and the partial sums reduce
// over the 8 row lanes as in the plain-state layout (refit_sty). Ends with a barrier.
template <int kT, int kBits>
__device__ __forceinline__ void tile_sty(const TileRefitLds<kT, kBits>& L, const f32x4 (&s)[2][8], int wave, int lane) {
    constexpr int kC = kT / 4, kJ = kT / 2;
    const int uu = 8 * wave + (lane & 7), ro = lane >> 3;
    const int b3 = ro & 1, b4 = (ro >> 1) & 1, b5 = ro >> 2;
    f32x4 acc[4][kC];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h = 0; h < kC; ++h) acc[e][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        if ((wave >> 1) == hf) TileRows{s, lane}(L.half, 32 * (wave & 1));
        __syncthreads();
        // (with 8 tokens the slice is consumed two rows at a time: a fully unrolled loop loads
        // all of it, and Y, ahead of the products and runs out of registers)
        constexpr int kSliceUnroll = kT == 8 ? 4 : 8;
#pragma unroll kSliceUnroll
        for (int it = 0; it < 8; ++it) {
            const f32x4 sv = state_unit(L.half, 8 * it + ro, uu);
            const int row = 8 * (8 * hf + it) + ro;
#pragma unroll
            for (int h = 0; h < kC; ++h) {
                f32x4 yv;
                if constexpr (kT == 8) {
                    yv = reinterpret_cast<const f32x4*>(L.Y)[row * kC + (h ^ b3)];
                } else {
                    const f32x2* Y2 = reinterpret_cast<const f32x2*>(L.Y);
                    const f32x2 lo = Y2[row * 2 + b3], hi = Y2[row * 2 + (b3 ^ 1)];
                    yv = f32x4{lo.x, lo.y, hi.x, hi.y};
                }
                acc[0][h] = axpy(sv.x, yv, acc[0][h]);
                acc[1][h] = axpy(sv.y, yv, acc[1][h]);
                acc[2][h] = axpy(sv.z, yv, acc[2][h]);
                acc[3][h] = axpy(sv.w, yv, acc[3][h]);
            }
        }
        __syncthreads();
    }
    float ra[4][kJ];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < kJ; ++j)
            ra[e][j] = acc[e][0][j] + dpp<kDppRor8>(kT == 8 ? acc[e][kC - 1][j] : acc[e][0][(j + 2) & 3]);
    float rb[2][kJ];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < kJ; ++j) rb[e][j] = add_pair16(ra[e][j], ra[e + 2][j]);
    float* Wf = reinterpret_cast<float*>(L.W) + (4 * uu + 2 * b4 + b5) * kT + kJ * b3;
    if constexpr (kT == 8) {
        *reinterpret_cast<f32x4*>(Wf) = f32x4{add_pair32(rb[0][0], rb[1][0]), add_pair32(rb[0][1], rb[1][1]),
                                               add_pair32(rb[0][2], rb[1][2]), add_pair32(rb[0][3], rb[1][3])};
    } else {
        *reinterpret_cast<f32x2*>(Wf) = f32x2{add_pair32(rb[0][0], rb[1][0]), add_pair32(rb[0][1], rb[1][1])};
    }
    __syncthreads();
}

// The refit of one head from the tile layout (s: the state, consumed). On entry W holds the start
// vectors; every thread of the workgroup calls it. Writes the codes (Zh: the head's payload as
// 32-bit words), B, c and the fp16 tokens [kT][128].
template <int kT, int kBits>
__device__ __forceinline__ void lq_refit_tiles(const TileRefitLds<kT, kBits>& L, f32x4 (&s)[2][8], int n_iter,
                                               int tid, uint32_t* __restrict__ Zh, float* __restrict__ Bh,
                                               float* __restrict__ Ch, half_t* __restrict__ Kh,
                                               half_t* __restrict__ Uh) {
    using Cfg = RefitCfg<kT, kBits>;
    constexpr int kC = kT / 4;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    tile_mgs<kT>(L.W, L.VT, wave, lane);
    for (int it = 0; it < n_iter; ++it) {
        tile_sv<kT>(s, L.VT, L.Y, wave, lane);
        __syncthreads();
        tile_sty(L, s, wave, lane);
        tile_mgs<kT>(L.W, L.VT, wave, lane);
    }
    tile_sv<kT>(s, L.VT, L.Y, wave, lane);  // Kt = S V
    __syncthreads();

    // fp16 tokens (stored), and their exact fp32 values for the residual
    if (tid < kD) {
#pragma unroll
        for (int h = 0; h < kC; ++h) {
            const f32x4 kv = *reinterpret_cast<const f32x4*>(L.Y + tid * kT + 4 * h);
            f32x4 kr, ur;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const half_t kh = static_cast<half_t>(kv[e]);
                const half_t uh = static_cast<half_t>(L.VT[(4 * h + e) * kD + tid]);
                kr[e] = static_cast<float>(kh);
                ur[e] = static_cast<float>(uh);
                Kh[(4 * h + e) * kD + tid] = kh;
                Uh[(4 * h + e) * kD + tid] = uh;
            }
            *reinterpret_cast<f32x4*>(L.Kr + tid * kT + 4 * h) = kr;
            *reinterpret_cast<f32x4*>(L.Ur + tid * kT + 4 * h) = ur;
        }
    }
    __syncthreads();

    // residual R = S - Kt Ut^T on the matrix cores: tile (a, ct) += (-Ut of columns 16ct + m) (Kt of
    // rows 16(2w + a) + n)^T, 4 tokens per instruction
#pragma unroll
    for (int g = 0; g < kC; ++g) {
        const float bk0 = L.Kr[(32 * wave + lr) * kT + 4 * g + lq];
        const float bk1 = L.Kr[(32 * wave + 16 + lr) * kT + 4 * g + lq];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float au = -L.Ur[(16 * ct + lr) * kT + 4 * g + lq];
            s[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(au, bk0, s[0][ct], 0, 0, 0);
            s[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(au, bk1, s[1][ct], 0, 0, 0);
        }
    }

    // smoothing: each row's sum of |R| over its 32 columns per lane and the 4 lanes that hold it
    float ic[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        float t = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            t += (fabsf(s[a][ct].x) + fabsf(s[a][ct].y)) + (fabsf(s[a][ct].z) + fabsf(s[a][ct].w));
        t = add_xor32(add_xor16(t));
        const float cs = fmaxf(sqrtf(t * (1.f / kD)), kSmoothFloor);
        ic[a] = 1.f / cs;
        if (lq == 0) Ch[32 * wave + 16 * a + lr] = cs;
    }

    // X = R / c, the per-value-channel absmax B (the lane's two rows, its DPP row, then the 4
    // waves) and the code scale qmax / B
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        s[0][ct] = scale(ic[0], s[0][ct]);
        s[1][ct] = scale(ic[1], s[1][ct]);
        u32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m[e] = row16_max_bits(__float_as_uint(fmaxf(fabsf(s[0][ct][e]), fabsf(s[1][ct][e]))));
        if (lr == 0) *reinterpret_cast<u32x4*>(L.cmax + wave * kD + 16 * ct + 4 * lq) = m;
    }
    __syncthreads();
    uint32_t* cmw = reinterpret_cast<uint32_t*>(L.cmax);
    if (tid < kD) {
        const float B = __uint_as_float(max(max(cmw[tid], cmw[kD + tid]), max(cmw[2 * kD + tid], cmw[3 * kD + tid])));
        Bh[tid] = B;
        // a column maximum below 2^-64 scales the column by 2^64 first (exact). The factor goes
        // to slot tid of cmax and the wave's "any such column" flag (lane 0) to slot kD + tid:
        // slots only this thread has read.
        const float f = tiny_factor(B);
        L.sc[tid] = B > 0.f ? __fdiv_rn(static_cast<float>(Cfg::kQmax), B * f) : 0.f;
        L.cmax[tid] = f;
        const bool any_tiny = __ballot(f != 1.f) != 0;
        if (lane == 0) cmw[kD + tid] = any_tiny;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(cmw[kD] | cmw[kD + 64])) {  // rare
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 f = *reinterpret_cast<const f32x4*>(L.cmax + 16 * ct + 4 * lq);
            s[0][ct] *= f;
            s[1][ct] *= f;
        }
    }

    // codes of the lane's 4 columns in each of its two rows, staged so that whole rows leave together
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(L.sc + 16 * ct + 4 * lq);
        const int u = 4 * ct + lq;  // the 4-column unit
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int row = 32 * wave + 16 * a + lr;
            const f32x4 x = s[a][ct];
            if constexpr (kBits == 8) {
                L.codes[row * Cfg::kCodeStride + u] =
                    pack_low_bytes(lq_code_t<8>(x.x * sc.x), lq_code_t<8>(x.y * sc.y), lq_code_t<8>(x.z * sc.z),
                                   lq_code_t<8>(x.w * sc.w));
            } else if constexpr (kBits == 4) {
                reinterpret_cast<uint16_t*>(L.codes)[row * 2 * Cfg::kCodeStride + u] = static_cast<uint16_t>(
                    (lq_code_t<4>(x.x * sc.x) & 0xfu) | ((lq_code_t<4>(x.y * sc.y) & 0xfu) << 4) |
                    ((lq_code_t<4>(x.z * sc.z) & 0xfu) << 8) | ((lq_code_t<4>(x.w * sc.w) & 0xfu) << 12));
            } else {
                const uint32_t z0 = lq_code_t<6>(x.x * sc.x), z1 = lq_code_t<6>(x.y * sc.y);
                const uint32_t z2 = lq_code_t<6>(x.z * sc.z), z3 = lq_code_t<6>(x.w * sc.w);
                reinterpret_cast<uint16_t*>(L.codes)[row * 2 * Cfg::kCodeStride + u] = static_cast<uint16_t>(
                    ((z0 >> 2) & 0xfu) | (((z1 >> 2) & 0xfu) << 4) | (((z2 >> 2) & 0xfu) << 8) | (((z3 >> 2) & 0xfu) << 12));
                reinterpret_cast<uint8_t*>(L.codes)[row * 4 * Cfg::kCodeStride + 64 + u] =
                    static_cast<uint8_t>((z0 & 3u) | ((z1 & 3u) << 2) | ((z2 & 3u) << 4) | ((z3 & 3u) << 6));
            }
        }
    }
    __syncthreads();
    constexpr int kQuads = Cfg::kRowWords / 4;  // 16-byte pieces per row
#pragma unroll
    for (int mm = 0; mm < kD * kQuads / kThreads; ++mm) {
        const int qd = tid + kThreads * mm;
        const int row = qd / kQuads, d = 4 * (qd % kQuads);
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(L.codes + row * Cfg::kCodeStride + d);
        __builtin_nontemporal_store(w4, reinterpret_cast<u32x4*>(Zh + row * Cfg::kRowWords + d));
    }
}

// ---------------------------------------------------------------- conversion of a plain state
// The state is loaded straight into the tile layout, the start is the first kT Walsh columns.
template <int kT, int kBits>
__global__ __launch_bounds__(kThreads) void lq_quantize_kernel(const float* __restrict__ S, int n_iter,
                                                               uint32_t* __restrict__ Z, float* __restrict__ B,
                                                               float* __restrict__ Cs, half_t* __restrict__ Kc,
                                                               half_t* __restrict__ Uc) {
    using L_t = TileRefitLds<kT, kBits>;
    constexpr int kC = kT / 4;
    extern __shared__ __align__(16) float lds[];
    const L_t L(lds, lds + L_t::kRegionFloats);
    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    const float* Sh = S + static_cast<size_t>(h) * kD * kD;
    f32x4 s[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) s[a][ct] = stream_load(Sh + (32 * wave + 16 * a + lr) * kD + 16 * ct + 4 * lq);
    if (tid < kD) {  // the first kT Walsh columns: (-1)^popcount(i & t) / sqrt(128)
        constexpr float sq = 0.08838834764831845f;
#pragma unroll
        for (int hh = 0; hh < kC; ++hh) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__builtin_popcount(tid & (4 * hh + e)) & 1) ? -sq : sq;
            L.W[tid * kC + hh] = w;
        }
    }
    __syncthreads();
    const size_t vo = static_cast<size_t>(h) * kD;
    lq_refit_tiles(L, s, n_iter, tid, Z + static_cast<size_t>(h) * kD * RefitCfg<kT, kBits>::kRowWords, B + vo,
                   Cs + vo, Kc + vo * kT, Uc + vo * kT);
}

__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const __bf16 a = static_cast<__bf16>(x);
    const float r1 = x - static_cast<float>(a);
    const __bf16 b = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(b);
    const __bf16 c = static_cast<__bf16>(r2);
    hi = __builtin_bit_cast(uint16_t, a);
    mid = __builtin_bit_cast(uint16_t, b);
    lo = __builtin_bit_cast(uint16_t, c);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kThreads) void lq_boundary_kernel(
    int W, int pos, int n_iter, int8_t* __restrict__ Z, float* __restrict__ Bcol, float* __restrict__ Csm,
    half_t* __restrict__ Kc, half_t* __restrict__ Uc, const bf16_t* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    constexpr int kRec = 16;
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ f32x2 rowv[kD];
    __shared__ f32x2 coef[kRec];
    __shared__ f32x2 ctok[kTok];
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];
    __shared__ float gam[kRec];

    // step-phase views of the dynamic region
    u32x4* Kt = reinterpret_cast<u32x4*>(dyn_lds);                 // [2][128]
    u32x4* Ut = Kt + 2 * kD;                                        // [3][2][128]
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Ut + 3 * 2 * kD);   // [128][33]
    float* Ktok = reinterpret_cast<float*>(Zs + kD * kZsStride);   // [4][128]
    float* Utok = Ktok + kTok * kD;                                 // [4][128], scaled by Gamma_{1:W}
    f32x2* red = reinterpret_cast<f32x2*>(Utok + kTok * kD);       // [4][128]
    f32x2* recp = red + 4 * kD;                                     // [128]
    // refit views (its region overlaps every step-phase array above; W and bscs do not)
    static_assert(TileRefitLds<4, 8>::kRegionFloats <= kLqRegionFloats, "the refit's region fits");
    const TileRefitLds<4, 8> LT(dyn_lds, dyn_lds + kLqRegionFloats);
    f32x4* const LW = LT.W;
    float* bscs = dyn_lds + kLqRegionFloats + 4 * kD;   // B / 127 of the old payload

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const int grp = tid >> 4, ch = tid & 15;
    const int cc = tid & (kD - 1), half = tid >> 7;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kTok * kD;
    const bool first = tid < kD;

    // ---- loads
    uint32_t kcr[4] = {0u, 0u, 0u, 0u};
    if (0 < pos) {
        const uint4 x = *reinterpret_cast<const uint4*>(Kbuf + rec0 + static_cast<size_t>(grp < pos ? grp : 0) * kD + 8 * ch);
        kcr[0] = x.x; kcr[1] = x.y; kcr[2] = x.z; kcr[3] = x.w;
    }
    float ucol[8];
    uint32_t kcol[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const size_t at = rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + cc;
        const float ul = Ubuf[at];  // unconditional: at is clamped to slot 0 (in bounds), the value dropped for j >= pos
        const uint32_t kl = static_cast<uint32_t>(Kbuf[at]);
        ucol[e] = j < pos ? ul : 0.f;
        const uint32_t kb = j < pos ? kl : 0u;
        kcol[e >> 1] = (e & 1) ? (kcol[e >> 1] | (kb << 16)) : kb;
    }
    uint4 ktw = {0u, 0u, 0u, 0u};
    if (grp < kTok) ktw = *reinterpret_cast<const uint4*>(Kc + tok0 + grp * kD + 8 * ch);
    // token t at row / column cc (threads < 128: keys; threads >= 128: values)
    half_t tokv[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) tokv[t] = (first ? Kc : Uc)[tok0 + t * kD + cc];
    const float g_lane = lane < pos ? Gbuf[static_cast<size_t>(h) * W + lane] : 1.f;
    const uint4 kchw = *reinterpret_cast<const uint4*>(k + vec_off + 8 * ch);
    const uint4 qchw = *reinterpret_cast<const uint4*>(q + vec_off + 8 * ch);
    const float kr = load_in(k, vec_off + cc), qr = load_in(q, vec_off + cc);
    const float gr = gate[h];
    const float cr = Csm[vec_off + cc];
    const float bcc = Bcol[vec_off + cc];
    const float vr = load_in(v, vec_off + cc);
    const float bt = beta[h];
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + lq_row(it, wave, ro) * (kD / 4) + c4);

    // ---- gate products (newest first): after record grp, after record = lane, all
    // (a suffix scan over the record lanes, g = 1 from record pos on)
    const float Sfx = suffix_prod<16>(g_lane, lane);
    const float Gl = suffix_prod_excl<16>(Sfx, lane);
    const float Gg = lane_gather(Gl, grp), Gall = lane_value(Sfx, 0);
    const float gam_all = Gall * gr;  // Gamma_{1:W}
    if (wave == 0 && lane < kRec) gam[lane] = lane < pos ? Gl * gr : 1.f;
    const uint32_t kcw[4] = {kchw.x, kchw.y, kchw.z, kchw.w};
    const uint32_t qcw[4] = {qchw.x, qchw.y, qchw.z, qchw.w};
    auto bfe = [](const uint32_t (&w)[4], int e) {
        return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    };
    if (0 < pos) {
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = bfe(kcr, e) * (Gg * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < pos) coef[grp] = f32x2{ck, cq};
    }
    if (wave == 0) {
        const half_t* kt = reinterpret_cast<const half_t*>(&ktw);
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = static_cast<float>(kt[e]) * gam_all;
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0) ctok[grp] = f32x2{ck, cq};
    }
    if (first) {
        const float c0 = cr * gam_all;
        rowv[cc] = f32x2{c0 * kr, c0 * qr};
        zcoef[cc] = c0;
        bscs[cc] = bcc * (1.f / 127.f);
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    // token operands of the contraction, and the unscaled values as the refit's start
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        const float x = static_cast<float>(tokv[t]);
        if (first) Ktok[t * kD + cc] = x;
        else Utok[t * kD + cc] = x * gam_all;
    }
    if (!first) LW[cc] = f32x4{static_cast<float>(tokv[0]), static_cast<float>(tokv[1]),
                               static_cast<float>(tokv[2]), static_cast<float>(tokv[3])};
    Kt[half * kD + cc] = u32x4{kcol[0], kcol[1], kcol[2], kcol[3]};
    __syncthreads();

    // ---- payload sweep; record terms per column; scaled records staged for the MFMA
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x2 rvv = rowv[lq_row(it, wave, ro)];
        const f32x4 zf = unpack_codes(zw[it]);
        p1 += zf * rvv.x;
        p2 += zf * rvv.y;
    }
    f32x2 rp = {0.f, 0.f};
    u32x4 part[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const f32x2 c = j < pos ? coef[j] : f32x2{0.f, 0.f};
        rp += c * ucol[e];
        uint32_t hi, mid, lo;
        split3_bf16(gam[j] * ucol[e], hi, mid, lo);
        const int sh = 16 * (e & 1);
        part[0][e >> 1] = (e & 1) ? (part[0][e >> 1] | (hi << sh)) : hi;
        part[1][e >> 1] = (e & 1) ? (part[1][e >> 1] | (mid << sh)) : mid;
        part[2][e >> 1] = (e & 1) ? (part[2][e >> 1] | (lo << sh)) : lo;
    }
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) Ut[(pp * 2 + half) * kD + cc] = part[pp];
    p1 = f32x4{add_xor32(p1.x), add_xor32(p1.y), add_xor32(p1.z), add_xor32(p1.w)};
    p2 = f32x4{add_xor32(p2.x), add_xor32(p2.y), add_xor32(p2.z), add_xor32(p2.w)};
    if (ro == 0) {
        red[wave * kD + 4 * c4 + 0] = f32x2{p1.x, p2.x};
        red[wave * kD + 4 * c4 + 1] = f32x2{p1.y, p2.y};
        red[wave * kD + 4 * c4 + 2] = f32x2{p1.z, p2.z};
        red[wave * kD + 4 * c4 + 3] = f32x2{p1.w, p2.w};
    }
    if (half == 1) recp[cc] = rp;
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) Zs[lq_row(it, wave, ro) * kZsStride + c4] = zw[it];
    __syncthreads();

    // ---- correction and output; the current record joins the contraction operands
    if (first) {
        const int c = cc;
        f32x2 acc = (red[c] + red[kD + c] + red[2 * kD + c] + red[3 * kD + c]) * bscs[c];
        acc += rp + recp[c];
        const f32x4 ut = LW[c];
        acc += ctok[0] * ut.x + ctok[1] * ut.y + ctok[2] * ut.z + ctok[3] * ut.w;
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        uint32_t uh, um, ul;
        split3_bf16(u, uh, um, ul);
        reinterpret_cast<uint16_t*>(&Ut[(0 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(uh);
        reinterpret_cast<uint16_t*>(&Ut[(1 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(um);
        reinterpret_cast<uint16_t*>(&Ut[(2 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(ul);
        reinterpret_cast<uint16_t*>(&Kt[(pos >> 3) * kD + c])[pos & 7] = static_cast<uint16_t>(__float_as_uint(kr) >> 16);
    }
    __syncthreads();

    // ---- S_W on the matrix cores, both bands of the wave's 32 rows held in registers.
    // Lane l holds, in tile ct of band a, key row 32w + 16a + l%16 and value columns
    // 16ct + 4(l/16) .. +3 (result layout of v_mfma_f32_16x16x{32_bf16,4f32}).
    const int lr = lane & 15, lq = lane >> 4, blk = lq & 1;
    f32x4 acc[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, Kt[blk * kD + row]);
        const float zc = zcoef[row];
        const float bk = Ktok[lq * kD + row];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 bs = *reinterpret_cast<const f32x4*>(bscs + 16 * ct + 4 * lq);
            acc[a][ct] = unpack_codes(Zs[row * kZsStride + 4 * ct + lq]) * (bs * zc);
            const int col = 16 * ct + lr;
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, Ut[((lq < 2 ? 0 : 1) * 2 + blk) * kD + col]);
            const u32x4 lo = Ut[(2 * 2 + blk) * kD + col];
            const bf16x8 a2 = __builtin_bit_cast(bf16x8, lq < 2 ? lo : u32x4{0u, 0u, 0u, 0u});
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv, acc[a][ct], 0, 0, 0);
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, bv, acc[a][ct], 0, 0, 0);
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(Utok[lq * kD + col], bk, acc[a][ct], 0, 0, 0);
        }
    }
    __syncthreads();  // every read of the step-phase arrays is done: the region is the refit's
    lq_refit_tiles(LT, acc, n_iter, tid, Zh, Bcol + vec_off, Csm + vec_off, Kc + tok0, Uc + tok0);
}

// ---------------------------------------------------------------- the last step, per-key gates
// KDA's boundary. The step as in the general per-row int8 boundary: records, their gates
// and keys staged in LDS as fp32, the decayed keys E_j = Gamma_{j+1:W} k_j formed by one
// thread per key row walking the records backwards; the payload terms scaled by c and B,
// and the token pairs as four more records whose keys carry the whole window's decay.
// S_W = Gamma_{1:W} (C dequant(Z, B) + Kt Ut^T) + sum_j E_j u_j^T then forms on the
// matrix cores in fp32 (the decayed keys are not bf16-exact): per 16 x 16 tile the
// payload initialises the accumulator, four v_mfma_f32_16x16x4f32 add the 16 records and
// one adds the 4 tokens, in the GDN boundaries' tile layout (lane l of wave w holds, in tile ct
// of band a, row 16(2w + a) + (l & 15) and columns 16ct + 4(l >> 4) .. +3), which the refit
// keeps.
constexpr int kKdaRec = 16;
// floats of the step-phase arrays: KE, Us, Gs [16][128], Zs, decayed token keys and
// token values [4][128], red [4][128] x 2
constexpr int kKdaStepFloats = 3 * kKdaRec * kD + kD * kZsStride + 2 * kTok * kD + 4 * kD * 2;
// W (the refit's start) is written once the step arrays are dead, right after the refit's
// region; B / 127 of the old payload follows the step arrays. 50 KB in all: three workgroups
// per CU.
constexpr int kKdaWOffset = TileRefitLds<4, 8>::kRegionFloats;
static_assert(kKdaWOffset + 4 * kD <= kKdaStepFloats, "W must lie inside the step region, clear of the refit's arrays");
constexpr int kLqKdaBoundaryFloats = kKdaStepFloats + kD;

__global__ __launch_bounds__(kThreads) void lq_boundary_kda_kernel(
    int W, int pos, int n_iter, int8_t* __restrict__ Z, float* __restrict__ Bcol, float* __restrict__ Csm,
    half_t* __restrict__ Kc, half_t* __restrict__ Uc, const bf16_t* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ f32x2 rowv[kD];       // c_r Gamma_{1:W,r} (k_r, q_r)
    __shared__ f32x2 kq_row[kD];     // (k_r, q_r)
    __shared__ f32x2 coef[kKdaRec];  // per record (E_j . k, E_j . q)
    __shared__ f32x2 ctok[kTok];     // per token ((Gamma Kt_t) . k, (Gamma Kt_t) . q)
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];      // c_r Gamma_{1:W,r}

    float* KE = dyn_lds;                                            // [16][128]
    float* Us = KE + kKdaRec * kD;                                  // [16][128]
    float* Gs = Us + kKdaRec * kD;                                  // [16][128]
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Gs + kKdaRec * kD);  // [128][33]
    float* Kt4 = reinterpret_cast<float*>(Zs + kD * kZsStride);    // [4][128] Gamma_{1:W} Kt
    float* Ut4 = Kt4 + kTok * kD;                                   // [4][128] Ut
    f32x2* red = reinterpret_cast<f32x2*>(Ut4 + kTok * kD);        // [4][128]
    const TileRefitLds<4, 8> L(dyn_lds, dyn_lds + kKdaWOffset);
    float* bscs = dyn_lds + kKdaStepFloats;                         // B / 127 of the old payload

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c4 = lane & 31, ro = lane >> 5;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kTok * kD;
    uint32_t* Zh = reinterpret_cast<uint32_t*>(Z + static_cast<size_t>(h) * kD * kD);

    // ---- loads: records, gates, tokens and inputs first, then the codes
    Stager<bf16_t, kKdaRec * kD> sk;
    Stager<float, kKdaRec * kD> su;
    Stager<float, kKdaRec * kD> sg;
    sk.load(Kbuf + rec0, pos * kD, tid);
    su.load(Ubuf + rec0, pos * kD, tid);
    sg.load(Gbuf + rec0, pos * kD, tid);
    half_t tokv[kTok];  // token t at row / column r (threads < 128: keys; threads >= 128: values)
#pragma unroll
    for (int t = 0; t < kTok; ++t) tokv[t] = (first ? Kc : Uc)[tok0 + t * kD + r];
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = gate[vec_off + r];
    const float cr = Csm[vec_off + r];
    const float bcc = Bcol[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    uint32_t zw[kRowsPerThread];
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it)
        zw[it] = __builtin_nontemporal_load(Zh + lq_row(it, wave, ro) * (kD / 4) + c4);

    sk.store(KE, tid);
    su.store(Us, tid);
    sg.store(Gs, tid);
    for (int i = pos * kD + tid; i < kKdaRec * kD; i += kThreads) Us[i] = 0.f;  // rows pos .. 15
    __syncthreads();

    // ---- decayed keys in place (thread r < 128 walks key row r from the newest record),
    // read vectors, token keys with the whole window's decay; token values and the refit's
    // start (the old Ut, unscaled) from threads >= 128
    if (first) {
        float G = 1.f;
        for (int j = pos - 1; j >= 0; --j) {
            KE[j * kD + r] *= G * gr;
            G *= Gs[j * kD + r];
        }
        const float gam = G * gr;  // Gamma_{1:W} at row r
        const float c0 = cr * gam;
        rowv[r] = f32x2{c0 * kr, c0 * qr};
        kq_row[r] = f32x2{kr, qr};
        zcoef[r] = c0;
        KE[pos * kD + r] = kr;  // the current record: no decay after it
        for (int j = pos + 1; j < kKdaRec; ++j) KE[j * kD + r] = 0.f;
#pragma unroll
        for (int t = 0; t < kTok; ++t) Kt4[t * kD + r] = static_cast<float>(tokv[t]) * gam;
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    } else {
#pragma unroll
        for (int t = 0; t < kTok; ++t) Ut4[t * kD + r] = static_cast<float>(tokv[t]);
        bscs[r] = bcc * (1.f / 127.f);
    }
    __syncthreads();

    // ---- record and token coefficients: the 16 lanes of a DPP row reduce one (8 rows each)
    {
        const int chunk = tid & 15, j = tid >> 4;
        auto dot8 = [&](const float* e) {
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(e + 8 * chunk);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(e + 8 * chunk + 4);
            const f32x2* kqr = kq_row + 8 * chunk;
            f32x2 c = e0.x * kqr[0] + e0.y * kqr[1] + e0.z * kqr[2] + e0.w * kqr[3] + e1.x * kqr[4] +
                      e1.y * kqr[5] + e1.z * kqr[6] + e1.w * kqr[7];
            return f32x2{row16_sum(c.x), row16_sum(c.y)};
        };
        const f32x2 c = dot8(KE + (j < pos ? j : 0) * kD);
        if (chunk == 0 && j < pos) coef[j] = c;
        if (wave == 0) {  // groups 0..3 again: the tokens
            const f32x2 ct = dot8(Kt4 + j * kD);
            if (chunk == 0) ctok[j] = ct;
        }
    }
    __syncthreads();

    // ---- payload sweep scaled per column, record and token terms; codes re-laid out
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) {
        const f32x2 rv = rowv[lq_row(it, wave, ro)];
        const f32x4 zf = unpack_codes(zw[it]);
        p1 += zf * rv.x;
        p2 += zf * rv.y;
    }
    const f32x4 bs = *reinterpret_cast<const f32x4*>(bscs + 4 * c4);
    p1 *= bs;
    p2 *= bs;
    const int owner = 2 * wave + ro;
    for (int j = owner; j < pos; j += 8) {
        const f32x2 c = coef[j];
        const f32x4 u = *reinterpret_cast<const f32x4*>(Us + j * kD + 4 * c4);
        p1 += u * c.x;
        p2 += u * c.y;
    }
    if (owner < kTok) {
        const f32x2 c = ctok[owner];
        const f32x4 u = *reinterpret_cast<const f32x4*>(Ut4 + owner * kD + 4 * c4);
        p1 += u * c.x;
        p2 += u * c.y;
    }
    p1 = f32x4{add_xor32(p1.x), add_xor32(p1.y), add_xor32(p1.z), add_xor32(p1.w)};
    p2 = f32x4{add_xor32(p2.x), add_xor32(p2.y), add_xor32(p2.z), add_xor32(p2.w)};
    if (ro == 0) {
        red[wave * kD + 4 * c4 + 0] = f32x2{p1.x, p2.x};
        red[wave * kD + 4 * c4 + 1] = f32x2{p1.y, p2.y};
        red[wave * kD + 4 * c4 + 2] = f32x2{p1.z, p2.z};
        red[wave * kD + 4 * c4 + 3] = f32x2{p1.w, p2.w};
    }
#pragma unroll
    for (int it = 0; it < kRowsPerThread; ++it) Zs[lq_row(it, wave, ro) * kZsStride + c4] = zw[it];
    __syncthreads();

    // ---- correction and output; u of this step becomes row pos of Us
    if (first) {
        const int c = tid;
        const f32x2 acc = red[c] + red[kD + c] + red[2 * kD + c] + red[3 * kD + c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        Us[pos * kD + c] = u;
    }
    __syncthreads();

    // ---- S_W on the matrix cores, both 16-row bands of the wave held in registers
    const int lr = lane & 15, lq = lane >> 4;
    // (A: the records' and tokens' values of columns 16ct + m; B: their decayed keys of rows
    // 16(2w + a) + n; the result layout is the tile layout)
    f32x4 acc[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const float zc = zcoef[row];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 bs = *reinterpret_cast<const f32x4*>(bscs + 16 * ct + 4 * lq);
            acc[a][ct] = unpack_codes(Zs[row * kZsStride + 4 * ct + lq]) * (bs * zc);
        }
    }
#pragma unroll
    for (int s4 = 0; s4 < kKdaRec / 4; ++s4) {
        const float eb0 = KE[(4 * s4 + lq) * kD + 32 * wave + lr], eb1 = KE[(4 * s4 + lq) * kD + 32 * wave + 16 + lr];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float ua = Us[(4 * s4 + lq) * kD + 16 * ct + lr];
            acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua, eb0, acc[0][ct], 0, 0, 0);
            acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua, eb1, acc[1][ct], 0, 0, 0);
        }
    }
    {
        const float kb0 = Kt4[lq * kD + 32 * wave + lr], kb1 = Kt4[lq * kD + 32 * wave + 16 + lr];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float ut = Ut4[lq * kD + 16 * ct + lr];
            acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ut, kb0, acc[0][ct], 0, 0, 0);
            acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ut, kb1, acc[1][ct], 0, 0, 0);
        }
    }
    __syncthreads();  // every read of the step-phase arrays is done: the region is the refit's, and W
    if (!first)
        L.W[r] = f32x4{static_cast<float>(tokv[0]), static_cast<float>(tokv[1]), static_cast<float>(tokv[2]),
                       static_cast<float>(tokv[3])};
    __syncthreads();
    lq_refit_tiles(L, acc, n_iter, tid, Zh, Bcol + vec_off, Csm + vec_off, Kc + tok0, Uc + tok0);
}

// ---------------------------------------------------------------- 4 and 6 bits
// LeapQuant at 4 bits (sec. 4.1 fits r = 8 tokens there): codes in [-7, 7], two per byte
// (the even column in the low nibble), dequant Z B / 7, 8 KiB of payload per head.
// At 6 bits (r = 4 tokens): codes in [-31, 31], dequant Z B / 31, a row of 96 bytes: the
// high parts z >> 2 as nibbles in the 4-bit layout (bytes 0..63), then the low parts z & 3,
// four per byte, column 4b + i in bits 2i .. 2i+1 of byte 64 + b; 12 KiB per head.
// The low-bit sweep has its own layout: lane l of wave w owns the 32-bit nibble word of 8
// columns 8 (l & 15) .. +7 (and at 6 bits their 16 bits of low parts) in the rows
// 16 it + 4 w + (l >> 4), it = 0..7; a word's 4 row lanes (l, l^16, l^32, l^48) combine by
// lane swaps, the 4 waves through LDS. Record and token terms are added per value column:
// thread c + 128 h (h = 0, 1) adds records 8h .. 8h+7 and the h-th half of the tokens.
template <int kBits>
struct LowBits {
    static_assert(kBits == 4 || kBits == 6, "4- or 6-bit codes");
    static constexpr int kT = kBits == 4 ? 8 : 4;           // compensator tokens
    static constexpr int kTh = kT / 2;                       // tokens per column thread
    static constexpr int kC = kT / 4;                        // f32x4 chunks of a token vector
    static constexpr int kQmax = (1 << (kBits - 1)) - 1;     // 7 or 31
    static constexpr int kRowWords = kD * kBits / 32;        // 16 or 24 words per row
    static constexpr int kZsStride = kRowWords + 1;          // staged row stride of the boundary
    // the sweep multiplies by 16 z (4 bits) or 4 z (6 bits): the read vectors carry the inverse
    static constexpr float kReadScale = kBits == 4 ? 0.0625f : 0.25f;
};

__device__ __forceinline__ int low_row(int it, int wave, int rl) { return 16 * it + 4 * wave + rl; }

// Payload sweep of the low-bit steps: the lane's 8 code words (rows low_row(it, wave, l >> 4),
// value columns 8 (l & 15) .. +7) against the two read vectors, whose rowv entries are the read
// vectors times kReadScale. A 4-bit code is read as the signed high nibble of a byte, i.e. as
// 16 z with one sign-extending byte conversion (the even columns from w << 4, the odd ones from
// w). At 6 bits the nibble is the high part and the low part z & 3 goes into bits 2..3 of the
// same byte, which then reads 16 (z >> 2) + 4 (z & 3) = 4 z. Either way the products equal z
// times the unscaled entries exactly. The 4 row lanes l, l^16, l^32, l^48 are
// summed by two lane swaps that halve the live values: lanes with bit 4 set keep columns 4..7 of
// the eight, lanes with bit 5 set the upper pair of their four. Each lane stores {p1, p2} of its two
// columns 4 b4 + 2 b5 + (0, 1) into red_w (the wave's [128] partials).
template <int kBits>
__device__ __forceinline__ void sweep_low(const uint32_t (&zw)[8], const uint32_t (&zl)[8], const f32x2* rowv,
                                          int wave, int lane, f32x2* red_w) {
    const int c16 = lane & 15, rl = lane >> 4;
    float p1[8], p2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p1[e] = p2[e] = 0.f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const f32x2 rv = rowv[low_row(it, wave, rl)];
        uint32_t ev = (zw[it] << 4) & 0xF0F0F0F0u, od = zw[it] & 0xF0F0F0F0u;
        if constexpr (kBits == 6) {
            // the 8 low parts (column e in bits 2e) spread to one nibble per byte: byte j holds
            // column 2j in bits 0..1 and column 2j + 1 in bits 2..3
            uint32_t sp = (zl[it] | (zl[it] << 8)) & 0x00FF00FFu;
            sp = (sp | (sp << 4)) & 0x0F0F0F0Fu;
            ev |= (sp << 2) & 0x0C0C0C0Cu;
            od |= sp & 0x0C0C0C0Cu;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float ze = static_cast<float>(static_cast<int8_t>(ev >> (8 * j)));
            const float zo = static_cast<float>(static_cast<int8_t>(od >> (8 * j)));
            p1[2 * j] = fmaf(ze, rv.x, p1[2 * j]);
            p2[2 * j] = fmaf(ze, rv.y, p2[2 * j]);
            p1[2 * j + 1] = fmaf(zo, rv.x, p1[2 * j + 1]);
            p2[2 * j + 1] = fmaf(zo, rv.y, p2[2 * j + 1]);
        }
    }
    float q1[4], q2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        q1[e] = add_pair16(p1[e], p1[e + 4]);
        q2[e] = add_pair16(p2[e], p2[e + 4]);
    }
    const int b4 = (lane >> 4) & 1, b5 = lane >> 5;
    *reinterpret_cast<f32x4*>(red_w + 8 * c16 + 4 * b4 + 2 * b5) =
        f32x4{add_pair32(q1[0], q1[2]), add_pair32(q2[0], q2[2]), add_pair32(q1[1], q1[3]), add_pair32(q2[1], q2[3])};
}

// With per-key gates (KDA) the records' gates are staged in LDS and each lane forms the
// decay products of its 8 keys as in the 8-bit step; the read vectors take the decay of
// their own row.
template <int kBits, bool kPerKey>
__global__ __launch_bounds__(kThreads) void lq_low_step_kernel(
    int W, int pos, const uint32_t* __restrict__ Z, const float* __restrict__ Bcol, const float* __restrict__ Csm,
    const half_t* __restrict__ Kc, const half_t* __restrict__ Uc, bf16_t* __restrict__ Kbuf,
    float* __restrict__ Ubuf, float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    extern __shared__ __align__(16) float gs_lds[];   // KDA: the records' gates [pos][128]
    __shared__ f32x2 rowv[kD];
    __shared__ f32x2 coef[16];
    using Cfg = LowBits<kBits>;
    constexpr int kT = Cfg::kT, kTh = Cfg::kTh;
    __shared__ f32x2 ctok[kT];
    __shared__ __align__(16) float gtot[kPerKey ? kD : 4];  // KDA: the product of all record gates per key
    __shared__ f32x2 red[4][kD];
    __shared__ f32x2 recp[kD];
    __shared__ float kq_part[2];

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const int grp = tid >> 4, ch = tid & 15;
    const int cc = tid & (kD - 1), half = tid >> 7;
    const bool first = tid < kD;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kT * kD;

    // ---- loads: record keys (group grp) and values (column cc), tokens, inputs, codes
    // (unconditional, so that no branch makes the compiler wait for them: slots and tokens
    // are clamped in bounds; what a clamped lane loads is never used or meets a zero coefficient)
    uint32_t kc[4];
    {  // (at pos 0 the lane's own input keys, loaded anyway)
        const uint4 x = *reinterpret_cast<const uint4*>(
            0 < pos ? Kbuf + rec0 + static_cast<size_t>(grp < pos ? grp : 0) * kD + 8 * ch : k + vec_off + 8 * ch);
        kc[0] = x.x; kc[1] = x.y; kc[2] = x.z; kc[3] = x.w;
    }
    float ucol[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const float ul = Ubuf[rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + cc];  // slot clamped to 0: in bounds, no branch
        ucol[e] = j < pos ? ul : 0.f;
    }
    const uint4 ktw = *reinterpret_cast<const uint4*>(Kc + tok0 + (grp & (kT - 1)) * kD + 8 * ch);
    half_t utv[kTh];
#pragma unroll
    for (int e = 0; e < kTh; ++e) utv[e] = Uc[tok0 + (kTh * half + e) * kD + cc];
    float g_lane = 1.f;  // GDN: lane i holds the gate of record i
    Stager<float, kPerKey ? 16 * kD : 8> sg;
    if constexpr (kPerKey) sg.load(Gbuf + rec0, pos * kD, tid);
    else if (lane < pos) g_lane = Gbuf[static_cast<size_t>(h) * W + lane];
    const uint4 kchw = *reinterpret_cast<const uint4*>(k + vec_off + 8 * ch);
    const uint4 qchw = *reinterpret_cast<const uint4*>(q + vec_off + 8 * ch);
    f32x4 gch_lo = {1.f, 1.f, 1.f, 1.f}, gch_hi = {1.f, 1.f, 1.f, 1.f};  // KDA: current gates of the 8 keys
    if constexpr (kPerKey) {
        gch_lo = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch);
        gch_hi = *reinterpret_cast<const f32x4*>(gate + vec_off + 8 * ch + 4);
    }
    const float kr = load_in(k, vec_off + cc), qr = load_in(q, vec_off + cc);
    const float gr = kPerKey ? gate[vec_off + cc] : gate[h];
    const float cr = Csm[vec_off + cc];
    const float bcc = Bcol[vec_off + cc];
    const float vr = load_in(v, vec_off + cc);
    const float bt = beta[h];
    const uint32_t* Zh = Z + static_cast<size_t>(h) * kD * Cfg::kRowWords;
    uint32_t zw[8], zl[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const uint32_t* zrow = Zh + low_row(it, wave, rl) * Cfg::kRowWords;
        zw[it] = __builtin_nontemporal_load(zrow + c16);
        if constexpr (kBits == 6)  // the low parts: bytes 64 + 2 c16, +1 of the row
            zl[it] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(zrow + 16) + c16);
        else
            zl[it] = 0u;
    }

    // ---- decays (newest gate first): after record grp, and over the whole window so far.
    // Per key (KDA): Ge[e] after record grp and Gt[e] over the window for the lane's 8 keys,
    // Gall for row cc; the current gate comes on top of each.
    float Gg = 1.f, Gall = 1.f;
    float Ge[kPerKey ? 8 : 1], Gt[kPerKey ? 8 : 1];
    if constexpr (!kPerKey) {
        // suffix scan over the record lanes (g = 1 from record pos on): the product of the
        // gates after each record, gathered for this lane's record group
        const float Sfx = suffix_prod<16>(g_lane, lane);
        Gg = lane_gather(suffix_prod_excl<16>(Sfx, lane), grp);
        Gall = lane_value(Sfx, 0);
    } else {
        // the gates' suffix products per key column, in place; the column totals in gtot
        sg.store(gs_lds, tid);
        __syncthreads();
        if (first) {
            Gall = column_suffix_products<16>(gs_lds, pos, cc);
            gtot[cc] = Gall;
        }
        __syncthreads();
        const bool rec = grp < pos;
        const f32x4 lo = rec ? *reinterpret_cast<const f32x4*>(gs_lds + grp * kD + 8 * ch) : f32x4{1.f, 1.f, 1.f, 1.f};
        const f32x4 hi = rec ? *reinterpret_cast<const f32x4*>(gs_lds + grp * kD + 8 * ch + 4) : f32x4{1.f, 1.f, 1.f, 1.f};
        const f32x4 tlo = *reinterpret_cast<const f32x4*>(gtot + 8 * ch);
        const f32x4 thi = *reinterpret_cast<const f32x4*>(gtot + 8 * ch + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Ge[e] = lo[e];
            Ge[e + 4] = hi[e];
            Gt[e] = tlo[e];
            Gt[e + 4] = thi[e];
        }
    }
    auto gcur = [&](int e) { return e < 4 ? gch_lo[e] : gch_hi[e - 4]; };
    const uint32_t kcw[4] = {kchw.x, kchw.y, kchw.z, kchw.w};
    const uint32_t qcw[4] = {qchw.x, qchw.y, qchw.z, qchw.w};
    auto bfe = [](const uint32_t (&w)[4], int e) {
        return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    };
    if (0 < pos) {
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = bfe(kc, e) * (kPerKey ? Ge[e] * gcur(e) : Gg * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < pos) coef[grp] = f32x2{ck, cq};
    }
    if (first) {  // groups 0..kT-1: the tokens, decayed by every gate of the window
        const half_t* kt = reinterpret_cast<const half_t*>(&ktw);
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = static_cast<float>(kt[e]) * (kPerKey ? Gt[e] * gcur(e) : Gall * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < kT) ctok[grp] = f32x2{ck, cq};
        const float c0 = cr * Gall * gr;  // c_r Gamma_{1:l} at row r
        rowv[cc] = f32x2{c0 * kr, c0 * qr} * Cfg::kReadScale;  // see sweep_low
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    }
    __syncthreads();

    // ---- payload sweep over the lane's 8 words; the 4 row lanes, then the waves
    sweep_low<kBits>(zw, zl, rowv, wave, lane, red[wave]);
    // record and token terms of column cc
    f32x2 rp = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        if (j < pos) rp += coef[j] * ucol[e];
    }
#pragma unroll
    for (int e = 0; e < kTh; ++e) rp += ctok[kTh * half + e] * static_cast<float>(utv[e]);
    if (half == 1) recp[cc] = rp;
    __syncthreads();

    if (first) {
        const int c = cc;
        f32x2 acc = (red[0][c] + red[1][c] + red[2][c] + red[3][c]) * (bcc * (1.f / Cfg::kQmax));
        acc += rp + recp[c];
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

// The window's last step at 4 or 6 bits: the step as above, then S_W on the matrix cores as
// in the 8-bit boundary (payload init from the staged codes, the records' two bf16 MFMAs per
// tile, the tokens' fp32 MFMAs, one per 4 tokens), through LDS into the refit's layout, and
// the refit with low-bit codes. One region of dynamic LDS serves the step arrays, the state
// in transit (half of it at a time) and the refit's arrays in turn; after it lie W (the old
// Ut) and the old payload's B / qmax: 47 KB (4 bits) or 40 KB (6 bits) in all.
template <int kBits>
struct LowBitsLds {
    using Cfg = LowBits<kBits>;
    static constexpr int kStep = 2 * kD * 4 + 3 * 2 * kD * 4 + kD * Cfg::kZsStride + 2 * Cfg::kT * kD + 4 * kD * 2 + kD * 2;
    static constexpr int kRefit = TileRefitLds<Cfg::kT, kBits>::kRegionFloats;
    static constexpr int kRegion = kStep > kRefit ? kStep : kRefit;
    static constexpr int kBoundary = kRegion + Cfg::kT * kD + kD;
    static_assert(kRegion % 4 == 0, "W after the region must be 16-byte aligned");
};

template <int kBits>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void lq_low_boundary_kernel(
    int W, int pos, int n_iter, uint32_t* __restrict__ Z, float* __restrict__ Bcol, float* __restrict__ Csm,
    half_t* __restrict__ Kc, half_t* __restrict__ Uc, const bf16_t* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    using Cfg = LowBits<kBits>;
    constexpr int kT = Cfg::kT, kTh = Cfg::kTh, kC = Cfg::kC, kZsStride = Cfg::kZsStride;
    constexpr int kRegion = LowBitsLds<kBits>::kRegion;
    constexpr int kRec = 16;
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ f32x2 rowv[kD];
    __shared__ f32x2 coef[kRec];
    __shared__ f32x2 ctok[kT];
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];
    __shared__ float gam[kRec];

    u32x4* Kt = reinterpret_cast<u32x4*>(dyn_lds);                 // [2][128] keys, 8 records per word
    u32x4* Ut = Kt + 2 * kD;                                        // [3][2][128] scaled values, 3 parts
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Ut + 3 * 2 * kD);   // [128][kZsStride] the old codes
    float* Ktok = reinterpret_cast<float*>(Zs + kD * kZsStride);   // [kT][128]
    float* Utok = Ktok + kT * kD;                                   // [kT][128], scaled by Gamma_{1:W}
    f32x2* red = reinterpret_cast<f32x2*>(Utok + kT * kD);         // [4][128]
    f32x2* recp = red + 4 * kD;                                     // [128]
    const TileRefitLds<kT, kBits> L(dyn_lds, dyn_lds + kRegion);
    float* bscs = dyn_lds + kRegion + kT * kD;                      // B / qmax of the old payload

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const int grp = tid >> 4, ch = tid & 15;
    const int cc = tid & (kD - 1), half = tid >> 7;
    const bool first = tid < kD;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kT * kD;
    uint32_t* Zh = Z + static_cast<size_t>(h) * kD * Cfg::kRowWords;

    // ---- loads
    uint32_t kcr[4] = {0u, 0u, 0u, 0u};
    if (0 < pos) {
        const uint4 x = *reinterpret_cast<const uint4*>(Kbuf + rec0 + static_cast<size_t>(grp < pos ? grp : 0) * kD + 8 * ch);
        kcr[0] = x.x; kcr[1] = x.y; kcr[2] = x.z; kcr[3] = x.w;
    }
    float ucol[8];
    uint32_t kcol[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const size_t at = rec0 + static_cast<size_t>(j < pos ? j : 0) * kD + cc;
        const float ul = Ubuf[at];  // unconditional: at is clamped to slot 0 (in bounds), the value dropped for j >= pos
        const uint32_t kl = static_cast<uint32_t>(Kbuf[at]);
        ucol[e] = j < pos ? ul : 0.f;
        const uint32_t kb = j < pos ? kl : 0u;
        kcol[e >> 1] = (e & 1) ? (kcol[e >> 1] | (kb << 16)) : kb;
    }
    const uint4 ktw = *reinterpret_cast<const uint4*>(Kc + tok0 + (grp & (kT - 1)) * kD + 8 * ch);
    half_t tokv[kT];  // token t at row / column cc (threads < 128: keys; threads >= 128: values)
#pragma unroll
    for (int t = 0; t < kT; ++t) tokv[t] = (first ? Kc : Uc)[tok0 + t * kD + cc];
    const float g_lane = lane < pos ? Gbuf[static_cast<size_t>(h) * W + lane] : 1.f;
    const uint4 kchw = *reinterpret_cast<const uint4*>(k + vec_off + 8 * ch);
    const uint4 qchw = *reinterpret_cast<const uint4*>(q + vec_off + 8 * ch);
    const float kr = load_in(k, vec_off + cc), qr = load_in(q, vec_off + cc);
    const float gr = gate[h];
    const float cr = Csm[vec_off + cc];
    const float bcc = Bcol[vec_off + cc];
    const float vr = load_in(v, vec_off + cc);
    const float bt = beta[h];
    uint32_t zw[8], zl[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const uint32_t* zrow = Zh + low_row(it, wave, rl) * Cfg::kRowWords;
        zw[it] = __builtin_nontemporal_load(zrow + c16);
        if constexpr (kBits == 6)  // the low parts: bytes 64 + 2 c16, +1 of the row
            zl[it] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(zrow + 16) + c16);
        else
            zl[it] = 0u;
    }

    // ---- gate products (newest first): after record grp, after record = lane, all
    // (a suffix scan over the record lanes, g = 1 from record pos on)
    const float Sfx = suffix_prod<16>(g_lane, lane);
    const float Gl = suffix_prod_excl<16>(Sfx, lane);
    const float Gg = lane_gather(Gl, grp), Gall = lane_value(Sfx, 0);
    const float gam_all = Gall * gr;  // Gamma_{1:W}
    if (wave == 0 && lane < kRec) gam[lane] = lane < pos ? Gl * gr : 1.f;
    const uint32_t kcw[4] = {kchw.x, kchw.y, kchw.z, kchw.w};
    const uint32_t qcw[4] = {qchw.x, qchw.y, qchw.z, qchw.w};
    auto bfe = [](const uint32_t (&w)[4], int e) {
        return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    };
    if (0 < pos) {
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = bfe(kcr, e) * (Gg * gr);
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < pos) coef[grp] = f32x2{ck, cq};
    }
    if (first) {
        const half_t* kt = reinterpret_cast<const half_t*>(&ktw);
        float ck = 0.f, cq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ej = static_cast<float>(kt[e]) * gam_all;
            ck += ej * bfe(kcw, e);
            cq += ej * bfe(qcw, e);
        }
        ck = row16_sum(ck);
        cq = row16_sum(cq);
        if (ch == 0 && grp < kT) ctok[grp] = f32x2{ck, cq};
        const float c0 = cr * gam_all;
        rowv[cc] = f32x2{c0 * kr, c0 * qr} * Cfg::kReadScale;  // see sweep_low
        zcoef[cc] = c0;
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    } else {
        bscs[cc] = bcc * (1.f / Cfg::kQmax);
    }
    // token operands of the contraction, and the unscaled values as the refit's start
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        const float x = static_cast<float>(tokv[t]);
        if (first) Ktok[t * kD + cc] = x;
        else Utok[t * kD + cc] = x * gam_all;
    }
    if (!first)
#pragma unroll
        for (int hh = 0; hh < kC; ++hh)
            L.W[cc * kC + hh] = f32x4{static_cast<float>(tokv[4 * hh]), static_cast<float>(tokv[4 * hh + 1]),
                                     static_cast<float>(tokv[4 * hh + 2]), static_cast<float>(tokv[4 * hh + 3])};
    Kt[half * kD + cc] = u32x4{kcol[0], kcol[1], kcol[2], kcol[3]};
    __syncthreads();

    // ---- payload sweep; record and token terms per column; scaled records staged for the MFMA
    sweep_low<kBits>(zw, zl, rowv, wave, lane, red + wave * kD);
    f32x2 rp = {0.f, 0.f};
    u32x4 part[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * half + e;
        const f32x2 c = j < pos ? coef[j] : f32x2{0.f, 0.f};
        rp += c * ucol[e];
        uint32_t hi, mid, lo;
        split3_bf16(gam[j] * ucol[e], hi, mid, lo);
        const int sh = 16 * (e & 1);
        part[0][e >> 1] = (e & 1) ? (part[0][e >> 1] | (hi << sh)) : hi;
        part[1][e >> 1] = (e & 1) ? (part[1][e >> 1] | (mid << sh)) : mid;
        part[2][e >> 1] = (e & 1) ? (part[2][e >> 1] | (lo << sh)) : lo;
    }
#pragma unroll
    for (int e = 0; e < kTh; ++e) {  // tokens kTh half .. +kTh-1 of column cc (L.W holds their unscaled values)
        const int t = kTh * half + e;
        rp += ctok[t] * L.W[cc * kC + (t >> 2)][t & 3];
    }
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) Ut[(pp * 2 + half) * kD + cc] = part[pp];
    if (half == 1) recp[cc] = rp;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        uint32_t* zs_row = Zs + low_row(it, wave, rl) * kZsStride;
        zs_row[c16] = zw[it];
        if constexpr (kBits == 6) reinterpret_cast<uint16_t*>(zs_row + 16)[c16] = static_cast<uint16_t>(zl[it]);
    }
    __syncthreads();

    // ---- correction and output; the current record joins the contraction operands
    if (first) {
        const int c = cc;
        f32x2 acc = (red[c] + red[kD + c] + red[2 * kD + c] + red[3 * kD + c]) * bscs[c];
        acc += rp + recp[c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        uint32_t uh, um, ul;
        split3_bf16(u, uh, um, ul);
        reinterpret_cast<uint16_t*>(&Ut[(0 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(uh);
        reinterpret_cast<uint16_t*>(&Ut[(1 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(um);
        reinterpret_cast<uint16_t*>(&Ut[(2 * 2 + (pos >> 3)) * kD + c])[pos & 7] = static_cast<uint16_t>(ul);
        reinterpret_cast<uint16_t*>(&Kt[(pos >> 3) * kD + c])[pos & 7] = static_cast<uint16_t>(__float_as_uint(kr) >> 16);
    }
    __syncthreads();

    // ---- S_W on the matrix cores (result layout of v_mfma_f32_16x16x{32_bf16,4f32}: lane l
    // holds key row 32w + 16a + l%16 and value columns 16ct + 4(l/16) .. +3 of tile ct)
    const int lr = lane & 15, lq = lane >> 4, blk = lq & 1;
    f32x4 acc[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, Kt[blk * kD + row]);
        const float zc = zcoef[row];
        const float bk0 = Ktok[lq * kD + row], bk1 = kT == 8 ? Ktok[(4 + lq) * kD + row] : 0.f;
        const uint16_t* z16 = reinterpret_cast<const uint16_t*>(Zs + row * kZsStride);
        const uint8_t* z8lo = reinterpret_cast<const uint8_t*>(Zs + row * kZsStride + 16);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 bs = *reinterpret_cast<const f32x4*>(bscs + 16 * ct + 4 * lq);
            const uint32_t zz = z16[4 * ct + lq];  // the 4 nibbles of columns 16ct + 4lq .. +3
            f32x4 zf;
            if constexpr (kBits == 4) {
                zf = f32x4{static_cast<float>(static_cast<int>(zz << 28) >> 28),
                           static_cast<float>(static_cast<int>(zz << 24) >> 28),
                           static_cast<float>(static_cast<int>(zz << 20) >> 28),
                           static_cast<float>(static_cast<int>(zz << 16) >> 28)};
            } else {  // 4 (z >> 2) + (z & 3), the low parts of the same 4 columns in one byte
                const uint32_t zb = z8lo[4 * ct + lq];
                zf = f32x4{static_cast<float>(4 * (static_cast<int>(zz << 28) >> 28) + static_cast<int>(zb & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 24) >> 28) + static_cast<int>((zb >> 2) & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 20) >> 28) + static_cast<int>((zb >> 4) & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 16) >> 28) + static_cast<int>(zb >> 6))};
            }
            acc[a][ct] = zf * (bs * zc);
            const int col = 16 * ct + lr;
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, Ut[((lq < 2 ? 0 : 1) * 2 + blk) * kD + col]);
            const u32x4 lo = Ut[(2 * 2 + blk) * kD + col];
            const bf16x8 a2 = __builtin_bit_cast(bf16x8, lq < 2 ? lo : u32x4{0u, 0u, 0u, 0u});
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv, acc[a][ct], 0, 0, 0);
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, bv, acc[a][ct], 0, 0, 0);
            acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(Utok[lq * kD + col], bk0, acc[a][ct], 0, 0, 0);
            if constexpr (kT == 8)
                acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(Utok[(4 + lq) * kD + col], bk1, acc[a][ct], 0, 0, 0);
        }
    }
    __syncthreads();  // every read of the step-phase arrays is done: the region is the refit's
    lq_refit_tiles(L, acc, n_iter, tid, Zh, Bcol + vec_off, Csm + vec_off, Kc + tok0, Uc + tok0);
}

// ---------------------------------------------------------------- 4 and 6 bits, per-key gates
// KDA's boundary at low bit widths: the step as in the 8-bit KDA boundary (records, their
// gates and keys staged in LDS as fp32, the decayed keys formed by one thread per key row
// walking the records backwards) with the low-bit payload sweep; the record and token terms
// are added per value column after the sweep. S_W forms on the matrix cores in fp32 in the
// 8-bit KDA boundary's operand layout (the payload init decodes the staged low-bit codes of
// columns 32 (l / 16) + 8 i + ct), passes through LDS into the refit's layout and is refitted
// with low-bit codes. W (the refit's start) lies after the refit's arrays and the half state
// in transit, inside the step arrays (written once they are dead); B / qmax of the old
// payload follows both.
template <int kBits>
struct LowKdaLds {
    using Cfg = LowBits<kBits>;
    static constexpr int kStep = 3 * kKdaRec * kD + kD * Cfg::kZsStride + 2 * Cfg::kT * kD + 4 * kD * 2;
    static constexpr int kW = TileRefitLds<Cfg::kT, kBits>::kRegionFloats;
    static constexpr int kBscs = kStep > kW + Cfg::kT * kD ? kStep : kW + Cfg::kT * kD;
    static constexpr int kTotal = kBscs + kD;
    static_assert(kW % 4 == 0 && (3 * kKdaRec * kD + kD * Cfg::kZsStride + 2 * Cfg::kT * kD) % 2 == 0,
                  "W must be 16-byte and red 8-byte aligned");
};

template <int kBits>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void lq_low_boundary_kda_kernel(
    int W, int pos, int n_iter, uint32_t* __restrict__ Z, float* __restrict__ Bcol, float* __restrict__ Csm,
    half_t* __restrict__ Kc, half_t* __restrict__ Uc, const bf16_t* __restrict__ Kbuf,
    const float* __restrict__ Ubuf, const float* __restrict__ Gbuf, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ y) {
    using Cfg = LowBits<kBits>;
    using Lds = LowKdaLds<kBits>;
    constexpr int kT = Cfg::kT, kC = Cfg::kC, kZsStride = Cfg::kZsStride;
    extern __shared__ __align__(16) float dyn_lds[];
    __shared__ f32x2 rowv[kD];       // c_r Gamma_{1:W,r} (k_r, q_r) kReadScale
    __shared__ f32x2 kq_row[kD];     // (k_r, q_r)
    __shared__ f32x2 coef[kKdaRec];  // per record (E_j . k, E_j . q)
    __shared__ f32x2 ctok[kT];       // per token ((Gamma Kt_t) . k, (Gamma Kt_t) . q)
    __shared__ float kq_part[2];
    __shared__ float zcoef[kD];      // c_r Gamma_{1:W,r}

    float* KE = dyn_lds;                                            // [16][128]
    float* Us = KE + kKdaRec * kD;                                  // [16][128]
    float* Gs = Us + kKdaRec * kD;                                  // [16][128]
    uint32_t* Zs = reinterpret_cast<uint32_t*>(Gs + kKdaRec * kD);  // [128][kZsStride]
    float* Ktk = reinterpret_cast<float*>(Zs + kD * kZsStride);    // [kT][128] Gamma_{1:W} Kt
    float* Utk = Ktk + kT * kD;                                     // [kT][128] Ut
    f32x2* red = reinterpret_cast<f32x2*>(Utk + kT * kD);          // [4][128]
    const TileRefitLds<kT, kBits> L(dyn_lds, dyn_lds + Lds::kW);
    float* bscs = dyn_lds + Lds::kBscs;                             // B / qmax of the old payload

    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const int r = tid & (kD - 1);
    const bool first = tid < kD;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    const size_t rec0 = static_cast<size_t>(h) * W * kD;
    const size_t tok0 = static_cast<size_t>(h) * kT * kD;
    uint32_t* Zh = Z + static_cast<size_t>(h) * kD * Cfg::kRowWords;

    // ---- loads: records, gates, tokens and inputs first, then the codes
    Stager<bf16_t, kKdaRec * kD> sk;
    Stager<float, kKdaRec * kD> su;
    Stager<float, kKdaRec * kD> sg;
    sk.load(Kbuf + rec0, pos * kD, tid);
    su.load(Ubuf + rec0, pos * kD, tid);
    sg.load(Gbuf + rec0, pos * kD, tid);
    half_t tokv[kT];  // token t at row / column r (threads < 128: keys; threads >= 128: values)
#pragma unroll
    for (int t = 0; t < kT; ++t) tokv[t] = (first ? Kc : Uc)[tok0 + t * kD + r];
    const float kr = load_in(k, vec_off + r), qr = load_in(q, vec_off + r);
    const float gr = gate[vec_off + r];
    const float cr = Csm[vec_off + r];
    const float bcc = Bcol[vec_off + r];
    const float vr = load_in(v, vec_off + r);
    const float bt = beta[h];
    uint32_t zw[8], zl[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const uint32_t* zrow = Zh + low_row(it, wave, rl) * Cfg::kRowWords;
        zw[it] = __builtin_nontemporal_load(zrow + c16);
        if constexpr (kBits == 6)
            zl[it] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(zrow + 16) + c16);
        else
            zl[it] = 0u;
    }

    sk.store(KE, tid);
    su.store(Us, tid);
    sg.store(Gs, tid);
    for (int i = pos * kD + tid; i < kKdaRec * kD; i += kThreads) Us[i] = 0.f;  // rows pos .. 15
    __syncthreads();

    // ---- decayed keys in place (thread r < 128 walks key row r from the newest record),
    // read vectors, token keys with the whole window's decay; token values from threads >= 128
    if (first) {
        float G = 1.f;
        for (int j = pos - 1; j >= 0; --j) {
            KE[j * kD + r] *= G * gr;
            G *= Gs[j * kD + r];
        }
        const float gam = G * gr;  // Gamma_{1:W} at row r
        const float c0 = cr * gam;
        rowv[r] = f32x2{c0 * kr, c0 * qr} * Cfg::kReadScale;  // see sweep_low
        kq_row[r] = f32x2{kr, qr};
        zcoef[r] = c0;
        KE[pos * kD + r] = kr;  // the current record: no decay after it
        for (int j = pos + 1; j < kKdaRec; ++j) KE[j * kD + r] = 0.f;
#pragma unroll
        for (int t = 0; t < kT; ++t) Ktk[t * kD + r] = static_cast<float>(tokv[t]) * gam;
        const float kq = wave_sum(kr * qr);
        if (lane == 0) kq_part[wave] = kq;
    } else {
#pragma unroll
        for (int t = 0; t < kT; ++t) Utk[t * kD + r] = static_cast<float>(tokv[t]);
        bscs[r] = bcc * (1.f / Cfg::kQmax);
    }
    __syncthreads();

    // ---- record and token coefficients: the 16 lanes of a DPP row reduce one (8 rows each)
    {
        const int chunk = tid & 15, j = tid >> 4;
        auto dot8 = [&](const float* e) {
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(e + 8 * chunk);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(e + 8 * chunk + 4);
            const f32x2* kqr = kq_row + 8 * chunk;
            f32x2 c = e0.x * kqr[0] + e0.y * kqr[1] + e0.z * kqr[2] + e0.w * kqr[3] + e1.x * kqr[4] +
                      e1.y * kqr[5] + e1.z * kqr[6] + e1.w * kqr[7];
            return f32x2{row16_sum(c.x), row16_sum(c.y)};
        };
        const f32x2 c = dot8(KE + (j < pos ? j : 0) * kD);
        if (chunk == 0 && j < pos) coef[j] = c;
        if (j < kT) {  // the first kT groups again (whole waves): the tokens
            const f32x2 ct = dot8(Ktk + j * kD);
            if (chunk == 0) ctok[j] = ct;
        }
    }
    __syncthreads();

    // ---- payload sweep; the codes staged for the payload init
    sweep_low<kBits>(zw, zl, rowv, wave, lane, red + wave * kD);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        uint32_t* zs_row = Zs + low_row(it, wave, rl) * kZsStride;
        zs_row[c16] = zw[it];
        if constexpr (kBits == 6) reinterpret_cast<uint16_t*>(zs_row + 16)[c16] = static_cast<uint16_t>(zl[it]);
    }
    __syncthreads();

    // ---- correction and output with the record and token terms of column c; u of this step
    // becomes row pos of Us
    if (first) {
        const int c = tid;
        f32x2 acc = (red[c] + red[kD + c] + red[2 * kD + c] + red[3 * kD + c]) * bscs[c];
        for (int j = 0; j < pos; ++j) acc += coef[j] * Us[j * kD + c];
#pragma unroll
        for (int t = 0; t < kT; ++t) acc += ctok[t] * Utk[t * kD + c];
        const float kq = kq_part[0] + kq_part[1];
        const float u = bt * (vr - acc.x);
        y[vec_off + c] = acc.y + u * kq;
        Us[pos * kD + c] = u;
    }
    __syncthreads();

    // ---- S_W on the matrix cores in the tile layout (A: the records' and tokens' values of
    // columns 16ct + m; B: their decayed keys of rows 16(2w + a) + n), both bands in registers
    const int lr = lane & 15, lq = lane >> 4;
    f32x4 acc[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int row = 16 * (2 * wave + a) + lr;
        const float zc = zcoef[row];
        const uint16_t* z16 = reinterpret_cast<const uint16_t*>(Zs + row * kZsStride);
        const uint8_t* z8lo = reinterpret_cast<const uint8_t*>(Zs + row * kZsStride + 16);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {  // the 4 codes of columns 16ct + 4lq .. +3
            const f32x4 bs = *reinterpret_cast<const f32x4*>(bscs + 16 * ct + 4 * lq);
            const uint32_t zz = z16[4 * ct + lq];
            f32x4 zf;
            if constexpr (kBits == 4) {
                zf = f32x4{static_cast<float>(static_cast<int>(zz << 28) >> 28),
                           static_cast<float>(static_cast<int>(zz << 24) >> 28),
                           static_cast<float>(static_cast<int>(zz << 20) >> 28),
                           static_cast<float>(static_cast<int>(zz << 16) >> 28)};
            } else {
                const uint32_t zb = z8lo[4 * ct + lq];
                zf = f32x4{static_cast<float>(4 * (static_cast<int>(zz << 28) >> 28) + static_cast<int>(zb & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 24) >> 28) + static_cast<int>((zb >> 2) & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 20) >> 28) + static_cast<int>((zb >> 4) & 3u)),
                           static_cast<float>(4 * (static_cast<int>(zz << 16) >> 28) + static_cast<int>(zb >> 6))};
            }
            acc[a][ct] = zf * (bs * zc);
        }
    }
#pragma unroll
    for (int s4 = 0; s4 < kKdaRec / 4; ++s4) {
        const float eb0 = KE[(4 * s4 + lq) * kD + 32 * wave + lr], eb1 = KE[(4 * s4 + lq) * kD + 32 * wave + 16 + lr];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float ua = Us[(4 * s4 + lq) * kD + 16 * ct + lr];
            acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua, eb0, acc[0][ct], 0, 0, 0);
            acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua, eb1, acc[1][ct], 0, 0, 0);
        }
    }
#pragma unroll
    for (int g = 0; g < kC; ++g) {
        const float kb0 = Ktk[(4 * g + lq) * kD + 32 * wave + lr], kb1 = Ktk[(4 * g + lq) * kD + 32 * wave + 16 + lr];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float ut = Utk[(4 * g + lq) * kD + 16 * ct + lr];
            acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ut, kb0, acc[0][ct], 0, 0, 0);
            acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ut, kb1, acc[1][ct], 0, 0, 0);
        }
    }
    __syncthreads();  // every read of the step-phase arrays is done: the region is the refit's, and W
    if (!first)
#pragma unroll
        for (int hh = 0; hh < kC; ++hh)
            L.W[r * kC + hh] = f32x4{static_cast<float>(tokv[4 * hh]), static_cast<float>(tokv[4 * hh + 1]),
                                     static_cast<float>(tokv[4 * hh + 2]), static_cast<float>(tokv[4 * hh + 3])};
    __syncthreads();
    lq_refit_tiles(L, acc, n_iter, tid, Zh, Bcol + vec_off, Csm + vec_off, Kc + tok0, Uc + tok0);
}

// ---------------------------------------------------------------- launchers
static hipError_t set_lds(const void* fn, int floats) {
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(sizeof(float) * floats));
}

hipError_t launch_lq_quantize(int heads, const float* S, int n_iter, int8_t* Z, float* B, float* C,
                              void* Kc, void* Uc, hipStream_t stream) {
    using L_t = TileRefitLds<4, 8>;
    constexpr int floats = L_t::kRegionFloats + L_t::kWFloats;
    static const hipError_t attr = set_lds(reinterpret_cast<const void*>(lq_quantize_kernel<4, 8>), floats);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((lq_quantize_kernel<4, 8>), dim3(heads), dim3(kThreads), sizeof(float) * floats, stream,
                       S, n_iter, reinterpret_cast<uint32_t*>(Z), B, C, static_cast<half_t*>(Kc),
                       static_cast<half_t*>(Uc));
    return hipGetLastError();
}

hipError_t launch_lq_window(const StepArgs& a, const LqArgs& w, bool per_key, hipStream_t stream) {
    if (w.pos == w.W - 1) {
        static const hipError_t attr_gdn = set_lds(reinterpret_cast<const void*>(lq_boundary_kernel), kLqBoundaryFloats);
        static const hipError_t attr_kda = set_lds(reinterpret_cast<const void*>(lq_boundary_kda_kernel), kLqKdaBoundaryFloats);
        if (hipError_t e = per_key ? attr_kda : attr_gdn) return e;
        if (per_key)
            hipLaunchKernelGGL(lq_boundary_kda_kernel, dim3(a.heads), dim3(kThreads), sizeof(float) * kLqKdaBoundaryFloats,
                               stream, w.W, w.pos, w.n_iter, w.Z, w.B, w.C, static_cast<half_t*>(w.Kc),
                               static_cast<half_t*>(w.Uc), static_cast<const bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf,
                               static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                               static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
        else
            hipLaunchKernelGGL(lq_boundary_kernel, dim3(a.heads), dim3(kThreads), sizeof(float) * kLqBoundaryFloats,
                               stream, w.W, w.pos, w.n_iter, w.Z, w.B, w.C, static_cast<half_t*>(w.Kc),
                               static_cast<half_t*>(w.Uc), static_cast<const bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf,
                               static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                               static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
        return hipGetLastError();
    }
    if (per_key)
        hipLaunchKernelGGL(lq_step_kernel<true>, dim3(a.heads), dim3(kThreads), sizeof(float) * w.pos * kD, stream,
                           w.W, w.pos, w.Z, w.B, w.C, static_cast<const half_t*>(w.Kc),
                           static_cast<const half_t*>(w.Uc), static_cast<bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf,
                           static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                           static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
    else
        hipLaunchKernelGGL(lq_step_kernel<false>, dim3(a.heads), dim3(kThreads), 0, stream, w.W, w.pos, w.Z, w.B,
                           w.C, static_cast<const half_t*>(w.Kc), static_cast<const half_t*>(w.Uc),
                           static_cast<bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf, static_cast<const bf16_t*>(a.q),
                           static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

template <int kBits>
static hipError_t launch_low_quantize(int heads, const float* S, int n_iter, void* Z, float* B, float* C, void* Kc,
                                      void* Uc, hipStream_t stream) {
    constexpr int kT = LowBits<kBits>::kT;
    using L_t = TileRefitLds<kT, kBits>;
    constexpr int floats = L_t::kRegionFloats + L_t::kWFloats;
    static const hipError_t attr = set_lds(reinterpret_cast<const void*>(lq_quantize_kernel<kT, kBits>), floats);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((lq_quantize_kernel<kT, kBits>), dim3(heads), dim3(kThreads), sizeof(float) * floats, stream,
                       S, n_iter, static_cast<uint32_t*>(Z), B, C, static_cast<half_t*>(Kc),
                       static_cast<half_t*>(Uc));
    return hipGetLastError();
}

template <int kBits, bool kPerKey>
static hipError_t launch_low_window(const StepArgs& a, const LqArgs& w, hipStream_t stream) {
    if (w.pos == w.W - 1) {
        constexpr auto kernel = kPerKey ? lq_low_boundary_kda_kernel<kBits> : lq_low_boundary_kernel<kBits>;
        constexpr int floats = kPerKey ? LowKdaLds<kBits>::kTotal : LowBitsLds<kBits>::kBoundary;
        static const hipError_t attr = set_lds(reinterpret_cast<const void*>(kernel), floats);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(kernel, dim3(a.heads), dim3(kThreads), sizeof(float) * floats,
                           stream, w.W, w.pos, w.n_iter, reinterpret_cast<uint32_t*>(w.Z), w.B, w.C,
                           static_cast<half_t*>(w.Kc), static_cast<half_t*>(w.Uc),
                           static_cast<const bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf, static_cast<const bf16_t*>(a.q),
                           static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((lq_low_step_kernel<kBits, kPerKey>), dim3(a.heads), dim3(kThreads),
                       kPerKey ? sizeof(float) * w.pos * kD : 0, stream, w.W, w.pos,
                       reinterpret_cast<const uint32_t*>(w.Z), w.B, w.C, static_cast<const half_t*>(w.Kc),
                       static_cast<const half_t*>(w.Uc), static_cast<bf16_t*>(w.Kbuf), w.Ubuf, w.Gbuf,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.gate, a.beta, a.y);
    return hipGetLastError();
}

hipError_t launch_lq_low_quantize(int bits, int heads, const float* S, int n_iter, void* Z, float* B, float* C,
                                  void* Kc, void* Uc, hipStream_t stream) {
    return bits == 4 ? launch_low_quantize<4>(heads, S, n_iter, Z, B, C, Kc, Uc, stream)
                     : launch_low_quantize<6>(heads, S, n_iter, Z, B, C, Kc, Uc, stream);
}

hipError_t launch_lq_low_window(int bits, const StepArgs& a, const LqArgs& w, bool per_key, hipStream_t stream) {
    if (per_key) return bits == 4 ? launch_low_window<4, true>(a, w, stream) : launch_low_window<6, true>(a, w, stream);
    return bits == 4 ? launch_low_window<4, false>(a, w, stream) : launch_low_window<6, false>(a, w, stream);
}

}  // namespace rsu
