// stepq.hip -- the per-step packed state of the STEPQuant notes (the key-row-aware dual-axis
// fit): element (i, j) of a head's 128 x 128 state is r_i c_j z_ij, with fp16 key-row factors
// r_i, fp16 value-column factors c_j and 4-bit codes z_ij (two per byte, the even value column
// in the low nibble), and the state is packed again after every decode step.
//
// The packing of a state X (one workgroup per head):
//   w_i = omega_i^(1/8) / (their geometric mean over the head's rows)   (row influence weights;
//         the compression exponent 0.25 applied to the RMS read weight sqrt(omega_i))
//   r_i = fp16(sqrt(m_i / w_i)),  m_i = mean_j |X_ij|                   (0 for a zero row)
//   a_j = max_i |X_ij / r_i|,  z_ij = rne(X_ij / r_i * 7 / a_j) in [-7, 7]    (0 if a_j = 0)
//   c_j = fp16(sum_i w_i^2 r_i z_ij X_ij / sum_i w_i^2 r_i^2 z_ij^2)    (weighted least squares)
// and a decode step decodes X_{t-1}, applies the dense update (decayed delta read, rank-one
// write, y = X_t^T q from the updated state) and packs X_t, all in registers: the packed state
// is read once and written once per step. The same kernel also runs the step as two launches,
// the readout and then the repack, for callers that hide the repack on a second stream.
//
// Thread layout (as in the 4-bit LeapQuant sweep): lane l of wave w owns the code word of
// value columns 8(l & 15) .. +7 in the key rows 16 it + 4 w + (l >> 4), it = 0..7, and keeps
// those 64 elements of X in registers. Row sums run over the 16 lanes of a DPP row; column
// sums over the 4 row lanes (two lane swaps) and then the 4 waves through LDS.
#include <type_traits>

#include "kernels.hpp"
#include "rsu_device.hpp"
#include "codes.hpp"
#include "swaps.hpp"

namespace rsu {

typedef _Float16 half_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr float kSqQmax = 7.f;

__device__ __forceinline__ int sq_row(int it, int wave, int rl) { return 16 * it + 4 * wave + rl; }

// Workgroup-shared arrays of the packing.
struct SqLds {
    float iw[kD];         // 1 / w_i
    float wsq[kD];        // w_i^2
    float ir[kD];         // 1 / r_i, 0 for a zero row
    float wrr[kD];        // w_i^2 r_i^2
    float sc[kD];         // 7 / a_j, 0 for a zero column
    half_t rh[kD];        // r_i, stored coalesced after the row phase
    f32x2 red[4][kD];     // per-wave column partials
};

// Row influence weights from omega [128]: threads < 128 write 1 / w_i and w_i^2 of row tid into
// L, with w_i = omega_i^(1/8) / (their geometric mean) = 2^(l_i - mean(l)), l_i = log2(omega_i) / 8.
// Each of the two waves reads all 128 scores, so the mean needs no exchange between waves; the
// caller's next barrier publishes the weights.
__device__ __forceinline__ void sq_row_weights(SqLds& L, const float* __restrict__ omega_h, int tid) {
    if (tid < kD) {
        const int lane = tid & 63;
        const float l0 = __log2f(omega_h[lane]) * 0.125f, l1 = __log2f(omega_h[lane + 64]) * 0.125f;
        const float mean = wave_sum(l0 + l1) * (1.f / kD);
        const float d = (tid < 64 ? l0 : l1) - mean;  // log2 w_i
        L.iw[tid] = exp2f(-d);
        L.wsq[tid] = exp2f(2.f * d);
    }
}

// Three bf16 parts of an fp32 value (hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid);
// both differences are exact in fp32): hi + mid + lo equals x to about 2^-24 |x|.
__device__ __forceinline__ void sq_split3(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    const __bf16 h = static_cast<__bf16>(x);
    const float r1 = x - static_cast<float>(h);
    const __bf16 m = static_cast<__bf16>(r1);
    const __bf16 l = static_cast<__bf16>(r1 - static_cast<float>(m));
    hi = __builtin_bit_cast(uint16_t, h);
    mid = __builtin_bit_cast(uint16_t, m);
    lo = __builtin_bit_cast(uint16_t, l);
}

// c ? x : y as one bitfield insert on the values' bits.
__device__ __forceinline__ float bit_select(int c, float x, float y) {
    const uint32_t m = c ? 0xffffffffu : 0u;
    return __uint_as_float((__float_as_uint(x) & m) | (__float_as_uint(y) & ~m));
}

// 1.5 * 2^23: adding it rounds to an integer (half to even); for integers in [-7, 7] the low
// byte of the sum's bits is that integer's two's complement
constexpr float kRne = 12582912.0f;

// Packs the lane's 64 elements x (rows sq_row(it, wave, l >> 4), columns 8 (l & 15) + e):
// row factors, column ranges, codes (stored), weighted least squares column factors.
// Overwrites x with u = x / r. L.iw and L.wsq must hold the row weights (published by a barrier).
// Every thread calls it.
__device__ __forceinline__ void sq_pack(SqLds& L, float (&x)[8][8], int tid, uint32_t* __restrict__ Zh,
                                        half_t* __restrict__ Rh, half_t* __restrict__ Ch) {
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const int b4 = (lane >> 4) & 1, b5 = lane >> 5;

    // ---- r_i from the row means: the 16 lanes of a DPP row hold the lane's 8 key rows; lane
    // c16 then takes row c16 & 7 (lanes 8..15 repeat it)
    {
        float a[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += fabsf(x[it][e]);
            a[it] = row16_sum(t);
        }
        // a[c16 & 7] by three rounds of bitwise selects (written as selects, the compiler turns
        // them into an index into a private array, which lives in scratch memory)
        float s1[4], s2[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) s1[j] = bit_select(c16 & 1, a[2 * j + 1], a[2 * j]);
#pragma unroll
        for (int j = 0; j < 2; ++j) s2[j] = bit_select(c16 & 2, s1[2 * j + 1], s1[2 * j]);
        const float sum = bit_select(c16 & 4, s2[1], s2[0]);
        const int row = sq_row(c16 & 7, wave, rl);
        const half_t rh = static_cast<half_t>(sqrtf(sum * (1.f / kD) * L.iw[row]));
        const float r = static_cast<float>(rh);
        if (c16 < 8) {
            L.ir[row] = r > 0.f ? 1.f / r : 0.f;
            L.wrr[row] = L.wsq[row] * r * r;
            L.rh[row] = rh;
        }
    }
    __syncthreads();
    if (tid < kD) Rh[tid] = L.rh[tid];

    // ---- u = x / r in place, and the column ranges a_j = max_i |u_ij|: the lane's 8 rows, its
    // 4 row lanes, the 4 waves
    {
        float m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = 0.f;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const float ir = L.ir[sq_row(it, wave, rl)];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[it][e] *= ir;
                m[e] = fmaxf(m[e], fabsf(x[it][e]));
            }
        }
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = max_pair16(m[e], m[e + 4]);      // column e + 4 b4
        const float m0 = max_pair32(q[0], q[2]), m1 = max_pair32(q[1], q[3]);  // columns + 2 b5, + 1
        float* redf = reinterpret_cast<float*>(L.red);
        *reinterpret_cast<f32x2*>(redf + wave * kD + 8 * c16 + 4 * b4 + 2 * b5) = f32x2{m0, m1};
    }
    __syncthreads();
    if (tid < kD) {
        const float* redf = reinterpret_cast<const float*>(L.red);
        const float a = fmaxf(fmaxf(redf[tid], redf[kD + tid]), fmaxf(redf[2 * kD + tid], redf[3 * kD + tid]));
        // capped so that |u| s stays below 7.5 even where 7 / a overflows (a subnormal range):
        // every code then rounds into [-7, 7] with no clamp
        L.sc[tid] = a > 0.f ? fminf(__fdiv_rn(kSqQmax, a), 3.402823466e38f) : 0.f;
    }
    __syncthreads();

    // ---- codes (stored), and the least-squares sums of the lane's columns. With u = x / r,
    // sum_i w^2 r z x = sum_i (w^2 r^2) z u.
    float s[8];
    {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(L.sc + 8 * c16);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(L.sc + 8 * c16 + 4);
        s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
        s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    }
    float num[8], den[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = den[e] = 0.f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = sq_row(it, wave, rl);
        const float W = L.wrr[row];
        uint32_t bits[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // the code rne(u s) from the exact product (one rounding); |u| <= a_j and s_j is
            // 7 / a_j rounded, so |u s| <= 7 (1 + 2^-23) and the code lies in [-7, 7]
            const float f = __builtin_fmaf(x[it][e], s[e], kRne);
            bits[e] = static_cast<uint32_t>(__float_as_int(f));
            const float z = f - kRne;
            const float t = W * z;
            num[e] = fmaf(t, x[it][e], num[e]);
            den[e] = fmaf(t, z, den[e]);
        }
        // low bytes hold the codes' two's complement; nibbles of the even columns from E, the
        // odd ones from O shifted into the high nibbles
        const uint32_t E = pack_low_bytes(bits[0], bits[2], bits[4], bits[6]);
        const uint32_t O = pack_low_bytes(bits[1], bits[3], bits[5], bits[7]);
        Zh[row * (kD / 8) + c16] = (E & 0x0F0F0F0Fu) | ((O << 4) & 0xF0F0F0F0u);
    }
    {
        float qn[4], qd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qn[e] = add_pair16(num[e], num[e + 4]);
            qd[e] = add_pair16(den[e], den[e + 4]);
        }
        *reinterpret_cast<f32x4*>(L.red[wave] + 8 * c16 + 4 * b4 + 2 * b5) =
            f32x4{add_pair32(qn[0], qn[2]), add_pair32(qd[0], qd[2]), add_pair32(qn[1], qn[3]),
                  add_pair32(qd[1], qd[3])};
    }
    __syncthreads();
    if (tid < kD) {
        const f32x2 t = (L.red[0][tid] + L.red[1][tid]) + (L.red[2][tid] + L.red[3][tid]);
        Ch[tid] = static_cast<half_t>(t.y > 0.f ? t.x / t.y : 0.f);
    }
}

// ---- a plain fp32 state [heads, 128, 128] into the packed format
__global__ __launch_bounds__(kThreads) void sq_pack_kernel(const float* __restrict__ S,
                                                           const float* __restrict__ omega,
                                                           uint32_t* __restrict__ Z, half_t* __restrict__ R,
                                                           half_t* __restrict__ C) {
    __shared__ SqLds L;
    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const float* Sh = S + static_cast<size_t>(h) * kD * kD;
    float x[8][8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const float* src = Sh + sq_row(it, wave, rl) * kD + 8 * c16;
        const f32x4 a = stream_load(src), b = stream_load(src + 4);
        x[it][0] = a.x; x[it][1] = a.y; x[it][2] = a.z; x[it][3] = a.w;
        x[it][4] = b.x; x[it][5] = b.y; x[it][6] = b.z; x[it][7] = b.w;
    }
    sq_row_weights(L, omega + static_cast<size_t>(h) * kD, tid);
    __syncthreads();
    sq_pack(L, x, tid, Z + static_cast<size_t>(h) * kD * (kD / 8), R + static_cast<size_t>(h) * kD,
            C + static_cast<size_t>(h) * kD);
}

// ---- one decode step on the packed state, in place (kMode = kSqFused), or the same step in two
// launches: the readout (decode, both column sums, u and y; the packed state is only read) and the
// repack (decode again, X_t = Diag(g) X_{t-1} + k u^T, pack), which a caller may run on a second
// stream behind other work. The two launches repeat the fused step's arithmetic operation for
// operation, so their y, u and packed state equal the fused step's bit for bit.
constexpr int kSqFused = 0, kSqReadout = 1, kSqRepack = 2;

template <int kMode, bool kPerKey, typename T>
__global__ __launch_bounds__(kThreads) void sq_step_kernel(uint32_t* __restrict__ Z, half_t* __restrict__ R,
                                                           half_t* __restrict__ C, const float* __restrict__ omega,
                                                           const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ gate,
                                                           const float* __restrict__ beta, float* __restrict__ u_io,
                                                           float* __restrict__ y) {
    constexpr bool kRead = kMode != kSqRepack, kPack = kMode != kSqReadout;
    __shared__ SqLds L;
    __shared__ f32x2 rowv[kD];   // (r g, k) of key row i
    __shared__ float ucol[kD];   // u_j
    __shared__ float kq_part[2];
    // The column sums p = X^T (g k) and o = X^T (g q) run on the matrix cores: per value column
    // e of a lane, one v_mfma_f32_16x16x32_bf16 with B = the lane's 8 codes of that column (as
    // 16 z, exact in bf16; k = 8 rl + it indexes the wave's 32 rows) and A = the read vectors
    // r g k and r g q of those rows, each in three bf16 parts (rows m = 0..2 and 4..6 of A; the
    // products are exact and accumulate in fp32). apart[3 v + part][wave][rl] holds the 8 bf16
    // of rows lq_row(it = 0..7) that lane (m, rl) supplies.
    __shared__ uint4 apart[6][4][4];
    __shared__ f32x4 redpo[2][4][kD / 4];  // per-wave column sums of the old state: p, o
    const int h = head_of_block(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c16 = lane & 15, rl = lane >> 4;
    const size_t vec_off = static_cast<size_t>(h) * kD;
    uint32_t* Zh = Z + static_cast<size_t>(h) * kD * (kD / 8);

    // ---- loads: the lane's code words and column factors, the key-side inputs of row tid
    uint32_t zw[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) zw[it] = __builtin_nontemporal_load(Zh + sq_row(it, wave, rl) * (kD / 8) + c16);
    const uint4 cw = *reinterpret_cast<const uint4*>(C + vec_off + 8 * c16);
    float kr = 0.f, qr = 0.f, gr = 1.f, rr = 0.f, vr = 0.f;
    if (tid < kD) {
        kr = load_in(k, vec_off + tid);
        gr = kPerKey ? gate[vec_off + tid] : gate[h];
        rr = static_cast<float>(R[vec_off + tid]);
        if constexpr (kRead) {
            qr = load_in(q, vec_off + tid);
            vr = load_in(v, vec_off + tid);
        } else {
            ucol[tid] = u_io[vec_off + tid];
        }
    }
    const float bt = kRead ? beta[h] : 0.f;
    if (tid < kD) {
        const float rg = rr * gr;
        rowv[tid] = f32x2{rg, kr};
        if constexpr (kRead) {
            const int it = tid >> 4, w = (tid >> 2) & 3, r4 = tid & 3;  // tid = sq_row(it, w, r4)
            uint16_t* ap = reinterpret_cast<uint16_t*>(apart);
            uint16_t hi, mid, lo;
            sq_split3(rg * kr, hi, mid, lo);
            ap[((0 * 4 + w) * 4 + r4) * 8 + it] = hi;
            ap[((1 * 4 + w) * 4 + r4) * 8 + it] = mid;
            ap[((2 * 4 + w) * 4 + r4) * 8 + it] = lo;
            sq_split3(rg * qr, hi, mid, lo);
            ap[((3 * 4 + w) * 4 + r4) * 8 + it] = hi;
            ap[((4 * 4 + w) * 4 + r4) * 8 + it] = mid;
            ap[((5 * 4 + w) * 4 + r4) * 8 + it] = lo;
        }
        if constexpr (kRead) {
            const float kq = wave_sum(kr * qr);
            if (lane == 0) kq_part[wave] = kq;
        }
    }
    if constexpr (kPack) sq_row_weights(L, omega + vec_off, tid);
    __syncthreads();  // publishes rowv, the row weights and (repack) ucol

    // ---- the codes as floats 16 z, the two column sums of the old state p = X^T (g k) and
    // o = X^T (g q) on the matrix cores (c / 16 applied to each column's sum), and the decoded
    // X_{t-1} = r c z (the column factor applied here, the row factor with the gate in rowv)
    float cc[8];
    {
        const half_t* ch = reinterpret_cast<const half_t*>(&cw);
#pragma unroll
        for (int e = 0; e < 8; ++e) cc[e] = static_cast<float>(ch[e]) * 0.0625f;  // the codes come as 16 z
    }
    float zf[8][8];  // 16 z
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const uint32_t ev = (zw[it] << 4) & 0xF0F0F0F0u, od = zw[it] & 0xF0F0F0F0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            zf[it][2 * j] = static_cast<float>(static_cast<int8_t>(ev >> (8 * j)));
            zf[it][2 * j + 1] = static_cast<float>(static_cast<int8_t>(od >> (8 * j)));
        }
    }
    if constexpr (kRead) {
        // lane (m = l & 15, rl): A row m is part m % 4 of read vector m / 4 (m % 4 == 3 and m >= 8: zero)
        const int m = c16, am = (m >> 2) * 3 + (m & 3);
        const bool live = m < 8 && (m & 3) != 3;
        const uint4 aw = live ? apart[am][wave][rl] : uint4{0u, 0u, 0u, 0u};
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, aw);
        float part[8];  // lane rl = 0: p of column 8 c16 + e; rl = 1: o; others unused
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint4 bw;
            bw.x = __builtin_amdgcn_perm(__float_as_uint(zf[1][e]), __float_as_uint(zf[0][e]), 0x07060302u);
            bw.y = __builtin_amdgcn_perm(__float_as_uint(zf[3][e]), __float_as_uint(zf[2][e]), 0x07060302u);
            bw.z = __builtin_amdgcn_perm(__float_as_uint(zf[5][e]), __float_as_uint(zf[4][e]), 0x07060302u);
            bw.w = __builtin_amdgcn_perm(__float_as_uint(zf[7][e]), __float_as_uint(zf[6][e]), 0x07060302u);
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bw),
                                                                    f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            part[e] = (d.x + d.y + d.z) * cc[e];
        }
        if (rl < 2) {
            f32x4* dst = redpo[rl][wave] + 2 * c16;
            dst[0] = f32x4{part[0], part[1], part[2], part[3]};
            dst[1] = f32x4{part[4], part[5], part[6], part[7]};
        }
        __syncthreads();
        if (tid < kD) {  // column tid: correction, output
            const float* rp = reinterpret_cast<const float*>(redpo[0]);
            const float* ro = reinterpret_cast<const float*>(redpo[1]);
            const float pt = (rp[tid] + rp[kD + tid]) + (rp[2 * kD + tid] + rp[3 * kD + tid]);
            const float ot = (ro[tid] + ro[kD + tid]) + (ro[2 * kD + tid] + ro[3 * kD + tid]);
            const float u = bt * (vr - pt);
            y[vec_off + tid] = ot + u * (kq_part[0] + kq_part[1]);
            if constexpr (kMode == kSqReadout)
                u_io[vec_off + tid] = u;
            else
                ucol[tid] = u;
        }
        if constexpr (kMode == kSqReadout) return;
        __syncthreads();
    }
    float cz[8][8];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int e = 0; e < 8; ++e) cz[it][e] = zf[it][e] * cc[e];

    // ---- X_t = Diag(g) X_{t-1} + k u^T in registers, then packed
    float uc[8];
    {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(ucol + 8 * c16);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(ucol + 8 * c16 + 4);
        uc[0] = u0.x; uc[1] = u0.y; uc[2] = u0.z; uc[3] = u0.w;
        uc[4] = u1.x; uc[5] = u1.y; uc[6] = u1.z; uc[7] = u1.w;
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const f32x2 rv = rowv[sq_row(it, wave, rl)];
#pragma unroll
        for (int e = 0; e < 8; ++e) cz[it][e] = fmaf(rv.x, cz[it][e], rv.y * uc[e]);
    }
    sq_pack(L, cz, tid, Zh, R + vec_off, C + vec_off);
}

}  // namespace

hipError_t launch_sq_pack(int heads, const float* S, const float* omega, void* Z, void* R, void* C,
                          hipStream_t stream) {
    hipLaunchKernelGGL(sq_pack_kernel, dim3(heads), dim3(kThreads), 0, stream, S, omega,
                       static_cast<uint32_t*>(Z), static_cast<half_t*>(R), static_cast<half_t*>(C));
    return hipGetLastError();
}

hipError_t launch_sq_step(const StepArgs& a, int mode, void* Z, void* R, void* C, const float* omega, float* u,
                          bool per_key, bool bf16, hipStream_t stream) {
    auto go = [&](auto kernel, auto tag) {
        using T = decltype(tag);
        hipLaunchKernelGGL(kernel, dim3(a.heads), dim3(kThreads), 0, stream, static_cast<uint32_t*>(Z),
                           static_cast<half_t*>(R), static_cast<half_t*>(C), omega, static_cast<const T*>(a.q),
                           static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.gate, a.beta, u, a.y);
    };
    auto by_mode = [&](auto mode_tag) {
        constexpr int M = decltype(mode_tag)::value;
        if (per_key) {
            if (bf16) go(sq_step_kernel<M, true, bf16_t>, bf16_t{});
            else go(sq_step_kernel<M, true, float>, float{});
        } else {
            if (bf16) go(sq_step_kernel<M, false, bf16_t>, bf16_t{});
            else go(sq_step_kernel<M, false, float>, float{});
        }
    };
    if (mode == kSqReadout) by_mode(std::integral_constant<int, kSqReadout>{});
    else if (mode == kSqRepack) by_mode(std::integral_constant<int, kSqRepack>{});
    else by_mode(std::integral_constant<int, kSqFused>{});
    return hipGetLastError();
}

}  // namespace rsu
