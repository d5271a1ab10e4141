// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsu {

constexpr int kMaxW = 32;  // window length limit of the int8 path (LDS of the boundary step)
constexpr int kMaxC = 63;  // log capacity limit of the base + log path (M = C + 1 <= 64)

// Per-step inputs shared by every representation; pointers are device pointers.
struct StepArgs {
    int heads;                    // B * H (one workgroup per head)
    float* S;                     // dense fp32 state, or the base of the log path
    const void *q, *k, *v;        // [heads, 128] in fp32 or bf16
    const float* gate;            // [heads] or [heads, 128]
    const float* beta;            // [heads]
    float* y;                     // [heads, 128]
};

struct WindowArgs {
    int W, pos;
    int8_t* Z;                    // [heads, 128, 128]
    float* A;                     // [heads, 128] row absmax
    void* Kbuf;                   // [heads, W, 128] in the input dtype
    float* Ubuf;                  // [heads, W, 128]
    float* Gbuf;                  // [heads, W] or [heads, W, 128]
};

struct LogArgs {
    int C, L;                     // capacity; batch-uniform live length
    int* Lslot;                   // per-slot live lengths [heads] (per-slot calls only)
    float* lbar;                  // [heads] or [heads, 128]
    void* Klog;                   // [heads, C, 128] in the input dtype
    void* Ulog;                   // [heads, C, 128] fp32 (delta rule) or the input dtype (RWKV6)
    float* Lam;                   // [heads, C] or [heads, C, 128]
};

hipError_t launch_dense(const StepArgs& a, bool per_key, bool bf16, hipStream_t stream);
// RWKV6: S <- Diag(w) S + k v^T, y = S^T q (gate = w [heads, 128]; beta unused)
hipError_t launch_rwkv6(const StepArgs& a, bool bf16, hipStream_t stream);
// RWKV7: erase along kappa read with erase_rate * kappa, then write k v^T (gate = w [heads, 128];
// kappa [heads, 128] in the input dtype, erase_rate [heads, 128] fp32; beta unused)
hipError_t launch_rwkv7(const StepArgs& a, const void* kappa, const float* erase_rate, bool bf16,
                        hipStream_t stream);
// DeltaProduct with n sub-steps (1 <= n <= 4): k, v [heads, n, 128] in the input dtype, gate = alpha
// [heads], beta [heads, n]
hipError_t launch_deltaproduct(const StepArgs& a, int n, bool bf16, hipStream_t stream);
// Per-head metadata write counters of the log kernels, kept only by a build with
// RSU_CHECK_METADATA defined (kinds: K_log row, Lam entry, lbar, L, U_log row elements).
constexpr int kMetaCheckHeads = 1 << 16, kMetaKinds = 8;
enum MetaKind { kMetaK = 0, kMetaLam = 1, kMetaLbar = 2, kMetaL = 3, kMetaU = 4 };
// Copies the counters of the first `heads` heads to host memory after the stream's work
// has finished, then clears all counters; hipErrorNotSupported in the ordinary build.
hipError_t read_metadata_counts(unsigned* host, int64_t heads, hipStream_t stream);
hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t stream);
hipError_t launch_read_probe(const float* src, float* sums, int tiles, hipStream_t stream);
hipError_t launch_write_probe(float* dst, float value, int tiles, hipStream_t stream);
hipError_t launch_q8_quantize(int heads, const float* S, int8_t* Z, float* A, hipStream_t stream);
hipError_t launch_q8_window(const StepArgs& a, const WindowArgs& w, bool per_key, bool bf16,
                            hipStream_t stream);
// RWKV7 on the int8 window, two records per token (W <= 16; Kbuf, Ubuf, Gbuf hold 2W
// records per head, Gbuf per key): gate = w, kappa in the input dtype, erase [heads, 128]
hipError_t launch_rwkv7_q8_window(const StepArgs& a, const WindowArgs& w, const void* kappa, const float* erase,
                                  bool bf16, hipStream_t stream);
// DeltaProduct on the int8 window, one record per sub-step (n records per token, n W <= 32):
// k, v [heads, n, 128] in the input dtype, gate = alpha [heads], beta [heads, n]; Kbuf [heads, nW, 128],
// Ubuf [heads, nW, 128], Gbuf [heads, nW] scalar gates. At pos = W - 1 a second launch requantizes.
hipError_t launch_dp_q8_window(const StepArgs& a, const WindowArgs& w, int n, bool bf16, hipStream_t stream);
// LeapQuant's boundary format (GDN or KDA, bf16 keys, W <= 16): payload, per-column absmax,
// per-row smoothing scales, fp16 token pairs [heads][4][128], and the window's records.
struct LqArgs {
    int W, pos, n_iter;
    int8_t* Z;                    // [heads, 128, 128]
    float* B;                     // [heads, 128] per value column
    float* C;                     // [heads, 128] per key row
    void* Kc;                     // [heads, 4, 128] fp16
    void* Uc;                     // [heads, 4, 128] fp16
    void* Kbuf;                   // [heads, W, 128] bf16
    float* Ubuf;                  // [heads, W, 128]
    float* Gbuf;                  // [heads, W] (GDN) or [heads, W, 128] (KDA)
};

hipError_t launch_lq_quantize(int heads, const float* S, int n_iter, int8_t* Z, float* B, float* C,
                              void* Kc, void* Uc, hipStream_t stream);
hipError_t launch_lq_window(const StepArgs& a, const LqArgs& w, bool per_key, hipStream_t stream);
// The same format at low bit widths (GDN, or KDA with per_key): bits = 4 with 8 tokens, Z [heads, 128, 64] packed
// nibbles, Kc, Uc [heads, 8, 128] fp16; bits = 6 with 4 tokens, Z [heads, 128, 96] bytes (the
// high parts as nibbles, then the low 2-bit parts), Kc, Uc [heads, 4, 128] fp16.
hipError_t launch_lq_low_quantize(int bits, int heads, const float* S, int n_iter, void* Z, float* B, float* C,
                                  void* Kc, void* Uc, hipStream_t stream);
hipError_t launch_lq_low_window(int bits, const StepArgs& a, const LqArgs& w, bool per_key, hipStream_t stream);

// STEPQuant's packed state (4-bit codes with fp16 key-row and value-column factors):
// Z [heads, 128, 16] words of 8 signed nibbles, R [heads, 128] and C [heads, 128] fp16,
// omega [heads, 128] row influence scores.
hipError_t launch_sq_pack(int heads, const float* S, const float* omega, void* Z, void* R, void* C,
                          hipStream_t stream);
// mode: 0 the fused step, 1 the readout alone (writes u [heads, 128] and y; Z, R, C only read),
// 2 the repack alone (reads u; q, v, beta, y unused)
hipError_t launch_sq_step(const StepArgs& a, int mode, void* Z, void* R, void* C, const float* omega, float* u,
                          bool per_key, bool bf16, hipStream_t stream);

// mode: 0 append, 1 merge, 2 per-slot live lengths
hipError_t launch_log(const StepArgs& a, const LogArgs& l, int mode, bool per_key, bool bf16,
                      hipStream_t stream);
hipError_t launch_rwkv6_log(const StepArgs& a, const LogArgs& l, int mode, bool bf16, hipStream_t stream);

}  // namespace rsu
