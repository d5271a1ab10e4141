/*
 * rsu.h -- C ABI of the MI355X (gfx950) decode-step library for delta-rule
 * recurrent states (Gated DeltaNet and Kimi Delta Attention), and for RWKV6's
 * and RWKV7's states in the same common form.
 *
 * Per head the state S is d_k x d_v = 128 x 128; row i is a key channel and
 * column j a value channel. One decode step applies the retention gate g
 * (a scalar alpha for GDN, a per-key vector d for KDA), reads the old value
 * along the key from the decayed state, writes the beta-weighted correction
 * and returns y = S^T q from the updated state:
 *
 *     u = beta (v - (Diag(g) S)^T k),   S <- Diag(g) S + k u^T,   y = S^T q
 *
 * (LeapQuant, sec. 3.1 eq. 1 and App. A, the GDN and KDA expansions with beta
 * carried by the correction; STEPQuant reading notes, the unified recurrence
 * with the step output read after the update.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array pointer is a DEVICE pointer owned by the caller,
 *           contiguous, row-major and 16-byte aligned. The library never
 *           allocates, frees or synchronises; each call enqueues its kernels on
 *           `stream` (NULL = the null stream) and returns without waiting.
 *           (The one exception is rsu_debug_metadata_counts, a checking call.)
 * Shapes.   B requests x H heads. d_k and d_v must both be 128. B*H == 0 is a
 *           valid empty batch: nothing is launched and 0 is returned.
 * Inputs.   q, k [B,H,d_k] and v [B,H,d_v] are fp32 or bf16 (dims->qkv_dtype).
 *           Gates and beta are fp32: alpha [B,H] (GDN) or d [B,H,d_k] (KDA),
 *           beta [B,H]. Gates must be > 0 for the log path (it takes ln g).
 * Outputs.  y [B,H,d_v] fp32.
 * Errors.   The return value is RSU_OK or a negative RSU_E_* code. On error
 *           nothing is launched and no buffer is written; rsu_last_error()
 *           returns a message (per calling thread). RSU_E_HIP reports a failed
 *           launch: the kernel did not run.
 * Overlap.  Calls that write the same buffers must be ordered by the caller
 *           (same stream, or events). Input and output arrays must not alias,
 *           except where a buffer is documented as updated in place.
 */
#ifndef RSU_H
#define RSU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ABI-compatible with hipStream_t */
typedef struct ihipStream_t *rsu_stream_t;

enum rsu_dtype { RSU_F32 = 0, RSU_BF16 = 1 };

enum rsu_status {
    RSU_OK = 0,
    RSU_E_NULL = -1,      /* a required pointer is NULL */
    RSU_E_DIMS = -2,      /* B or H negative, d_k or d_v not 128, or B*H too large */
    RSU_E_DTYPE = -3,     /* qkv_dtype not RSU_F32 / RSU_BF16 */
    RSU_E_ALIGN = -4,     /* a pointer is not 16-byte aligned */
    RSU_E_RANGE = -5,     /* W / pos / C / L out of range */
    RSU_E_HIP = -6,       /* the kernel launch failed */
    RSU_E_UNSUPPORTED = -7 /* the call needs a build option this library lacks */
};

typedef struct rsu_dims {
    int32_t B, H;         /* requests, heads per request */
    int32_t dk, dv;       /* must be 128, 128 */
    int32_t qkv_dtype;    /* enum rsu_dtype: element type of q, k, v and of the stored keys */
} rsu_dims;

/* Version of this ABI (incremented on any signature or semantic change). */
int rsu_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char *rsu_last_error(void);

/* ------------------------------------------------------------------------
 * Dense fp32 state, one eager decode step.
 * GDN (LeapQuant App. A, GDN expansion): the gate is alpha [B,H].
 * KDA (LeapQuant App. A, KDA expansion): the gate is d [B,H,d_k].
 * S [B,H,d_k,d_v] fp32 is read once and written once, updated in place.
 * ---------------------------------------------------------------------- */
int gdn_decode_step(const rsu_dims *dims, float *S, const void *q, const void *k,
                    const void *v, const float *alpha, const float *beta, float *y,
                    rsu_stream_t stream);
int kda_decode_step(const rsu_dims *dims, float *S, const void *q, const void *k,
                    const void *v, const float *d, const float *beta, float *y,
                    rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * Int8 state with per-key-row scales (STEPQuant notes, the per-row absmax
 * baseline; LeapQuant App. B.3, the /127 convention):
 *   a_i = max_j |S_ij| (fp32),  z_ij = clamp(rne(S_ij * (127 / a_i)), -127, 127),
 *   dequant = z_ij * a_i / 127;  a row of zeros gets a_i = 0 and z = 0.
 * The reciprocal 127/a_i is one correctly rounded fp32 division, the product
 * one fp32 multiplication, rounding is to nearest with ties to even. A row with
 * a_i below 2^-64 (where 127/a_i can overflow fp32) is decided as that row and
 * a_i multiplied by 2^64 (exact); a_i is stored unscaled. (The pages are silent
 * on such rows; this keeps the codes of rne(S_ij * 127 / a_i).)
 *
 * q8_quantize: quantize S [B,H,d_k,d_v] fp32 into Z [B,H,d_k,d_v] int8 and
 * row_absmax [B,H,d_k] fp32 (the state at the start of the first window).
 * ---------------------------------------------------------------------- */
int q8_quantize(const rsu_dims *dims, const float *S, int8_t *Z, float *row_absmax,
                rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * Per-window quantization (LeapQuant sec. 3.2, eqs. 3-4; readout App. B.2
 * eq. 9). (Z, row_absmax) is the quantized window-start state and stays fixed
 * inside the window; step pos (0 <= pos < W, the same for the whole batch)
 * computes the correction u and the output from it and the pos earlier
 * records, and stores its own record (g, k, u) in slot pos:
 *   Kbuf [B,H,W,d_k] in qkv_dtype, Ubuf [B,H,W,d_v] fp32,
 *   Gbuf [B,H,W] fp32 (GDN) or [B,H,W,d_k] fp32 (KDA).
 * At pos == W-1 the step output is read from the unquantized state S_W, then
 * S_W is requantized into Z and row_absmax in place (records of slot W-1 are
 * not stored; the caller's next call uses pos = 0). 1 <= W <= 32.
 * ---------------------------------------------------------------------- */
int gdn_q8_window(const rsu_dims *dims, int W, int pos, int8_t *Z, float *row_absmax,
                  void *Kbuf, float *Ubuf, float *Gbuf, const void *q, const void *k,
                  const void *v, const float *alpha, const float *beta, float *y,
                  rsu_stream_t stream);
int kda_q8_window(const rsu_dims *dims, int W, int pos, int8_t *Z, float *row_absmax,
                  void *Kbuf, float *Ubuf, float *Gbuf, const void *q, const void *k,
                  const void *v, const float *d, const float *beta, float *y,
                  rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * Dense base + bounded log (DeltaLog sec. 3.1, Algorithm 1, eqs. 4-7).
 * Physical state: base Sbase [B,H,d_k,d_v] fp32; cumulative log-decay lbar
 * [B,H] (GDN) or [B,H,d_k] (KDA) fp32; log of capacity C = M - 1 entries:
 *   Klog [B,H,C,d_k] in qkv_dtype (the key factor a = k, stored losslessly),
 *   Ulog [B,H,C,d_v] fp32 (the value factor b = u),
 *   Lam  [B,H,C] (GDN) or [B,H,C,d_k] (KDA) fp32 (lbar after the entry's decay).
 * L (0 <= L <= C, the same for the whole batch) is the live log length, kept
 * by the caller. The represented state is eq. 7:
 *   S = D(lbar) Sbase + sum_{m<L} D(lbar - Lam_m) K_m U_m^T,  D(l) = diag(exp l).
 *
 * *_log_append (requires 0 <= L < C): computes the correction and the output
 * from the represented state, adds ln g to lbar, and writes entry L
 * (Klog[L] = k, Ulog[L] = u, Lam[L] = lbar). Sbase is only read.
 * The caller then sets L = L + 1.
 *
 * *_log_merge (requires L == C >= 0): the same step, but instead of appending
 * it writes the represented state plus the current pair into Sbase (eq. 6)
 * and resets lbar to 0. The caller then sets L = 0.
 * 0 <= C <= 63 (M = C + 1 <= 64; DeltaLog sec. 4 sweeps M up to 64).
 * ---------------------------------------------------------------------- */
int gdn_log_append(const rsu_dims *dims, int C, int L, const float *Sbase, float *lbar,
                   void *Klog, float *Ulog, float *Lam, const void *q, const void *k,
                   const void *v, const float *alpha, const float *beta, float *y,
                   rsu_stream_t stream);
int kda_log_append(const rsu_dims *dims, int C, int L, const float *Sbase, float *lbar,
                   void *Klog, float *Ulog, float *Lam, const void *q, const void *k,
                   const void *v, const float *d, const float *beta, float *y,
                   rsu_stream_t stream);
int gdn_log_merge(const rsu_dims *dims, int C, int L, float *Sbase, float *lbar,
                  const void *Klog, const float *Ulog, const float *Lam, const void *q,
                  const void *k, const void *v, const float *alpha, const float *beta,
                  float *y, rsu_stream_t stream);
int kda_log_merge(const rsu_dims *dims, int C, int L, float *Sbase, float *lbar,
                  const void *Klog, const float *Ulog, const float *Lam, const void *q,
                  const void *k, const void *v, const float *d, const float *beta,
                  float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * LeapQuant's window-boundary format (LeapQuant sec. 3.3 eqs. 5-6, sec. 3.4
 * eq. 7, App. B.3 eq. 10), for scalar (GDN) and per-key (KDA) gates. A window
 * starts from
 *   S_0 = C dequant(Z, B) + Kt Ut^T,  C = Diag(row_smooth),
 *   dequant(Z, B)_ij = Z_ij * col_absmax_j / 127,
 * i.e. r = 4 compensator token pairs (Kt, Ut) in fp16 that hold the dominant
 * low-rank part, a per-key-row smoothing scale, and an int8 payload of the
 * smoothed residual with one fp32 absmax per value column.
 *   Z [B,H,d_k,d_v] int8, col_absmax [B,H,d_v] fp32, row_smooth [B,H,d_k] fp32,
 *   Kc, Uc [B,H,4,d] fp16 (token-major: Kc[b][h][t][i] is key row i of token t).
 * The tokens are fitted by subspace iteration: V <- MGS(S^T S V), n_iter times,
 * Kt = S V, Ut = V (MGS = modified Gram-Schmidt over the 4 columns in order), then
 * rounded to fp16; the residual R = S - Kt Ut^T (with the rounded tokens) gets
 * row_smooth_i = max(sqrt(mean_j |R_ij|), 1e-6) and the payload of R_ij / row_smooth_i,
 * rounded half to even into [-127, 127] per value column (a column whose absmax is
 * below 2^-64 is decided scaled by 2^64, as for the per-row int8 state).
 *
 * gdn_lq_quantize: converts plain fp32 states S into the format; the fit starts
 *   from the first 4 Walsh columns ((-1)^popcount(i & t) / sqrt(d)). S is only read.
 * gdn_lq_window: one decode step inside a window, like gdn_q8_window (records
 *   Kbuf [B,H,W,d] bf16, Ubuf [B,H,W,d] fp32, Gbuf [B,H,W] fp32 as there), reading
 *   by eq. 10; at pos = W-1 it forms S_W, refits the tokens starting from the
 *   current Ut, and rewrites Z, col_absmax, row_smooth, Kc and Uc in place.
 * kda_lq_window: the same with the per-key gate d [B,H,d_k] and Gbuf [B,H,W,d_k]
 *   (Gamma in eq. 10 is diagonal over the key rows). kda_lq_quantize is the same
 *   conversion as gdn_lq_quantize (the format does not depend on the gates).
 * Requires bf16 q/k/v (else RSU_E_DTYPE), 1 <= W <= 16, 0 <= pos < W,
 * 0 <= n_iter <= 64 (else RSU_E_RANGE). Other rules as for the int8 window.
 * ---------------------------------------------------------------------- */
int gdn_lq_quantize(const rsu_dims *dims, const float *S, int n_iter, int8_t *Z,
                    float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                    rsu_stream_t stream);
int gdn_lq_window(const rsu_dims *dims, int W, int pos, int n_iter, int8_t *Z,
                  float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                  float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                  const float *alpha, const float *beta, float *y, rsu_stream_t stream);
/* The same format at 4 bits with r = 8 tokens (LeapQuant sec. 4.1 fits 8 tokens at
 * 4 bits), GDN: codes in [-7, 7] with dequant Z_ij * col_absmax_j / 7, two per byte
 * (column 2m in the low nibble, 2m + 1 in the high nibble, two's complement):
 *   Z [B,H,d_k,d_v/2] bytes, Kc, Uc [B,H,8,d] fp16; col_absmax, row_smooth as above.
 * The fit starts from the first 8 Walsh columns; other rules as for gdn_lq_window. */
int gdn_lq4_quantize(const rsu_dims *dims, const float *S, int n_iter, void *Z,
                     float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                     rsu_stream_t stream);
int gdn_lq4_window(const rsu_dims *dims, int W, int pos, int n_iter, void *Z,
                   float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                   float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                   const float *alpha, const float *beta, float *y, rsu_stream_t stream);
/* The same format at 6 bits (LeapQuant sec. 4.1 and Table 1 evaluate a 6-bit group; the
 * token count stays r = 4), GDN: codes in [-31, 31] with dequant Z_ij * col_absmax_j / 31.
 * Row i of a head's payload is 96 bytes: bytes 0..63 hold the high parts z >> 2 (floor
 * division, 4-bit two's complement) two per byte as in gdn_lq4_window, bytes 64..95 the
 * low parts z & 3 four per byte, column 4b + m in bits 2m .. 2m+1 of byte 64 + b:
 *   Z [B,H,d_k,96] bytes, Kc, Uc [B,H,4,d] fp16; col_absmax, row_smooth as above.
 * The fit starts from the first 4 Walsh columns; other rules as for gdn_lq_window. */
int gdn_lq6_quantize(const rsu_dims *dims, const float *S, int n_iter, void *Z,
                     float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                     rsu_stream_t stream);
int gdn_lq6_window(const rsu_dims *dims, int W, int pos, int n_iter, void *Z,
                   float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                   float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                   const float *alpha, const float *beta, float *y, rsu_stream_t stream);
/* KDA at 4 and 6 bits (LeapQuant sec. 4.2 evaluates both widths on a KDA model): the
 * formats of gdn_lq4_window / gdn_lq6_window with the per-key gate d [B,H,d_k] and
 * Gbuf [B,H,W,d_k], as kda_lq_window is to gdn_lq_window. kda_lq4_quantize and
 * kda_lq6_quantize are the conversions of gdn_lq4_quantize / gdn_lq6_quantize (the
 * format does not depend on the gates). Rules as for gdn_lq_window. */
int kda_lq4_quantize(const rsu_dims *dims, const float *S, int n_iter, void *Z,
                     float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                     rsu_stream_t stream);
int kda_lq4_window(const rsu_dims *dims, int W, int pos, int n_iter, void *Z,
                   float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                   float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                   const float *d, const float *beta, float *y, rsu_stream_t stream);
int kda_lq6_quantize(const rsu_dims *dims, const float *S, int n_iter, void *Z,
                     float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                     rsu_stream_t stream);
int kda_lq6_window(const rsu_dims *dims, int W, int pos, int n_iter, void *Z,
                   float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                   float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                   const float *d, const float *beta, float *y, rsu_stream_t stream);
int kda_lq_quantize(const rsu_dims *dims, const float *S, int n_iter, int8_t *Z,
                    float *col_absmax, float *row_smooth, void *Kc, void *Uc,
                    rsu_stream_t stream);
int kda_lq_window(const rsu_dims *dims, int W, int pos, int n_iter, int8_t *Z,
                  float *col_absmax, float *row_smooth, void *Kc, void *Uc, void *Kbuf,
                  float *Ubuf, float *Gbuf, const void *q, const void *k, const void *v,
                  const float *d, const float *beta, float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * Per-slot live lengths. DeltaLog sec. 4 keeps the live-log length as per-slot
 * metadata; requests admitted at different times sit at different points of
 * their append/merge cycle, and its serving prototype splits them into
 * phase-uniform append and merge batches. These calls serve a mixed batch in
 * one call instead, without the host knowing any L: two launches on `stream`, an
 * append pass over the heads with L[h] < C, then a merge pass over the heads with
 * L[h] == C that also advances every L[h]. L is a device array [B,H] of int32,
 * read and advanced in place: a head with L[h] < C appends (as *_log_append) and
 * gets L[h] + 1; a head with L[h] == C merges (as *_log_merge) and gets 0.
 * Other arguments, layouts and ranges as for *_log_append; Sbase is written for
 * the merging heads only. L[h] outside [0, C] is not detected: the kernel clamps
 * it into [0, C] (so every access stays inside the caller's buffers), and the
 * result for that head is then that of the clamped length.
 * ---------------------------------------------------------------------- */
int gdn_log_step_slots(const rsu_dims *dims, int C, int *L, float *Sbase, float *lbar,
                       void *Klog, float *Ulog, float *Lam, const void *q, const void *k,
                       const void *v, const float *alpha, const float *beta, float *y,
                       rsu_stream_t stream);
int kda_log_step_slots(const rsu_dims *dims, int C, int *L, float *Sbase, float *lbar,
                       void *Klog, float *Ulog, float *Lam, const void *q, const void *k,
                       const void *v, const float *d, const float *beta, float *y,
                       rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * RWKV6 in the pages' common form (DeltaLog Table 1, the RWKV6 row: state
 * transform D(lambda) S, update pair (k, v), per-key decay; LeapQuant App. A,
 * eq. 1 with read vector 0): no delta read and no beta,
 *     S <- Diag(w) S + k v^T,   y = S^T q,
 * with w [B,H,d_k] fp32 the per-key decay (w > 0 for the log calls, which take
 * ln w). RWKV6's own extra term for the current token is not part of this form.
 *
 * rwkv6_decode_step: the dense fp32 state S, read once, written once, in place.
 * rwkv6_log_append / rwkv6_log_merge / rwkv6_log_step_slots: the base + log
 * representation as for KDA (lbar [B,H,d_k], Lam [B,H,C,d_k] fp32) with the
 * value factor b = v: Ulog [B,H,C,d_v] holds the raw values in qkv_dtype (the
 * page keeps both RWKV6 log factors in bf16, DeltaLog sec. 3.4 and Table 3).
 * Arguments, ranges, the live-length protocol and errors as for the KDA calls,
 * without beta.
 * ---------------------------------------------------------------------- */
int rwkv6_decode_step(const rsu_dims *dims, float *S, const void *q, const void *k,
                      const void *v, const float *w, float *y, rsu_stream_t stream);
int rwkv6_log_append(const rsu_dims *dims, int C, int L, const float *Sbase, float *lbar,
                     void *Klog, void *Ulog, float *Lam, const void *q, const void *k,
                     const void *v, const float *w, float *y, rsu_stream_t stream);
int rwkv6_log_merge(const rsu_dims *dims, int C, int L, float *Sbase, float *lbar,
                    const void *Klog, const void *Ulog, const float *Lam, const void *q,
                    const void *k, const void *v, const float *w, float *y,
                    rsu_stream_t stream);
int rwkv6_log_step_slots(const rsu_dims *dims, int C, int *L, float *Sbase, float *lbar,
                         void *Klog, void *Ulog, float *Lam, const void *q, const void *k,
                         const void *v, const float *w, float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * RWKV7 as two sub-steps of the general update (LeapQuant App. A, models with a
 * separate erase direction: the transition Diag(w) - kappa (a * kappa)^T):
 *     S' = Diag(w) S + kappa (0 - S^T (a * kappa))^T     erase along kappa
 *     S  = S' + k v^T,   y = S^T q                        write, then the output
 * q, k, v, kappa [B,H,d] in qkv_dtype (kappa is the removal key), w [B,H,d_k] fp32
 * the per-key decay, a [B,H,d_k] fp32 the per-key erase rate. No beta. The dense
 * state S is read once and written once, in place; both sub-steps happen in the same
 * pass. Arguments and errors as for rwkv6_decode_step.
 * ---------------------------------------------------------------------- */
int rwkv7_decode_step(const rsu_dims *dims, float *S, const void *q, const void *k,
                      const void *v, const void *kappa, const float *w, const float *a,
                      float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * RWKV7 on the per-window int8 state, two records per token (LeapQuant App. A:
 * the same treatment as a DeltaProduct token with two sub-steps). A window of W
 * tokens buffers 2W records; token pos writes record 2 pos = the erase
 * (gate w, key kappa, value 0 - S_{t-1}^T (a * kappa)) and record 2 pos + 1 = the
 * write (gate 1, key k, value v), and returns y = S_t^T q read by eq. 9 over the
 * window-start (Z, row_absmax) and the records:
 *   Kbuf [B,H,2W,d] in qkv_dtype, Ubuf [B,H,2W,d] fp32, Gbuf [B,H,2W,d_k] fp32.
 * At pos = W-1 the token's records are appended as well and S_W (eq. 4 over all
 * 2W records) is requantized into Z and row_absmax in place, by a second launch on
 * the same stream. 1 <= W <= 16, 0 <= pos < W. Inputs as for rwkv7_decode_step;
 * codes, scales and other rules as for the per-row int8 window.
 * ---------------------------------------------------------------------- */
int rwkv7_q8_window(const rsu_dims *dims, int W, int pos, int8_t *Z, float *row_absmax,
                    void *Kbuf, float *Ubuf, float *Gbuf, const void *q, const void *k,
                    const void *v, const void *kappa, const float *w, const float *a,
                    float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * DeltaProduct (LeapQuant App. A, Table 4: n delta-rule sub-steps of eq. 1 per
 * token). Sub-step i (0-based) has its own key k_i, value v_i and strength
 * beta_i; the token's scalar gate alpha decays the state once, in the first
 * sub-step; the output is read after the last:
 *     S' = d_i S (d_0 = alpha, d_i = 1 for i > 0),  u_i = beta_i (v_i - S'^T k_i),
 *     S  = S' + k_i u_i^T,   and after the n sub-steps  y = S^T q.
 * q [B,H,d_k], k [B,H,n,d_k], v [B,H,n,d_v] in qkv_dtype; alpha [B,H], beta [B,H,n]
 * fp32; 1 <= n <= 4 (else RSU_E_RANGE). With n = 1 this is gdn_decode_step.
 *
 * deltaproduct_decode_step: the dense fp32 state S [B,H,d_k,d_v], read once and
 *   written once, in place (every read of the token comes from the old state).
 * deltaproduct_q8_window: the per-row int8 window of gdn_q8_window with one record
 *   per sub-step (LeapQuant App. A treats a token with two sub-steps the same way):
 *   token pos writes records n pos .. n pos + n - 1 with gates alpha, 1, .., 1:
 *   Kbuf [B,H,nW,d_k] in qkv_dtype, Ubuf [B,H,nW,d_v] fp32, Gbuf [B,H,nW] fp32.
 *   At pos = W-1 the token's records are appended as well and S_W (eq. 4 over all
 *   nW records) is requantized into Z and row_absmax in place by a second launch
 *   on the same stream. 1 <= W, n W <= 32, 0 <= pos < W. Codes, scales and other
 *   rules as for the int8 window.
 * ---------------------------------------------------------------------- */
int deltaproduct_decode_step(const rsu_dims *dims, int n, float *S, const void *q,
                             const void *k, const void *v, const float *alpha,
                             const float *beta, float *y, rsu_stream_t stream);
int deltaproduct_q8_window(const rsu_dims *dims, int n, int W, int pos, int8_t *Z,
                           float *row_absmax, void *Kbuf, float *Ubuf, float *Gbuf,
                           const void *q, const void *k, const void *v, const float *alpha,
                           const float *beta, float *y, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * STEPQuant's per-step packed state (STEPQuant notes, the section on the
 * key-row-aware dual-axis fit, and the section on one decode step in SGLang):
 * element (i, j) of a head's state is R_i C_j z_ij with fp16 key-row factors R,
 * fp16 value-column factors C and 4-bit codes z in [-7, 7], refitted from the new
 * state after every decode step.
 *   Z     [B,H,d_k,d_v/2] bytes, two's complement nibbles, value column 2m in the
 *         low nibble of byte m, 2m + 1 in the high nibble
 *   R, C  [B,H,d] fp16
 *   omega [B,H,d_k] fp32 row influence scores (> 0), read only
 * The packing of a state X: w_i = omega_i^(1/8) over its geometric mean in the head
 * (the notes' compression exponent 0.25 on sqrt(omega)); R_i = fp16(sqrt(m_i / w_i))
 * with m_i = mean_j |X_ij|; a_j = max_i |X_ij / R_i|; z_ij = X_ij / R_i * 7 / a_j
 * rounded half to even and clamped to [-7, 7] (0 where R_i or a_j is 0); C_j = fp16
 * of the weighted least squares sum_i w_i^2 R_i z_ij X_ij / sum_i w_i^2 R_i^2 z_ij^2
 * (0 for a column without nonzero codes). The row factor's formula is a reading
 * (the notes name SmoothQuant's fractional power; its square root is taken). A column
 * with a_j below 2^-64 has C_j (about a_j / 7) zero in fp16 and decodes to zero; its
 * codes lie in [-7, 7] but are otherwise unspecified (7 / a_j is capped where it
 * overflows fp32).
 *
 * stepq_pack: packs fp32 states S [B,H,d,d] (only read); dims->qkv_dtype is not used.
 * gdn_stepq_step / kda_stepq_step: one decode step on the packed state in place:
 *   X = R C z, then the dense step of gdn_decode_step / kda_decode_step on X (y
 *   read from the updated state), then X_t packed into Z, R, C.
 * Other rules as for the dense step; calls that share Z, R, C must not overlap.
 * ---------------------------------------------------------------------- */
int stepq_pack(const rsu_dims *dims, const float *S, const float *omega, void *Z, void *R,
               void *C, rsu_stream_t stream);
int gdn_stepq_step(const rsu_dims *dims, void *Z, void *R, void *C, const float *omega,
                   const void *q, const void *k, const void *v, const float *alpha,
                   const float *beta, float *y, rsu_stream_t stream);
int kda_stepq_step(const rsu_dims *dims, void *Z, void *R, void *C, const float *omega,
                   const void *q, const void *k, const void *v, const float *d,
                   const float *beta, float *y, rsu_stream_t stream);
/* The same step in two launches, as the notes run it in SGLang: the readout first
 * (decode, update, y), the dual-axis repack on another stream behind the rest of the
 * model, done before the next read of the state.
 * gdn_stepq_readout / kda_stepq_readout: decode X = R C z, the correction
 *   u = beta (v - X^T (g k)) and y = X_t^T q; writes u [B,H,d_v] fp32 (caller-owned) and
 *   y; Z, R, C are only read.
 * gdn_stepq_repack / kda_stepq_repack: X_t = Diag(g) X + k u^T from the same packed
 *   state and the readout's u, packed into Z, R, C in place (k in dims->qkv_dtype).
 * The pair repeats the fused step's arithmetic: y, u and the new Z, R, C equal those
 * of gdn_stepq_step / kda_stepq_step bit for bit. The caller orders them (the repack
 * after its readout, the next readout after the repack; e.g. with HIP events across
 * two streams). Other rules as for the fused step. */
int gdn_stepq_readout(const rsu_dims *dims, const void *Z, const void *R, const void *C,
                      const void *q, const void *k, const void *v, const float *alpha,
                      const float *beta, float *u, float *y, rsu_stream_t stream);
int kda_stepq_readout(const rsu_dims *dims, const void *Z, const void *R, const void *C,
                      const void *q, const void *k, const void *v, const float *d,
                      const float *beta, float *u, float *y, rsu_stream_t stream);
int gdn_stepq_repack(const rsu_dims *dims, void *Z, void *R, void *C, const float *omega,
                     const void *k, const float *alpha, const float *u, rsu_stream_t stream);
int kda_stepq_repack(const rsu_dims *dims, void *Z, void *R, void *C, const float *omega,
                     const void *k, const float *d, const float *u, rsu_stream_t stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not part of the recurrence): dst[i] = src[i] for
 * n fp32 elements, with the same 128-bit non-temporal access pattern and grid
 * shape (64 KiB per workgroup) as the dense step. n must be a multiple of 4.
 * Used to find the practical read+write HBM ceiling and to calibrate counters.
 * ---------------------------------------------------------------------- */
int rsu_copy_f32(const float *src, float *dst, int64_t n, rsu_stream_t stream);

/* Measurement helpers (not part of the recurrence): a read-only and a write-only stream
 * over `tiles` whole 128 x 128 fp32 tiles (64 KiB each), with the same 128-bit
 * non-temporal access pattern, tile order and grid shape as the dense step. Their rates
 * are the HBM read and write rates that bound a step that reads each tile once and writes
 * it once.
 * rsu_read_f32: reads src [tiles,128,128] and writes the column sums of each tile to
 *   col_sums [tiles,128] (512 B written per 64 KiB read).
 * rsu_fill_f32: sets every element of dst [tiles,128,128] to value.
 * 0 <= tiles <= 2^31 - 1; pointers 16-byte aligned; errors as above. */
int rsu_read_f32(const float *src, float *col_sums, int64_t tiles, rsu_stream_t stream);
int rsu_fill_f32(float *dst, float value, int64_t tiles, rsu_stream_t stream);

/* Checking build only: the log's single-writer rule (DeltaLog, sec. 3.3 and the caption
 * of Fig. 5: one writer per head commits K_log[L], Lam_log[L], lbar and L).
 * A library built with RSU_CHECK_METADATA counts, per head (heads 0 .. 65535), every
 * element of log metadata its log kernels write (all *_log_append, *_log_merge and
 * *_log_step_slots entry points). This call waits for `stream`, copies the counters of
 * heads 0 .. heads-1 to the HOST array counts [heads][8] (uint32; columns: K_log row
 * elements, Lam elements, lbar elements, L, U_log row elements, then three unused), and
 * clears every counter. One step writes, per head: an append 128 K_log, 128 U_log
 * and 128 (KDA, RWKV6) or 1 (GDN) Lam and lbar elements; a merge only lbar (same count);
 * a per-slot step also writes L once. Unlike the other calls it synchronises.
 * Errors: RSU_E_NULL (counts), RSU_E_RANGE (heads outside 0 .. 65536),
 * RSU_E_UNSUPPORTED (an ordinary build, which keeps no counters), RSU_E_HIP. */
int rsu_debug_metadata_counts(uint32_t *counts, int64_t heads, rsu_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RSU_H */
