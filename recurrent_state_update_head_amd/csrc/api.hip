// api.hip -- the extern "C" entry points declared in include/rsu.h: argument
// validation, error reporting, kernel dispatch. Nothing here allocates memory
// or synchronises the device (except the checking build's counter read-back).
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>

#include "../../include/rsu.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

// dims, dtype; on success *heads = B * H
int check_dims(const rsu_dims* d, int* heads, const char* fn) {
    g_err[0] = '\0';
    if (!d) return fail(RSU_E_NULL, "%s: dims is NULL", fn);
    if (d->B < 0 || d->H < 0) return fail(RSU_E_DIMS, "%s: B=%d H=%d must be >= 0", fn, d->B, d->H);
    if (d->dk != 128 || d->dv != 128)
        return fail(RSU_E_DIMS, "%s: dk=%d dv=%d, only 128 x 128 states are supported", fn, d->dk, d->dv);
    const long long n = static_cast<long long>(d->B) * d->H;
    if (n > 0x7fffffffLL) return fail(RSU_E_DIMS, "%s: B*H=%lld exceeds the grid limit", fn, n);
    if (d->qkv_dtype != RSU_F32 && d->qkv_dtype != RSU_BF16)
        return fail(RSU_E_DTYPE, "%s: qkv_dtype=%d is neither RSU_F32 nor RSU_BF16", fn, d->qkv_dtype);
    *heads = static_cast<int>(n);
    return RSU_OK;
}

struct Ptr {
    const void* p;
    const char* name;
};

int check_ptrs(std::initializer_list<Ptr> ptrs, const char* fn) {
    for (const Ptr& x : ptrs)
        if (!x.p) return fail(RSU_E_NULL, "%s: %s is NULL", fn, x.name);
    for (const Ptr& x : ptrs)
        if (reinterpret_cast<uintptr_t>(x.p) % 16 != 0)
            return fail(RSU_E_ALIGN, "%s: %s is not 16-byte aligned", fn, x.name);
    return RSU_OK;
}

int launched(hipError_t e, const char* fn) {
    if (e != hipSuccess) return fail(RSU_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return RSU_OK;
}

rsu::StepArgs step_args(int heads, float* S, const void* q, const void* k, const void* v,
                        const float* gate, const float* beta, float* y) {
    rsu::StepArgs a;
    a.heads = heads;
    a.S = S;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gate = gate;
    a.beta = beta;
    a.y = y;
    return a;
}

// The update kinds: scalar gate with the delta rule (GDN), per-key gate with the delta
// rule (KDA), per-key decay without it (RWKV6: no beta).
enum class Kind { gdn, kda, rwkv6 };
const char* gate_name(Kind m) { return m == Kind::gdn ? "alpha" : m == Kind::kda ? "d" : "w"; }

int dense_common(const char* fn, Kind m, const rsu_dims* dims, float* S, const void* q,
                 const void* k, const void* v, const float* gate, const float* beta, float* y,
                 rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {q, "q"}, {k, "k"}, {v, "v"}, {gate, gate_name(m)}, {y, "y"}}, fn))
        return rc;
    if (m != Kind::rwkv6)
        if (int rc = check_ptrs({{beta, "beta"}}, fn)) return rc;
    const rsu::StepArgs a = step_args(heads, S, q, k, v, gate, beta, y);
    const bool bf16 = dims->qkv_dtype == RSU_BF16;
    return launched(m == Kind::rwkv6 ? rsu::launch_rwkv6(a, bf16, stream)
                                     : rsu::launch_dense(a, m == Kind::kda, bf16, stream),
                    fn);
}

int window_common(const char* fn, bool per_key, const rsu_dims* dims, int W, int pos, int8_t* Z,
                  float* A, void* Kbuf, float* Ubuf, float* Gbuf, const void* q, const void* k,
                  const void* v, const float* gate, const float* beta, float* y,
                  rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (W < 1 || W > rsu::kMaxW) return fail(RSU_E_RANGE, "%s: W=%d outside [1, %d]", fn, W, rsu::kMaxW);
    if (pos < 0 || pos >= W) return fail(RSU_E_RANGE, "%s: pos=%d outside [0, W=%d)", fn, pos, W);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {A, "row_absmax"}, {Kbuf, "Kbuf"}, {Ubuf, "Ubuf"},
                             {Gbuf, "Gbuf"}, {q, "q"}, {k, "k"}, {v, "v"},
                             {gate, per_key ? "d" : "alpha"}, {beta, "beta"}, {y, "y"}}, fn))
        return rc;
    rsu::WindowArgs w;
    w.W = W;
    w.pos = pos;
    w.Z = Z;
    w.A = A;
    w.Kbuf = Kbuf;
    w.Ubuf = Ubuf;
    w.Gbuf = Gbuf;
    return launched(rsu::launch_q8_window(step_args(heads, nullptr, q, k, v, gate, beta, y), w,
                                          per_key, dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

// mode: 0 append, 1 merge, 2 per-slot live lengths (L ignored, Lslot used)
int log_common(const char* fn, Kind m, int mode, const rsu_dims* dims, int C, int L,
               int* Lslot, float* Sbase, float* lbar, void* Klog, void* Ulog, float* Lam,
               const void* q, const void* k, const void* v, const float* gate, const float* beta,
               float* y, rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (C < 0 || C > rsu::kMaxC) return fail(RSU_E_RANGE, "%s: C=%d outside [0, %d]", fn, C, rsu::kMaxC);
    if (mode == 1 && L != C) return fail(RSU_E_RANGE, "%s: merge needs L == C, got L=%d C=%d", fn, L, C);
    if (mode == 0 && (L < 0 || L >= C))
        return fail(RSU_E_RANGE, "%s: append needs 0 <= L < C, got L=%d C=%d", fn, L, C);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Sbase, "Sbase"}, {lbar, "lbar"}, {q, "q"}, {k, "k"}, {v, "v"},
                             {gate, gate_name(m)}, {y, "y"}}, fn))
        return rc;
    if (m != Kind::rwkv6)
        if (int rc = check_ptrs({{beta, "beta"}}, fn)) return rc;
    if (C > 0)
        if (int rc = check_ptrs({{Klog, "Klog"}, {Ulog, "Ulog"}, {Lam, "Lam"}}, fn)) return rc;
    if (mode == 2)
        if (int rc = check_ptrs({{Lslot, "L"}}, fn)) return rc;
    rsu::LogArgs l;
    l.C = C;
    l.L = mode == 2 ? 0 : L;
    l.Lslot = Lslot;
    l.lbar = lbar;
    l.Klog = Klog;
    l.Ulog = Ulog;
    l.Lam = Lam;
    const rsu::StepArgs a = step_args(heads, Sbase, q, k, v, gate, beta, y);
    const bool bf16 = dims->qkv_dtype == RSU_BF16;
    return launched(m == Kind::rwkv6 ? rsu::launch_rwkv6_log(a, l, mode, bf16, stream)
                                     : rsu::launch_log(a, l, mode, m == Kind::kda, bf16, stream),
                    fn);
}

int lq_quantize_common(const char* fn, const rsu_dims* dims, const float* S, int n_iter, int8_t* Z,
                       float* col_absmax, float* row_smooth, void* Kc, void* Uc, rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (n_iter < 0 || n_iter > 64) return fail(RSU_E_RANGE, "%s: n_iter=%d outside [0, 64]", fn, n_iter);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {Z, "Z"}, {col_absmax, "col_absmax"}, {row_smooth, "row_smooth"},
                             {Kc, "Kc"}, {Uc, "Uc"}}, fn))
        return rc;
    return launched(rsu::launch_lq_quantize(heads, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream), fn);
}

int lq_low_quantize_common(const char* fn, int bits, const rsu_dims* dims, const float* S, int n_iter, void* Z,
                           float* col_absmax, float* row_smooth, void* Kc, void* Uc, rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (n_iter < 0 || n_iter > 64) return fail(RSU_E_RANGE, "%s: n_iter=%d outside [0, 64]", fn, n_iter);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {Z, "Z"}, {col_absmax, "col_absmax"}, {row_smooth, "row_smooth"},
                             {Kc, "Kc"}, {Uc, "Uc"}}, fn))
        return rc;
    return launched(rsu::launch_lq_low_quantize(bits, heads, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream),
                    fn);
}

int lq_window_common(const char* fn, Kind m, const rsu_dims* dims, int W, int pos, int n_iter, int8_t* Z,
                     float* col_absmax, float* row_smooth, void* Kc, void* Uc, void* Kbuf, float* Ubuf,
                     float* Gbuf, const void* q, const void* k, const void* v, const float* gate,
                     const float* beta, float* y, rsu_stream_t stream, int bits = 8) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (dims->qkv_dtype != RSU_BF16)
        return fail(RSU_E_DTYPE, "%s: only bf16 q/k/v are supported (the keys enter the MFMA exactly)", fn);
    if (W < 1 || W > 16) return fail(RSU_E_RANGE, "%s: W=%d outside [1, 16]", fn, W);
    if (pos < 0 || pos >= W) return fail(RSU_E_RANGE, "%s: pos=%d outside [0, W)", fn, pos);
    if (n_iter < 0 || n_iter > 64) return fail(RSU_E_RANGE, "%s: n_iter=%d outside [0, 64]", fn, n_iter);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {col_absmax, "col_absmax"}, {row_smooth, "row_smooth"}, {Kc, "Kc"},
                             {Uc, "Uc"}, {Kbuf, "Kbuf"}, {Ubuf, "Ubuf"}, {Gbuf, "Gbuf"}, {q, "q"}, {k, "k"},
                             {v, "v"}, {gate, gate_name(m)}, {beta, "beta"}, {y, "y"}}, fn))
        return rc;
    rsu::LqArgs w;
    w.W = W;
    w.pos = pos;
    w.n_iter = n_iter;
    w.Z = Z;
    w.B = col_absmax;
    w.C = row_smooth;
    w.Kc = Kc;
    w.Uc = Uc;
    w.Kbuf = Kbuf;
    w.Ubuf = Ubuf;
    w.Gbuf = Gbuf;
    const rsu::StepArgs a = step_args(heads, nullptr, q, k, v, gate, beta, y);
    if (bits != 8) return launched(rsu::launch_lq_low_window(bits, a, w, m == Kind::kda, stream), fn);
    return launched(rsu::launch_lq_window(a, w, m == Kind::kda, stream), fn);
}

int stepq_step_common(const char* fn, Kind m, const rsu_dims* dims, void* Z, void* R, void* C, const float* omega,
                      const void* q, const void* k, const void* v, const float* gate, const float* beta, float* y,
                      rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {R, "R"}, {C, "C"}, {omega, "omega"}, {q, "q"}, {k, "k"}, {v, "v"},
                             {gate, gate_name(m)}, {beta, "beta"}, {y, "y"}}, fn))
        return rc;
    return launched(rsu::launch_sq_step(step_args(heads, nullptr, q, k, v, gate, beta, y), 0, Z, R, C, omega,
                                        nullptr, m == Kind::kda, dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int stepq_readout_common(const char* fn, Kind m, const rsu_dims* dims, const void* Z, const void* R, const void* C,
                         const void* q, const void* k, const void* v, const float* gate, const float* beta,
                         float* u, float* y, rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {R, "R"}, {C, "C"}, {q, "q"}, {k, "k"}, {v, "v"}, {gate, gate_name(m)},
                             {beta, "beta"}, {u, "u"}, {y, "y"}}, fn))
        return rc;
    return launched(rsu::launch_sq_step(step_args(heads, nullptr, q, k, v, gate, beta, y), 1, const_cast<void*>(Z),
                                        const_cast<void*>(R), const_cast<void*>(C), nullptr, u, m == Kind::kda,
                                        dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int stepq_repack_common(const char* fn, Kind m, const rsu_dims* dims, void* Z, void* R, void* C, const float* omega,
                        const void* k, const float* gate, const float* u, rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {R, "R"}, {C, "C"}, {omega, "omega"}, {k, "k"}, {gate, gate_name(m)},
                             {u, "u"}}, fn))
        return rc;
    return launched(rsu::launch_sq_step(step_args(heads, nullptr, nullptr, k, nullptr, gate, nullptr, nullptr), 2, Z,
                                        R, C, omega, const_cast<float*>(u), m == Kind::kda,
                                        dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

}  // namespace

extern "C" {

int rsu_abi_version(void) { return 1; }

const char* rsu_last_error(void) { return g_err; }

int gdn_decode_step(const rsu_dims* dims, float* S, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return dense_common("gdn_decode_step", Kind::gdn, dims, S, q, k, v, alpha, beta, y, stream);
}

int kda_decode_step(const rsu_dims* dims, float* S, const void* q, const void* k, const void* v,
                    const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return dense_common("kda_decode_step", Kind::kda, dims, S, q, k, v, d, beta, y, stream);
}

int q8_quantize(const rsu_dims* dims, const float* S, int8_t* Z, float* row_absmax,
                rsu_stream_t stream) {
    int heads = 0;
    if (int rc = check_dims(dims, &heads, "q8_quantize")) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {Z, "Z"}, {row_absmax, "row_absmax"}}, "q8_quantize")) return rc;
    return launched(rsu::launch_q8_quantize(heads, S, Z, row_absmax, stream), "q8_quantize");
}

int gdn_q8_window(const rsu_dims* dims, int W, int pos, int8_t* Z, float* row_absmax, void* Kbuf,
                  float* Ubuf, float* Gbuf, const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return window_common("gdn_q8_window", false, dims, W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k,
                         v, alpha, beta, y, stream);
}

int kda_q8_window(const rsu_dims* dims, int W, int pos, int8_t* Z, float* row_absmax, void* Kbuf,
                  float* Ubuf, float* Gbuf, const void* q, const void* k, const void* v,
                  const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return window_common("kda_q8_window", true, dims, W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k,
                         v, d, beta, y, stream);
}

int gdn_log_append(const rsu_dims* dims, int C, int L, const float* Sbase, float* lbar, void* Klog,
                   float* Ulog, float* Lam, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("gdn_log_append", Kind::gdn, 0, dims, C, L, nullptr, const_cast<float*>(Sbase), lbar,
                      Klog, Ulog, Lam, q, k, v, alpha, beta, y, stream);
}

int kda_log_append(const rsu_dims* dims, int C, int L, const float* Sbase, float* lbar, void* Klog,
                   float* Ulog, float* Lam, const void* q, const void* k, const void* v,
                   const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("kda_log_append", Kind::kda, 0, dims, C, L, nullptr, const_cast<float*>(Sbase), lbar,
                      Klog, Ulog, Lam, q, k, v, d, beta, y, stream);
}

int gdn_log_merge(const rsu_dims* dims, int C, int L, float* Sbase, float* lbar, const void* Klog,
                  const float* Ulog, const float* Lam, const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("gdn_log_merge", Kind::gdn, 1, dims, C, L, nullptr, Sbase, lbar, const_cast<void*>(Klog),
                      const_cast<float*>(Ulog), const_cast<float*>(Lam), q, k, v, alpha, beta, y,
                      stream);
}

int kda_log_merge(const rsu_dims* dims, int C, int L, float* Sbase, float* lbar, const void* Klog,
                  const float* Ulog, const float* Lam, const void* q, const void* k, const void* v,
                  const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("kda_log_merge", Kind::kda, 1, dims, C, L, nullptr, Sbase, lbar, const_cast<void*>(Klog),
                      const_cast<float*>(Ulog), const_cast<float*>(Lam), q, k, v, d, beta, y, stream);
}

int gdn_lq_quantize(const rsu_dims* dims, const float* S, int n_iter, int8_t* Z, float* col_absmax,
                    float* row_smooth, void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_quantize_common("gdn_lq_quantize", dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int kda_lq_quantize(const rsu_dims* dims, const float* S, int n_iter, int8_t* Z, float* col_absmax,
                    float* row_smooth, void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_quantize_common("kda_lq_quantize", dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int gdn_lq4_quantize(const rsu_dims* dims, const float* S, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                     void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_low_quantize_common("gdn_lq4_quantize", 4, dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int gdn_lq6_quantize(const rsu_dims* dims, const float* S, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                     void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_low_quantize_common("gdn_lq6_quantize", 6, dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int kda_lq4_quantize(const rsu_dims* dims, const float* S, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                     void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_low_quantize_common("kda_lq4_quantize", 4, dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int kda_lq6_quantize(const rsu_dims* dims, const float* S, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                     void* Kc, void* Uc, rsu_stream_t stream) {
    return lq_low_quantize_common("kda_lq6_quantize", 6, dims, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, stream);
}

int kda_lq4_window(const rsu_dims* dims, int W, int pos, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                   void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf, const void* q, const void* k,
                   const void* v, const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return lq_window_common("kda_lq4_window", Kind::kda, dims, W, pos, n_iter, static_cast<int8_t*>(Z), col_absmax,
                            row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y, stream, 4);
}

int kda_lq6_window(const rsu_dims* dims, int W, int pos, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                   void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf, const void* q, const void* k,
                   const void* v, const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return lq_window_common("kda_lq6_window", Kind::kda, dims, W, pos, n_iter, static_cast<int8_t*>(Z), col_absmax,
                            row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y, stream, 6);
}

int gdn_lq6_window(const rsu_dims* dims, int W, int pos, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                   void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return lq_window_common("gdn_lq6_window", Kind::gdn, dims, W, pos, n_iter, static_cast<int8_t*>(Z), col_absmax,
                            row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y, stream, 6);
}

int gdn_lq4_window(const rsu_dims* dims, int W, int pos, int n_iter, void* Z, float* col_absmax, float* row_smooth,
                   void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return lq_window_common("gdn_lq4_window", Kind::gdn, dims, W, pos, n_iter, static_cast<int8_t*>(Z), col_absmax,
                            row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y, stream, 4);
}

int gdn_lq_window(const rsu_dims* dims, int W, int pos, int n_iter, int8_t* Z, float* col_absmax,
                  float* row_smooth, void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf,
                  const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                  float* y, rsu_stream_t stream) {
    return lq_window_common("gdn_lq_window", Kind::gdn, dims, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc,
                            Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y, stream);
}

int kda_lq_window(const rsu_dims* dims, int W, int pos, int n_iter, int8_t* Z, float* col_absmax,
                  float* row_smooth, void* Kc, void* Uc, void* Kbuf, float* Ubuf, float* Gbuf,
                  const void* q, const void* k, const void* v, const float* d, const float* beta,
                  float* y, rsu_stream_t stream) {
    return lq_window_common("kda_lq_window", Kind::kda, dims, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc,
                            Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y, stream);
}

int gdn_log_step_slots(const rsu_dims* dims, int C, int* L, float* Sbase, float* lbar, void* Klog,
                       float* Ulog, float* Lam, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("gdn_log_step_slots", Kind::gdn, 2, dims, C, 0, L, Sbase, lbar, Klog, Ulog, Lam, q, k,
                      v, alpha, beta, y, stream);
}

int kda_log_step_slots(const rsu_dims* dims, int C, int* L, float* Sbase, float* lbar, void* Klog,
                       float* Ulog, float* Lam, const void* q, const void* k, const void* v,
                       const float* d, const float* beta, float* y, rsu_stream_t stream) {
    return log_common("kda_log_step_slots", Kind::kda, 2, dims, C, 0, L, Sbase, lbar, Klog, Ulog, Lam, q, k,
                      v, d, beta, y, stream);
}

int rwkv6_decode_step(const rsu_dims* dims, float* S, const void* q, const void* k, const void* v,
                      const float* w, float* y, rsu_stream_t stream) {
    return dense_common("rwkv6_decode_step", Kind::rwkv6, dims, S, q, k, v, w, nullptr, y, stream);
}

int rwkv7_decode_step(const rsu_dims* dims, float* S, const void* q, const void* k, const void* v,
                      const void* kappa, const float* w, const float* a, float* y, rsu_stream_t stream) {
    const char* fn = "rwkv7_decode_step";
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {q, "q"}, {k, "k"}, {v, "v"}, {kappa, "kappa"}, {w, "w"}, {a, "a"},
                             {y, "y"}}, fn))
        return rc;
    return launched(rsu::launch_rwkv7(step_args(heads, S, q, k, v, w, nullptr, y), kappa, a,
                                      dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int rwkv7_q8_window(const rsu_dims* dims, int W, int pos, int8_t* Z, float* row_absmax, void* Kbuf, float* Ubuf,
                    float* Gbuf, const void* q, const void* k, const void* v, const void* kappa, const float* w,
                    const float* a, float* y, rsu_stream_t stream) {
    const char* fn = "rwkv7_q8_window";
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (W < 1 || W > 16) return fail(RSU_E_RANGE, "%s: W=%d outside [1, 16] (two records per token)", fn, W);
    if (pos < 0 || pos >= W) return fail(RSU_E_RANGE, "%s: pos=%d outside [0, W=%d)", fn, pos, W);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {row_absmax, "row_absmax"}, {Kbuf, "Kbuf"}, {Ubuf, "Ubuf"}, {Gbuf, "Gbuf"},
                             {q, "q"}, {k, "k"}, {v, "v"}, {kappa, "kappa"}, {w, "w"}, {a, "a"}, {y, "y"}}, fn))
        return rc;
    rsu::WindowArgs wa;
    wa.W = W;
    wa.pos = pos;
    wa.Z = Z;
    wa.A = row_absmax;
    wa.Kbuf = Kbuf;
    wa.Ubuf = Ubuf;
    wa.Gbuf = Gbuf;
    return launched(rsu::launch_rwkv7_q8_window(step_args(heads, nullptr, q, k, v, w, nullptr, y), wa, kappa, a,
                                                dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int rwkv6_log_append(const rsu_dims* dims, int C, int L, const float* Sbase, float* lbar, void* Klog,
                     void* Ulog, float* Lam, const void* q, const void* k, const void* v, const float* w,
                     float* y, rsu_stream_t stream) {
    return log_common("rwkv6_log_append", Kind::rwkv6, 0, dims, C, L, nullptr, const_cast<float*>(Sbase),
                      lbar, Klog, Ulog, Lam, q, k, v, w, nullptr, y, stream);
}

int rwkv6_log_merge(const rsu_dims* dims, int C, int L, float* Sbase, float* lbar, const void* Klog,
                    const void* Ulog, const float* Lam, const void* q, const void* k, const void* v,
                    const float* w, float* y, rsu_stream_t stream) {
    return log_common("rwkv6_log_merge", Kind::rwkv6, 1, dims, C, L, nullptr, Sbase, lbar,
                      const_cast<void*>(Klog), const_cast<void*>(Ulog), const_cast<float*>(Lam), q, k, v,
                      w, nullptr, y, stream);
}

int rwkv6_log_step_slots(const rsu_dims* dims, int C, int* L, float* Sbase, float* lbar, void* Klog,
                         void* Ulog, float* Lam, const void* q, const void* k, const void* v, const float* w,
                         float* y, rsu_stream_t stream) {
    return log_common("rwkv6_log_step_slots", Kind::rwkv6, 2, dims, C, 0, L, Sbase, lbar, Klog, Ulog, Lam, q,
                      k, v, w, nullptr, y, stream);
}

int deltaproduct_decode_step(const rsu_dims* dims, int n, float* S, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, float* y, rsu_stream_t stream) {
    const char* fn = "deltaproduct_decode_step";
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (n < 1 || n > 4) return fail(RSU_E_RANGE, "%s: n=%d outside [1, 4]", fn, n);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {q, "q"}, {k, "k"}, {v, "v"}, {alpha, "alpha"}, {beta, "beta"}, {y, "y"}}, fn))
        return rc;
    return launched(rsu::launch_deltaproduct(step_args(heads, S, q, k, v, alpha, beta, y), n,
                                             dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int deltaproduct_q8_window(const rsu_dims* dims, int n, int W, int pos, int8_t* Z, float* row_absmax, void* Kbuf,
                           float* Ubuf, float* Gbuf, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, float* y, rsu_stream_t stream) {
    const char* fn = "deltaproduct_q8_window";
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (n < 1 || n > 4) return fail(RSU_E_RANGE, "%s: n=%d outside [1, 4]", fn, n);
    if (W < 1 || n * W > rsu::kMaxW)
        return fail(RSU_E_RANGE, "%s: W=%d with n=%d: need 1 <= W and n W <= %d", fn, W, n, rsu::kMaxW);
    if (pos < 0 || pos >= W) return fail(RSU_E_RANGE, "%s: pos=%d outside [0, W=%d)", fn, pos, W);
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{Z, "Z"}, {row_absmax, "row_absmax"}, {Kbuf, "Kbuf"}, {Ubuf, "Ubuf"}, {Gbuf, "Gbuf"},
                             {q, "q"}, {k, "k"}, {v, "v"}, {alpha, "alpha"}, {beta, "beta"}, {y, "y"}}, fn))
        return rc;
    rsu::WindowArgs wa;
    wa.W = W;
    wa.pos = pos;
    wa.Z = Z;
    wa.A = row_absmax;
    wa.Kbuf = Kbuf;
    wa.Ubuf = Ubuf;
    wa.Gbuf = Gbuf;
    return launched(rsu::launch_dp_q8_window(step_args(heads, nullptr, q, k, v, alpha, beta, y), wa, n,
                                             dims->qkv_dtype == RSU_BF16, stream),
                    fn);
}

int rsu_copy_f32(const float* src, float* dst, int64_t n, rsu_stream_t stream) {
    g_err[0] = '\0';
    if (n < 0 || n % 4 != 0) return fail(RSU_E_DIMS, "rsu_copy_f32: n=%lld must be a multiple of 4", (long long)n);
    if (n / (128 * 128) >= 0x7fffffffLL) return fail(RSU_E_DIMS, "rsu_copy_f32: n too large");
    if (n == 0) return RSU_OK;
    if (int rc = check_ptrs({{src, "src"}, {dst, "dst"}}, "rsu_copy_f32")) return rc;
    return launched(rsu::launch_copy(src, dst, n, stream), "rsu_copy_f32");
}

int rsu_read_f32(const float* src, float* col_sums, int64_t tiles, rsu_stream_t stream) {
    g_err[0] = '\0';
    if (tiles < 0 || tiles > 0x7fffffffLL) return fail(RSU_E_DIMS, "rsu_read_f32: tiles=%lld out of range", (long long)tiles);
    if (tiles == 0) return RSU_OK;
    if (int rc = check_ptrs({{src, "src"}, {col_sums, "col_sums"}}, "rsu_read_f32")) return rc;
    return launched(rsu::launch_read_probe(src, col_sums, static_cast<int>(tiles), stream), "rsu_read_f32");
}

int rsu_fill_f32(float* dst, float value, int64_t tiles, rsu_stream_t stream) {
    g_err[0] = '\0';
    if (tiles < 0 || tiles > 0x7fffffffLL) return fail(RSU_E_DIMS, "rsu_fill_f32: tiles=%lld out of range", (long long)tiles);
    if (tiles == 0) return RSU_OK;
    if (int rc = check_ptrs({{dst, "dst"}}, "rsu_fill_f32")) return rc;
    return launched(rsu::launch_write_probe(dst, value, static_cast<int>(tiles), stream), "rsu_fill_f32");
}

int rsu_debug_metadata_counts(uint32_t* counts, int64_t heads, rsu_stream_t stream) {
    const char* fn = "rsu_debug_metadata_counts";
    g_err[0] = '\0';
    if (!counts) return fail(RSU_E_NULL, "%s: counts is NULL", fn);
    if (heads < 0 || heads > rsu::kMetaCheckHeads)
        return fail(RSU_E_RANGE, "%s: heads=%lld outside 0..%d", fn, (long long)heads, rsu::kMetaCheckHeads);
    const hipError_t e = rsu::read_metadata_counts(counts, heads, stream);
    if (e == hipErrorNotSupported)
        return fail(RSU_E_UNSUPPORTED, "%s: this library was built without RSU_CHECK_METADATA", fn);
    if (e != hipSuccess) return fail(RSU_E_HIP, "%s: %s", fn, hipGetErrorString(e));
    return RSU_OK;
}

int stepq_pack(const rsu_dims* dims, const float* S, const float* omega, void* Z, void* R, void* C,
               rsu_stream_t stream) {
    const char* fn = "stepq_pack";
    int heads = 0;
    if (int rc = check_dims(dims, &heads, fn)) return rc;
    if (heads == 0) return RSU_OK;
    if (int rc = check_ptrs({{S, "S"}, {omega, "omega"}, {Z, "Z"}, {R, "R"}, {C, "C"}}, fn)) return rc;
    return launched(rsu::launch_sq_pack(heads, S, omega, Z, R, C, stream), fn);
}

int gdn_stepq_step(const rsu_dims* dims, void* Z, void* R, void* C, const float* omega, const void* q,
                   const void* k, const void* v, const float* alpha, const float* beta, float* y,
                   rsu_stream_t stream) {
    return stepq_step_common("gdn_stepq_step", Kind::gdn, dims, Z, R, C, omega, q, k, v, alpha, beta, y, stream);
}

int kda_stepq_step(const rsu_dims* dims, void* Z, void* R, void* C, const float* omega, const void* q,
                   const void* k, const void* v, const float* d, const float* beta, float* y,
                   rsu_stream_t stream) {
    return stepq_step_common("kda_stepq_step", Kind::kda, dims, Z, R, C, omega, q, k, v, d, beta, y, stream);
}

int gdn_stepq_readout(const rsu_dims* dims, const void* Z, const void* R, const void* C, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta, float* u, float* y,
                      rsu_stream_t stream) {
    return stepq_readout_common("gdn_stepq_readout", Kind::gdn, dims, Z, R, C, q, k, v, alpha, beta, u, y, stream);
}

int kda_stepq_readout(const rsu_dims* dims, const void* Z, const void* R, const void* C, const void* q,
                      const void* k, const void* v, const float* d, const float* beta, float* u, float* y,
                      rsu_stream_t stream) {
    return stepq_readout_common("kda_stepq_readout", Kind::kda, dims, Z, R, C, q, k, v, d, beta, u, y, stream);
}

int gdn_stepq_repack(const rsu_dims* dims, void* Z, void* R, void* C, const float* omega, const void* k,
                     const float* alpha, const float* u, rsu_stream_t stream) {
    return stepq_repack_common("gdn_stepq_repack", Kind::gdn, dims, Z, R, C, omega, k, alpha, u, stream);
}

int kda_stepq_repack(const rsu_dims* dims, void* Z, void* R, void* C, const float* omega, const void* k,
                     const float* d, const float* u, rsu_stream_t stream) {
    return stepq_repack_common("kda_stepq_repack", Kind::kda, dims, Z, R, C, omega, k, d, u, stream);
}

}  // extern "C"
