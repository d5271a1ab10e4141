/*
 * rsu_oracle.c -- plain, slow, fp64 CPU reference of the delta-rule decode step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline use this file. It shares no code, header or constant with the HIP
 * library and includes none of it. Loops are written out plainly, one head at a
 * time (OpenMP only spreads independent heads over cores).
 *
 * Notation (LeapQuant, sec. 3.1 and App. A; STEPQuant notes, "from linear
 * attention to the delta rule"): per head the state S is d_k x d_v, row i is a
 * key channel, column j a value channel. g is the retention gate: a scalar alpha
 * repeated over the key channels (Gated DeltaNet) or a per-key vector d (Kimi
 * Delta Attention). beta in [0,1] is the scalar write strength.
 *
 * All arrays are row-major and contiguous:
 *   S[nh][dk][dv], q,k[nh][dk], v,y[nh][dv], gate[nh] or [nh][dk], beta[nh].
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IDX2(i, j, n2) ((size_t)(i) * (size_t)(n2) + (size_t)(j))

/* threads the oracle spreads heads over */
int oracle_num_threads(void) { return omp_get_max_threads(); }

static double gate_at(const double *gate_h, int per_key, int i)
{
    return per_key ? gate_h[i] : gate_h[0];
}

/*
 * One decode step, eager dense form (LeapQuant, App. A, the GDN and KDA
 * expansions, right-hand sides; STEPQuant notes: the step output is read after
 * the update):
 *   S' = Diag(g) S                 decay
 *   p  = S'^T k                    old value read along k, from the decayed state
 *   u  = beta (v - p)              correction, beta carried by u (App. A)
 *   S  = S' + k u^T                rank-one delta write
 *   y  = S^T q                     readout from the post-update state
 */
void oracle_dense_step(int64_t nh, int dk, int dv, int per_key, double *S,
                       const double *q, const double *k, const double *v,
                       const double *gate, const double *beta, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        double *Sh = S + (size_t)h * dk * dv;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk;
        const double *vh = v + (size_t)h * dv;
        const double *gh = gate + (per_key ? (size_t)h * dk : (size_t)h);
        double *yh = y + (size_t)h * dv;
        double *u = (double *)malloc(sizeof(double) * dv);

        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sh[IDX2(i, j, dv)] *= gate_at(gh, per_key, i);
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i)
                p += Sh[IDX2(i, j, dv)] * kh[i];
            u[j] = beta[h] * (vh[j] - p);
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sh[IDX2(i, j, dv)] += kh[i] * u[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += Sh[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        free(u);
    }
}

/*
 * One RWKV6 decode step in the common form the pages use (DeltaLog, Table 1, the
 * RWKV6 row: state transform D(lambda_t) S_{t-1}, update pair (k_t, v_t), diagonal
 * decay; LeapQuant, App. A, eq. 1 with read vector b_t = 0 and output o_t = S_t^T q_t).
 * w is the per-key decay factor (w = exp(lambda)); there is no delta read and no beta:
 *   S = Diag(w) S + k v^T,   y = S^T q
 */
void oracle_rwkv6_step(int64_t nh, int dk, int dv, double *S, const double *q, const double *k,
                       const double *v, const double *w, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        double *Sh = S + (size_t)h * dk * dv;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk;
        const double *vh = v + (size_t)h * dv, *wh = w + (size_t)h * dk;
        double *yh = y + (size_t)h * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sh[IDX2(i, j, dv)] = wh[i] * Sh[IDX2(i, j, dv)] + kh[i] * vh[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += Sh[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
    }
}

/*
 * One RWKV7 decode step as two sub-steps of the general update (LeapQuant, App. A,
 * "models with a separate erase direction": the transition Diag(w) - kappa (a * kappa)^T
 * splits into an erase with v = 0 and a pure write with D = I and read vector 0):
 *   S' = Diag(w) S + kappa (0 - S^T (a * kappa))^T      erase along kappa, read with a * kappa
 *   S  = S' + k v^T                                       write
 *   y  = S^T q
 * w is the per-key decay, kappa the removal key, a the per-key erase rate.
 */
void oracle_rwkv7_step(int64_t nh, int dk, int dv, double *S, const double *q, const double *k,
                       const double *v, const double *w, const double *kappa, const double *a,
                       double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        double *Sh = S + (size_t)h * dk * dv;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk;
        const double *vh = v + (size_t)h * dv, *wh = w + (size_t)h * dk;
        const double *ch = kappa + (size_t)h * dk, *ah = a + (size_t)h * dk;
        double *yh = y + (size_t)h * dv;
        double *u = (double *)malloc(sizeof(double) * dv);
        for (int j = 0; j < dv; ++j) {          /* erase: u = 0 - S^T (a * kappa) */
            double p = 0.0;
            for (int i = 0; i < dk; ++i)
                p += Sh[IDX2(i, j, dv)] * ah[i] * ch[i];
            u[j] = 0.0 - p;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sh[IDX2(i, j, dv)] = wh[i] * Sh[IDX2(i, j, dv)] + ch[i] * u[j];
        for (int i = 0; i < dk; ++i)            /* write */
            for (int j = 0; j < dv; ++j)
                Sh[IDX2(i, j, dv)] += kh[i] * vh[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += Sh[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        free(u);
    }
}

/*
 * One DeltaProduct token with n delta-rule sub-steps (LeapQuant, App. A: Table 4 lists
 * DeltaProduct as n sub-steps of eq. 1 per token). Sub-step i (0-based) has its own key
 * k_i, value v_i and strength beta_i; the token's scalar gate alpha decays the state once,
 * in the first sub-step:
 *   S' = d_i S,  d_0 = alpha, d_i = 1 for i > 0      decay
 *   u_i = beta_i (v_i - S'^T k_i)                      read along k_i from the decayed state
 *   S  = S' + k_i u_i^T                                rank-one delta write
 * and after the n sub-steps y = S^T q.
 * k[nh][n][dk], v[nh][n][dv], beta[nh][n], alpha[nh].
 */
void oracle_deltaproduct_step(int64_t nh, int dk, int dv, int n, double *S, const double *q,
                              const double *k, const double *v, const double *alpha,
                              const double *beta, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        double *Sh = S + (size_t)h * dk * dv;
        const double *qh = q + (size_t)h * dk;
        double *yh = y + (size_t)h * dv;
        double *u = (double *)malloc(sizeof(double) * dv);
        for (int s = 0; s < n; ++s) {
            const double *ks = k + ((size_t)h * n + s) * dk;
            const double *vs = v + ((size_t)h * n + s) * dv;
            const double bs = beta[(size_t)h * n + s];
            const double d = s == 0 ? alpha[h] : 1.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    Sh[IDX2(i, j, dv)] *= d;
            for (int j = 0; j < dv; ++j) {
                double p = 0.0;
                for (int i = 0; i < dk; ++i)
                    p += Sh[IDX2(i, j, dv)] * ks[i];
                u[j] = bs * (vs[j] - p);
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    Sh[IDX2(i, j, dv)] += ks[i] * u[j];
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += Sh[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        free(u);
    }
}

/*
 * Symmetric per-key-row int8 quantizer (STEPQuant notes, the uniform per-row
 * absmax baseline; LeapQuant, App. B.3, the /127 convention).
 *   a_i = max_j |S_ij|          stored as fp32
 *   z_ij = clamp(rne(S_ij * (127 / a_i)), -127, 127)   and z = 0 when a_i = 0
 *   dequant(z, a)_ij = z_ij * a_i / 127
 * The code is an integer decided by floating point, so the decision is taken in
 * fp32 exactly as the device does it: the value is first rounded to fp32, the
 * reciprocal scale 127/a_i is one correctly rounded fp32 division, the product
 * one fp32 multiplication, the rounding to nearest with ties to even.
 * A row whose maximum is below 2^-64 (where 127/a_i can overflow fp32: a
 * subnormal or nearly subnormal row) is first scaled by 2^64, which is exact for
 * its values and its maximum, and the same decision is taken on the scaled row;
 * a_i is stored unscaled. (The pages are silent on such rows; this keeps the
 * codes those of rne(S_ij * 127 / a_i) instead of saturating them.)
 * If w_out is not NULL it receives the exact pre-rounding code S_ij*127/a_i in
 * fp64 (used to find elements near a rounding tie).
 */
void oracle_q8_quantize(int64_t nrows, int ncols, const double *X, int8_t *Z, float *a,
                        double *w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const double *x = X + (size_t)r * ncols;
        float amax = 0.0f;
        for (int j = 0; j < ncols; ++j) {
            float xf = fabsf((float)x[j]);
            if (xf > amax)
                amax = xf;
        }
        const float f = amax < 0x1p-64f ? 0x1p64f : 1.0f;
        volatile float num = 127.0f;
        float scale = amax > 0.0f ? num / (amax * f) : 0.0f;
        a[r] = amax;
        for (int j = 0; j < ncols; ++j) {
            volatile float xs = (float)x[j] * f; /* exact */
            float w = xs * scale;
            float zr = rintf(w);
            if (zr > 127.0f)
                zr = 127.0f;
            if (zr < -127.0f)
                zr = -127.0f;
            Z[(size_t)r * ncols + j] = (int8_t)zr;
            if (w_out)
                w_out[(size_t)r * ncols + j] = amax > 0.0f ? x[j] * 127.0 / (double)amax : 0.0;
        }
    }
}

/* dequant of one head's int8 state (App. B.3 with per-row scales) */
static void dequant_head(int dk, int dv, const int8_t *Z, const float *a, double *out)
{
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            out[IDX2(i, j, dv)] = (double)Z[IDX2(i, j, dv)] * (double)a[i] / 127.0;
}

/*
 * Gamma_{from:to} for key channel i, with 0-based record indices: the product of
 * the gates of records from..to (inclusive); the empty product is 1 (LeapQuant,
 * sec. 3.2, the cumulative decay).
 */
static double window_gamma(const double *G, int per_key, int dk, int from, int to, int i)
{
    double g = 1.0;
    for (int m = from; m <= to; ++m)
        g *= per_key ? G[IDX2(m, i, dk)] : G[m];
    return g;
}

/*
 * S_l of eq. 4 (LeapQuant, sec. 3.2) for one head, from the fixed window-start
 * state and the first l records (0-based records 0..l-1):
 *   S_l = Gamma_{1:l} S0 + sum_{j=1..l} Gamma_{j+1:l} k_j u_j^T
 */
static void window_materialize(int dk, int dv, int per_key, int l, const double *S0,
                               const double *G, const double *K, const double *U, double *out)
{
    for (int i = 0; i < dk; ++i) {
        double g0 = window_gamma(G, per_key, dk, 0, l - 1, i);
        for (int j = 0; j < dv; ++j)
            out[IDX2(i, j, dv)] = g0 * S0[IDX2(i, j, dv)];
        for (int m = 0; m < l; ++m) {
            double c = window_gamma(G, per_key, dk, m + 1, l - 1, i) * K[IDX2(m, i, dk)];
            for (int j = 0; j < dv; ++j)
                out[IDX2(i, j, dv)] += c * U[IDX2(m, j, dv)];
        }
    }
}

/*
 * One step of per-window quantization (LeapQuant, sec. 3.2, eqs. 3-4; App. B.2).
 * The int8 state (Z, a) is the window-start state S^_0 and stays fixed inside
 * the window. Step pos (0-based; the page's l = pos + 1) buffers the record
 * (g_l, k_l, u_l) in higher precision:
 *   S_{l-1} from eq. 4,  u_l = beta (v - (Diag(g_l) S_{l-1})^T k_l)   (eq. 3, App. A)
 *   S_l     from eq. 4,  y = S_l^T q
 * and at the end of the window (l = W) S_W is quantized into the next window's
 * (Z, a) and the records are dropped (eq. 4, second line). The output of the
 * last step is read from the unquantized S_W (STEPQuant notes: the readout comes
 * before the quantization of the step).
 * Records: G[nh][W] (scalar gate) or G[nh][W][dk], K[nh][W][dk], U[nh][W][dv].
 * Sw_out, w_out (optional, boundary step only): S_W in fp64 and the pre-rounding codes.
 */
void oracle_q8_window_step(int64_t nh, int dk, int dv, int per_key, int W, int pos,
                           int8_t *Z, float *a, double *G, double *K, double *U,
                           const double *q, const double *k, const double *v,
                           const double *gate, const double *beta, double *y,
                           double *Sw_out, double *w_out)
{
    const int gdim = per_key ? dk : 1;
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        int8_t *Zh = Z + (size_t)h * dk * dv;
        float *ah = a + (size_t)h * dk;
        double *Gh = G + (size_t)h * W * gdim;
        double *Kh = K + (size_t)h * W * dk;
        double *Uh = U + (size_t)h * W * dv;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk;
        const double *vh = v + (size_t)h * dv;
        const double *gh = gate + (size_t)h * gdim;
        double *yh = y + (size_t)h * dv;
        const int l = pos + 1;

        double *S0 = (double *)malloc(sizeof(double) * dk * dv);
        double *St = (double *)malloc(sizeof(double) * dk * dv);
        dequant_head(dk, dv, Zh, ah, S0);

        /* the record's gate and key are known before its correction */
        for (int i = 0; i < gdim; ++i)
            Gh[IDX2(pos, i, gdim)] = gh[i];
        for (int i = 0; i < dk; ++i)
            Kh[IDX2(pos, i, dk)] = kh[i];

        /* correction from S_{l-1}, read along the decayed key */
        window_materialize(dk, dv, per_key, l - 1, S0, Gh, Kh, Uh, St);
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i)
                p += St[IDX2(i, j, dv)] * gate_at(gh, per_key, i) * kh[i];
            Uh[IDX2(pos, j, dv)] = beta[h] * (vh[j] - p);
        }

        /* readout from S_l */
        window_materialize(dk, dv, per_key, l, S0, Gh, Kh, Uh, St);
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += St[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }

        if (l == W) {
            if (Sw_out)
                memcpy(Sw_out + (size_t)h * dk * dv, St, sizeof(double) * dk * dv);
            oracle_q8_quantize(dk, dv, St, Zh, ah, w_out ? w_out + (size_t)h * dk * dv : NULL);
        }
        free(S0);
        free(St);
    }
}

/*
 * One RWKV7 token on the per-window int8 state. Each token is two records (LeapQuant,
 * App. A: an erase sub-step with D = Diag(w), key kappa, read vector a * kappa and v = 0,
 * then a write sub-step with D = I, key k and read vector 0), so a window of W tokens
 * buffers 2W records, erase_0, write_0, erase_1, ..., with gates w_0, 1, w_1, 1, ...;
 * eq. 4 over them is the same cumulative-decay sum as for one record per token.
 * Token pos (0-based) sees the 2 pos records before it:
 *   S_{t-1} = eq. 4 over records 0 .. 2pos-1
 *   u_e = 0 - S_{t-1}^T (a * kappa)        record 2 pos   = (w, kappa, u_e)
 *   u_w = v                                 record 2 pos+1 = (1, k, v)
 *   S_t = eq. 4 over records 0 .. 2pos+1,   y = S_t^T q
 * and at the last token (pos = W-1) S_W is quantized into the next window's (Z, a).
 * Records: G[nh][2W][dk], K[nh][2W][dk], U[nh][2W][dv].
 */
void oracle_rwkv7_q8_window_step(int64_t nh, int dk, int dv, int W, int pos, int8_t *Z, float *a,
                                 double *G, double *K, double *U, const double *q, const double *k,
                                 const double *v, const double *w, const double *kappa,
                                 const double *erase, double *y, double *Sw_out, double *w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        int8_t *Zh = Z + (size_t)h * dk * dv;
        float *ah = a + (size_t)h * dk;
        double *Gh = G + (size_t)h * 2 * W * dk;
        double *Kh = K + (size_t)h * 2 * W * dk;
        double *Uh = U + (size_t)h * 2 * W * dv;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk, *vh = v + (size_t)h * dv;
        const double *wh = w + (size_t)h * dk, *ch = kappa + (size_t)h * dk, *eh = erase + (size_t)h * dk;
        double *yh = y + (size_t)h * dv;
        const int re = 2 * pos, rw = 2 * pos + 1;

        double *S0 = (double *)malloc(sizeof(double) * dk * dv);
        double *St = (double *)malloc(sizeof(double) * dk * dv);
        dequant_head(dk, dv, Zh, ah, S0);
        window_materialize(dk, dv, 1, re, S0, Gh, Kh, Uh, St);          /* S_{t-1} */
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i)
                p += St[IDX2(i, j, dv)] * eh[i] * ch[i];
            Uh[IDX2(re, j, dv)] = 0.0 - p;
            Uh[IDX2(rw, j, dv)] = vh[j];
        }
        for (int i = 0; i < dk; ++i) {
            Gh[IDX2(re, i, dk)] = wh[i];
            Kh[IDX2(re, i, dk)] = ch[i];
            Gh[IDX2(rw, i, dk)] = 1.0;
            Kh[IDX2(rw, i, dk)] = kh[i];
        }
        window_materialize(dk, dv, 1, rw + 1, S0, Gh, Kh, Uh, St);      /* S_t */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += St[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        if (pos == W - 1) {
            if (Sw_out)
                memcpy(Sw_out + (size_t)h * dk * dv, St, sizeof(double) * dk * dv);
            oracle_q8_quantize(dk, dv, St, Zh, ah, w_out ? w_out + (size_t)h * dk * dv : NULL);
        }
        free(S0);
        free(St);
    }
}

/*
 * One DeltaProduct token on the per-window int8 state (LeapQuant, sec. 3.2 and App. A:
 * each of the n sub-steps is one buffered record, as the page does for a token with two
 * sub-steps). A window of W tokens buffers nW records with scalar gates alpha_t, 1, .., 1
 * per token. Token pos (0-based) owns records n pos .. n pos + n - 1; sub-step s:
 *   S_cur = eq. 4 over the records before n pos + s
 *   u_s = beta_s (v_s - (d_s S_cur)^T k_s),  d_0 = alpha, d_s = 1     record (d_s, k_s, u_s)
 * then y = S_t^T q with S_t = eq. 4 over all the token's records; at the last token
 * (pos = W-1) S_W is quantized into the next window's (Z, a).
 * Records: G[nh][nW], K[nh][nW][dk], U[nh][nW][dv]; k[nh][n][dk], v[nh][n][dv], beta[nh][n].
 */
void oracle_deltaproduct_q8_window_step(int64_t nh, int dk, int dv, int n, int W, int pos,
                                        int8_t *Z, float *a, double *G, double *K, double *U,
                                        const double *q, const double *k, const double *v,
                                        const double *alpha, const double *beta, double *y,
                                        double *Sw_out, double *w_out)
{
    const int R = n * W;
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        int8_t *Zh = Z + (size_t)h * dk * dv;
        float *ah = a + (size_t)h * dk;
        double *Gh = G + (size_t)h * R;
        double *Kh = K + (size_t)h * R * dk;
        double *Uh = U + (size_t)h * R * dv;
        const double *qh = q + (size_t)h * dk;
        double *yh = y + (size_t)h * dv;

        double *S0 = (double *)malloc(sizeof(double) * dk * dv);
        double *St = (double *)malloc(sizeof(double) * dk * dv);
        dequant_head(dk, dv, Zh, ah, S0);
        for (int s = 0; s < n; ++s) {
            const int rec = n * pos + s;
            const double *ks = k + ((size_t)h * n + s) * dk;
            const double *vs = v + ((size_t)h * n + s) * dv;
            const double d = s == 0 ? alpha[h] : 1.0;
            Gh[rec] = d;
            for (int i = 0; i < dk; ++i)
                Kh[IDX2(rec, i, dk)] = ks[i];
            window_materialize(dk, dv, 0, rec, S0, Gh, Kh, Uh, St);
            for (int j = 0; j < dv; ++j) {
                double p = 0.0;
                for (int i = 0; i < dk; ++i)
                    p += d * St[IDX2(i, j, dv)] * ks[i];
                Uh[IDX2(rec, j, dv)] = beta[(size_t)h * n + s] * (vs[j] - p);
            }
        }
        window_materialize(dk, dv, 0, n * pos + n, S0, Gh, Kh, Uh, St);
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += St[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        if (pos == W - 1) {
            if (Sw_out)
                memcpy(Sw_out + (size_t)h * dk * dv, St, sizeof(double) * dk * dv);
            oracle_q8_quantize(dk, dv, St, Zh, ah, w_out ? w_out + (size_t)h * dk * dv : NULL);
        }
        free(S0);
        free(St);
    }
}

/*
 * One step of the base + log representation (DeltaLog, sec. 3.1, Algorithm 1,
 * eqs. 2-7). The physical state of a head is the dense base Sbar, the cumulative
 * log-decay lbar (one value, or one per key channel) and L live log entries
 * (K_log[m], U_log[m], Lam_log[m]), m < L <= C. D(l) = diag(exp(l)).
 * The logical state (eq. 7) is
 *   S = D(lbar) Sbar + sum_{m<L} D(lbar - Lam_m) K_m U_m^T.
 * With lambda_t = ln g_t (eq. 3) the step follows Algorithm 1:
 *   1. read the old state: p = (D(lambda_t) S_{t-1})^T k    (the delta correction)
 *   2. lbar += lambda_t                                      (eq. 4)
 *   3. a = k, b = beta (v - p); y = S_t^T q with S_t of eq. 7 plus a b^T
 *   4. L <  C: append (a, b, lbar) into slot L               (eq. 5); the caller sets L += 1
 *   5. L == C: Sbar = S_t (eq. 6), lbar = 0; the caller sets L = 0.
 * Log arrays: K[nh][C][dk], U[nh][C][dv], Lam[nh][C] or [nh][C][dk];
 * lbar[nh] or [nh][dk].
 */
static void log_step_head(int64_t h, int dk, int dv, int per_key, int delta, int C, int L,
                          double *Sbar, double *lbar, double *Klog, double *Ulog, double *Lam,
                          const double *q, const double *k, const double *v,
                          const double *gate, const double *beta, double *y)
{
    const int gdim = per_key ? dk : 1;
    {
        double *Sh = Sbar + (size_t)h * dk * dv;
        double *lb = lbar + (size_t)h * gdim;
        double *Kh = Klog + (size_t)h * C * dk;
        double *Uh = Ulog + (size_t)h * C * dv;
        double *Lh = Lam + (size_t)h * C * gdim;
        const double *qh = q + (size_t)h * dk, *kh = k + (size_t)h * dk;
        const double *vh = v + (size_t)h * dv;
        const double *gh = gate + (size_t)h * gdim;
        double *yh = y + (size_t)h * dv;
        double *St = (double *)malloc(sizeof(double) * dk * dv);
        double *b = (double *)malloc(sizeof(double) * dv);

        /* eq. 7: the pre-update logical state */
        for (int i = 0; i < dk; ++i) {
            double li = lb[per_key ? i : 0];
            for (int j = 0; j < dv; ++j) {
                double s = exp(li) * Sh[IDX2(i, j, dv)];
                for (int m = 0; m < L; ++m)
                    s += exp(li - Lh[IDX2(m, per_key ? i : 0, gdim)]) * Kh[IDX2(m, i, dk)] *
                         Uh[IDX2(m, j, dv)];
                St[IDX2(i, j, dv)] = s;
            }
        }
        /* 1. the old-state read of the delta rule, along the decayed key:
              p = (D(lambda_t) S_{t-1})^T k with lambda_t = ln g_t; without the delta
              rule (RWKV6, DeltaLog Table 1) the value-side factor is v itself */
        for (int j = 0; j < dv; ++j) {
            if (!delta) {
                b[j] = vh[j];
                continue;
            }
            double p = 0.0;
            for (int i = 0; i < dk; ++i) {
                double lam = log(gate_at(gh, per_key, i));
                p += exp(lam) * St[IDX2(i, j, dv)] * kh[i];
            }
            b[j] = beta[h] * (vh[j] - p);
        }
        /* 2. cumulative log-decay */
        for (int i = 0; i < gdim; ++i)
            lb[i] += log(gh[i]);
        /* 3. post-update logical state (eq. 7 with the current pair a b^T) and output */
        for (int i = 0; i < dk; ++i) {
            double li = lb[per_key ? i : 0];
            for (int j = 0; j < dv; ++j) {
                double s = exp(li) * Sh[IDX2(i, j, dv)];
                for (int m = 0; m < L; ++m)
                    s += exp(li - Lh[IDX2(m, per_key ? i : 0, gdim)]) * Kh[IDX2(m, i, dk)] *
                         Uh[IDX2(m, j, dv)];
                St[IDX2(i, j, dv)] = s + kh[i] * b[j];
            }
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += St[IDX2(i, j, dv)] * qh[i];
            yh[j] = acc;
        }
        if (L < C) {
            /* 4. append, eq. 5 */
            for (int i = 0; i < dk; ++i)
                Kh[IDX2(L, i, dk)] = kh[i];
            for (int j = 0; j < dv; ++j)
                Uh[IDX2(L, j, dv)] = b[j];
            for (int i = 0; i < gdim; ++i)
                Lh[IDX2(L, i, gdim)] = lb[i];
        } else {
            /* 5. merge, eq. 6, and reset */
            memcpy(Sh, St, sizeof(double) * dk * dv);
            for (int i = 0; i < gdim; ++i)
                lb[i] = 0.0;
        }
        free(St);
        free(b);
    }
}

void oracle_log_step(int64_t nh, int dk, int dv, int per_key, int C, int L,
                     double *Sbar, double *lbar, double *Klog, double *Ulog, double *Lam,
                     const double *q, const double *k, const double *v,
                     const double *gate, const double *beta, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h)
        log_step_head(h, dk, dv, per_key, 1, C, L, Sbar, lbar, Klog, Ulog, Lam, q, k, v, gate, beta, y);
}

/* The same step with a live length per head (each request slot at its own point
 * of its append/merge cycle): Ls[h] in [0, C] selects append or merge for head h,
 * and is advanced here (L + 1 after an append, 0 after a merge). */
void oracle_log_step_slots(int64_t nh, int dk, int dv, int per_key, int C, int *Ls,
                           double *Sbar, double *lbar, double *Klog, double *Ulog, double *Lam,
                           const double *q, const double *k, const double *v,
                           const double *gate, const double *beta, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        log_step_head(h, dk, dv, per_key, 1, C, Ls[h], Sbar, lbar, Klog, Ulog, Lam, q, k, v, gate, beta, y);
        Ls[h] = Ls[h] < C ? Ls[h] + 1 : 0;
    }
}

/* The base + log step for RWKV6 (DeltaLog sec. 3.4: per-key log-decay metadata as for
 * KDA, update pair (k, v) with no old-state correction): Alg. 1 with b = v. */
void oracle_rwkv6_log_step(int64_t nh, int dk, int dv, int C, int L, double *Sbar, double *lbar,
                           double *Klog, double *Ulog, double *Lam, const double *q,
                           const double *k, const double *v, const double *w, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h)
        log_step_head(h, dk, dv, 1, 0, C, L, Sbar, lbar, Klog, Ulog, Lam, q, k, v, w, NULL, y);
}

void oracle_rwkv6_log_step_slots(int64_t nh, int dk, int dv, int C, int *Ls, double *Sbar,
                                 double *lbar, double *Klog, double *Ulog, double *Lam,
                                 const double *q, const double *k, const double *v,
                                 const double *w, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
        log_step_head(h, dk, dv, 1, 0, C, Ls[h], Sbar, lbar, Klog, Ulog, Lam, q, k, v, w, NULL, y);
        Ls[h] = Ls[h] < C ? Ls[h] + 1 : 0;
    }
}
