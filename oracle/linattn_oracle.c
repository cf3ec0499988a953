/*
 * linattn_oracle.c -- plain fp64 CPU oracle for causal linear attention with
 * the feature map phi(x) = elu(x) + 1.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header or constant with the HIP library and must
 * never be called from the product path.
 *
 * Every routine is the plain definition, one token at a time, in double
 * precision, with no blocking or reordering:
 *
 *   phi(x)  = elu(x) + 1, elu(x) = x for x >= 0 and exp(x) - 1 for x < 0
 *            ("Transformers are RNNs" review, feature-map table: elu row and
 *             the +1 offset row; "Linear Attention: accumulating KV into a
 *             fixed-size state", section "Why replace softmax").
 *   S_t     = a_t * S_{t-1} + phi(k_t) v_t^T     (a_t = 1 when ungated)
 *   z_t     = a_t * z_{t-1} + phi(k_t)
 *   o_t     = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps)
 *            (fixed-size-state page, section "State update and read as
 *             equations"; review page, causal-masking and RNN-form tables,
 *             which start from S_0 = 0, z_0 = 0; the scalar decay a_t on the
 *             whole summary follows "Linear Attention: what happens when you
 *             change the product order", section "The summary runs out of
 *             room", and the h_t = a h_{t-1} + x_t recurrence of the
 *             state-space-models page, section 3).
 *
 * The read uses the state *after* token t was added, so token t's own key and
 * value take part in o_t (inclusive diagonal).  oracle_backward is the adjoint
 * of the same recurrence (the gradients of a loss L given dL/dO).  eps is added after the dot
 * product.  parity pinned: see tests/test_oracle.py.
 *
 * Layout (row-major, contiguous, one (batch, head) pair after another):
 *   q [BH][N][Dk], k [BH][N][Dk], v [BH][N][Dv], alpha [BH][N],
 *   o [BH][N][Dv], s [BH][Dk][Dv] (row = key component, column = value
 *   component), z [BH][Dk].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHI_ELU1 0
#define PHI_IDENTITY 1

static double phi(double x, int mode)
{
    if (mode == PHI_IDENTITY)
        return x;
    /* elu(x) + 1: x + 1 on x >= 0; on x < 0, (exp(x) - 1) + 1, which is
     * exp(x) exactly (written so, to keep the small values of exp(x)). */
    return (x >= 0.0) ? x + 1.0 : exp(x);
}

/* One recurrence over N tokens for one (batch, head) pair.  s and z hold the
 * running state on entry and on exit. */
static void recur_one(const double *q, const double *k, const double *v,
                      const double *alpha, double *o, double *s, double *z,
                      int64_t N, int Dk, int Dv, int mode, double eps,
                      double *fq, double *fk, double *num)
{
    for (int64_t t = 0; t < N; ++t) {
        const double *qt = q + t * Dk;
        const double *kt = k + t * Dk;
        const double *vt = v + t * Dv;
        for (int i = 0; i < Dk; ++i) {
            fq[i] = phi(qt[i], mode);
            fk[i] = phi(kt[i], mode);
        }
        if (alpha) {
            double a = alpha[t];
            for (int i = 0; i < Dk; ++i) {
                z[i] *= a;
                for (int j = 0; j < Dv; ++j)
                    s[(int64_t)i * Dv + j] *= a;
            }
        }
        /* write: S += phi(k) v^T, z += phi(k) */
        for (int i = 0; i < Dk; ++i) {
            z[i] += fk[i];
            for (int j = 0; j < Dv; ++j)
                s[(int64_t)i * Dv + j] += fk[i] * vt[j];
        }
        /* read the updated state with phi(q) */
        double den = 0.0;
        for (int j = 0; j < Dv; ++j)
            num[j] = 0.0;
        for (int i = 0; i < Dk; ++i) {
            den += fq[i] * z[i];
            for (int j = 0; j < Dv; ++j)
                num[j] += fq[i] * s[(int64_t)i * Dv + j];
        }
        if (o) {
            double *ot = o + t * Dv;
            for (int j = 0; j < Dv; ++j)
                ot[j] = num[j] / (den + eps);
        }
    }
}

/* Causal forward, optionally gated (alpha == NULL means a_t = 1).
 * s_init / z_init may be NULL (zero state).  o, s_final, z_final may be NULL
 * when not wanted.  Returns 0, or -1 on a bad argument / allocation failure. */
int oracle_forward(const double *q, const double *k, const double *v,
                   const double *alpha, const double *s_init,
                   const double *z_init, double *o, double *s_final,
                   double *z_final, int64_t BH, int64_t N, int Dk, int Dv,
                   int mode, double eps, int nthreads)
{
    if (!q || !k || !v || BH < 0 || N < 0 || Dk < 1 || Dv < 1)
        return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double *s = calloc((size_t)Dk * Dv, sizeof(double));
        double *z = calloc((size_t)Dk, sizeof(double));
        double *fq = malloc(sizeof(double) * Dk);
        double *fk = malloc(sizeof(double) * Dk);
        double *num = malloc(sizeof(double) * Dv);
        if (!s || !z || !fq || !fk || !num) {
#pragma omp atomic write
            err = 1;
        } else {
            if (s_init)
                memcpy(s, s_init + bh * Dk * Dv, sizeof(double) * Dk * Dv);
            if (z_init)
                memcpy(z, z_init + bh * Dk, sizeof(double) * Dk);
            recur_one(q + bh * N * Dk, k + bh * N * Dk, v + bh * N * Dv,
                      alpha ? alpha + bh * N : NULL, o ? o + bh * N * Dv : NULL,
                      s, z, N, Dk, Dv, mode, eps, fq, fk, num);
            if (s_final)
                memcpy(s_final + bh * Dk * Dv, s, sizeof(double) * Dk * Dv);
            if (z_final)
                memcpy(z_final + bh * Dk, z, sizeof(double) * Dk);
        }
        free(s); free(z); free(fq); free(fk); free(num);
    }
    return err ? -1 : 0;
}

/* Non-causal: S = sum_t phi(k_t) v_t^T and z = sum_t phi(k_t) over the whole
 * sequence, computed once and read by every query ("Transformers are RNNs"
 * review, discussion of the non-causal case that reuses the summed key-value
 * matrix for all queries).  Zero initial state. */
int oracle_noncausal(const double *q, const double *k, const double *v,
                     double *o, double *s_out, double *z_out, int64_t BH,
                     int64_t N, int Dk, int Dv, int mode, double eps,
                     int nthreads)
{
    if (!q || !k || !v || BH < 0 || N < 0 || Dk < 1 || Dv < 1)
        return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double *s = calloc((size_t)Dk * Dv, sizeof(double));
        double *z = calloc((size_t)Dk, sizeof(double));
        double *fq = malloc(sizeof(double) * Dk);
        double *num = malloc(sizeof(double) * Dv);
        if (!s || !z || !fq || !num) {
#pragma omp atomic write
            err = 1;
        } else {
            const double *kb = k + bh * N * Dk, *vb = v + bh * N * Dv;
            const double *qb = q + bh * N * Dk;
            for (int64_t t = 0; t < N; ++t) {
                for (int i = 0; i < Dk; ++i) {
                    double f = phi(kb[t * Dk + i], mode);
                    z[i] += f;
                    for (int j = 0; j < Dv; ++j)
                        s[(int64_t)i * Dv + j] += f * vb[t * Dv + j];
                }
            }
            if (o) {
                for (int64_t t = 0; t < N; ++t) {
                    double den = 0.0;
                    for (int i = 0; i < Dk; ++i)
                        fq[i] = phi(qb[t * Dk + i], mode);
                    for (int j = 0; j < Dv; ++j)
                        num[j] = 0.0;
                    for (int i = 0; i < Dk; ++i) {
                        den += fq[i] * z[i];
                        for (int j = 0; j < Dv; ++j)
                            num[j] += fq[i] * s[(int64_t)i * Dv + j];
                    }
                    for (int j = 0; j < Dv; ++j)
                        o[bh * N * Dv + t * Dv + j] = num[j] / (den + eps);
                }
            }
            if (s_out)
                memcpy(s_out + bh * Dk * Dv, s, sizeof(double) * Dk * Dv);
            if (z_out)
                memcpy(z_out + bh * Dk, z, sizeof(double) * Dk);
        }
        free(s); free(z); free(fq); free(num);
    }
    return err ? -1 : 0;
}

/* One decode step per (batch, head): the loop body of the recurrence applied
 * once to the carried (S, z), which are updated in place ("Transformers are
 * RNNs" review: the RNN mode keeps only (S, z) and takes one token at a
 * time).  q, k: [BH][Dk]; v: [BH][Dv]; alpha: [BH] or NULL; o: [BH][Dv]. */
int oracle_decode_step(const double *q, const double *k, const double *v,
                       const double *alpha, double *s, double *z, double *o,
                       int64_t BH, int Dk, int Dv, int mode, double eps,
                       int nthreads)
{
    if (!q || !k || !v || !s || !z || BH < 0 || Dk < 1 || Dv < 1)
        return -1;
    int err = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double *fq = malloc(sizeof(double) * Dk);
        double *fk = malloc(sizeof(double) * Dk);
        double *num = malloc(sizeof(double) * Dv);
        if (!fq || !fk || !num) {
#pragma omp atomic write
            err = 1;
        } else {
            recur_one(q + bh * Dk, k + bh * Dk, v + bh * Dv,
                      alpha ? alpha + bh : NULL, o ? o + bh * Dv : NULL,
                      s + bh * Dk * Dv, z + bh * Dk, 1, Dk, Dv, mode, eps,
                      fq, fk, num);
        }
        free(fq); free(fk); free(num);
    }
    return err ? -1 : 0;
}

/* Round x to the nearest number with p significant bits, ties to even; below
 * 2^emin the grid is fixed at 2^(emin - p + 1) (subnormals).  bf16 is p = 8,
 * emin = -126; OCP fp8 e4m3 is p = 4, emin = -6, with 448 the largest finite
 * magnitude (a larger one is stored as NaN, as the gfx950 conversion does). */
static double round_sig(double x, int p, int emin)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    int e;
    frexp(x, &e); /* |x| in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < emin)
        ex = emin;
    const double q = ldexp(1.0, ex - (p - 1));
    return nearbyint(x / q) * q; /* default rounding mode: nearest, ties to even */
}

#define STATE_F32 0
#define STATE_BF16 1
#define STATE_FP8_E4M3 2

double oracle_state_round(double x, int sdt)
{
    if (sdt == STATE_BF16)
        return round_sig(x, 8, -126);
    if (sdt == STATE_FP8_E4M3) {
        const double r = round_sig(x, 4, -6);
        return fabs(r) > 448.0 ? NAN : r;
    }
    return (double)(float)x;
}

/* A decode step with the state stored in a narrower type (state dtype sdt):
 * S <- round(a S + phi(k) v^T), z <- round(a z + phi(k)) elementwise, then
 * o = phi(q)^T S / (phi(q)^T z + eps) from the stored values.  The rounding
 * decides a stored code, so it is taken on the same fp32 value the library
 * rounds: phi(k) in fp32, the product phi(k) v in fp32, then one fused
 * multiply-add a * S + phi(k) v in fp32; the read is in fp64. */
int oracle_decode_lowp(const double *q, const double *k, const double *v,
                       const double *alpha, double *s, double *z, double *o,
                       int64_t BH, int Dk, int Dv, int mode, double eps,
                       int sdt)
{
    if (!q || !k || !v || !s || !z || BH < 0 || Dk < 1 || Dv < 1)
        return -1;
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *qt = q + bh * Dk, *kt = k + bh * Dk, *vt = v + bh * Dv;
        double *sb = s + bh * Dk * Dv, *zb = z + bh * Dk;
        const float a = alpha ? (float)alpha[bh] : 1.0f;
        double den = 0.0;
        for (int i = 0; i < Dk; ++i) {
            const float fk = (float)phi(kt[i], mode);
            zb[i] = oracle_state_round((double)fmaf(a, (float)zb[i], fk), sdt);
            for (int j = 0; j < Dv; ++j) {
                const float pr = fk * (float)vt[j];
                sb[(int64_t)i * Dv + j] =
                    oracle_state_round((double)fmaf(a, (float)sb[(int64_t)i * Dv + j], pr), sdt);
            }
            den += phi(qt[i], mode) * zb[i];
        }
        if (o) {
            for (int j = 0; j < Dv; ++j) {
                double num = 0.0;
                for (int i = 0; i < Dk; ++i)
                    num += phi(qt[i], mode) * sb[(int64_t)i * Dv + j];
                o[bh * Dv + j] = num / (den + eps);
            }
        }
    }
    return 0;
}

/* The feature map alone, elementwise, for the closed-form pins. */
/* Derivative of phi: 1 on x >= 0 and exp(x) on x < 0 for elu + 1 (elu's
 * derivative, the +1 offset drops out); 1 everywhere for the identity map. */
static double dphi(double x, int mode)
{
    if (mode == PHI_IDENTITY)
        return 1.0;
    return (x >= 0.0) ? 1.0 : exp(x);
}

/* Backward of the causal forward for one (batch, head) pair: given
 * dout = dL/dO, the gradients of L with respect to q, k, v and the initial
 * state.  The gates (alpha == NULL means a_t = 1) are constants here.
 *
 * It is the adjoint of the recurrence above, written out from its definition:
 *   forward in time, with num_t = phi(q_t)^T S_t, den_t = phi(q_t)^T z_t + eps,
 *     dy_t  = dout_t / den_t                 (dL/dnum_t)
 *     dd_t  = -(dout_t . o_t) / den_t        (dL/dden_t)
 *     dq_t  = (S_t dy_t + dd_t z_t) * phi'(q_t)
 *   backward in time, with G_t = dL/dS_t and g_t = dL/dz_t over all later reads,
 *     G_t   = a_{t+1} G_{t+1} + phi(q_t) dy_t^T
 *     g_t   = a_{t+1} g_{t+1} + dd_t phi(q_t)
 *     dk_t  = (G_t v_t + g_t) * phi'(k_t)
 *     dv_t  = G_t^T phi(k_t)
 *   and the initial state enters S_0 with factor a_0:
 *     ds_init = a_0 G_0,  dz_init = a_0 g_0. */
static void backward_one(const double *q, const double *k, const double *v,
                         const double *alpha, const double *s_init,
                         const double *z_init, const double *dout, double *dq,
                         double *dk, double *dv, double *ds_init,
                         double *dz_init, int64_t N, int Dk, int Dv, int mode,
                         double eps, double *s, double *z, double *dy,
                         double *dd, double *fq, double *fk, double *num)
{
    /* forward sweep */
    for (int i = 0; i < Dk; ++i) {
        z[i] = z_init ? z_init[i] : 0.0;
        for (int j = 0; j < Dv; ++j)
            s[(int64_t)i * Dv + j] = s_init ? s_init[(int64_t)i * Dv + j] : 0.0;
    }
    for (int64_t t = 0; t < N; ++t) {
        const double *qt = q + t * Dk, *kt = k + t * Dk, *vt = v + t * Dv;
        const double *go = dout + t * Dv;
        for (int i = 0; i < Dk; ++i) {
            fq[i] = phi(qt[i], mode);
            fk[i] = phi(kt[i], mode);
        }
        const double a = alpha ? alpha[t] : 1.0;
        for (int i = 0; i < Dk; ++i) {
            z[i] = a * z[i] + fk[i];
            for (int j = 0; j < Dv; ++j)
                s[(int64_t)i * Dv + j] = a * s[(int64_t)i * Dv + j] + fk[i] * vt[j];
        }
        double den = eps;
        for (int j = 0; j < Dv; ++j)
            num[j] = 0.0;
        for (int i = 0; i < Dk; ++i) {
            den += fq[i] * z[i];
            for (int j = 0; j < Dv; ++j)
                num[j] += fq[i] * s[(int64_t)i * Dv + j];
        }
        double go_dot_o = 0.0;
        for (int j = 0; j < Dv; ++j) {
            dy[t * Dv + j] = go[j] / den;
            go_dot_o += go[j] * (num[j] / den);
        }
        dd[t] = -go_dot_o / den;
        for (int i = 0; i < Dk; ++i) {
            double acc = dd[t] * z[i];
            for (int j = 0; j < Dv; ++j)
                acc += s[(int64_t)i * Dv + j] * dy[t * Dv + j];
            dq[t * Dk + i] = acc * dphi(qt[i], mode);
        }
    }
    /* backward sweep: s, z now hold G and g */
    memset(s, 0, sizeof(double) * (size_t)Dk * Dv);
    memset(z, 0, sizeof(double) * (size_t)Dk);
    double a_next = 1.0;
    for (int64_t t = N - 1; t >= 0; --t) {
        const double *qt = q + t * Dk, *kt = k + t * Dk, *vt = v + t * Dv;
        for (int i = 0; i < Dk; ++i) {
            fq[i] = phi(qt[i], mode);
            fk[i] = phi(kt[i], mode);
        }
        for (int i = 0; i < Dk; ++i) {
            z[i] = a_next * z[i] + dd[t] * fq[i];
            for (int j = 0; j < Dv; ++j)
                s[(int64_t)i * Dv + j] = a_next * s[(int64_t)i * Dv + j] + fq[i] * dy[t * Dv + j];
        }
        for (int i = 0; i < Dk; ++i) {
            double acc = z[i];
            for (int j = 0; j < Dv; ++j)
                acc += s[(int64_t)i * Dv + j] * vt[j];
            dk[t * Dk + i] = acc * dphi(kt[i], mode);
        }
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i)
                acc += s[(int64_t)i * Dv + j] * fk[i];
            dv[t * Dv + j] = acc;
        }
        a_next = alpha ? alpha[t] : 1.0;
    }
    if (ds_init)
        for (int64_t e = 0; e < (int64_t)Dk * Dv; ++e)
            ds_init[e] = a_next * s[e];
    if (dz_init)
        for (int i = 0; i < Dk; ++i)
            dz_init[i] = a_next * z[i];
}

/* Backward over BH (batch, head) pairs; see backward_one.  alpha, s_init,
 * z_init, ds_init, dz_init may be NULL.  Returns 0, or -1 on a bad argument /
 * allocation failure. */
int oracle_backward(const double *q, const double *k, const double *v,
                    const double *alpha, const double *s_init,
                    const double *z_init, const double *dout, double *dq,
                    double *dk, double *dv, double *ds_init, double *dz_init,
                    int64_t BH, int64_t N, int Dk, int Dv, int mode, double eps,
                    int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || BH < 0 || N < 0 || Dk < 1 || Dv < 1)
        return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double *s = malloc(sizeof(double) * (size_t)Dk * Dv);
        double *z = malloc(sizeof(double) * (size_t)Dk);
        double *dy = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * Dv);
        double *dd = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *fq = malloc(sizeof(double) * Dk);
        double *fk = malloc(sizeof(double) * Dk);
        double *num = malloc(sizeof(double) * Dv);
        if (!s || !z || !dy || !dd || !fq || !fk || !num) {
#pragma omp atomic write
            err = 1;
        } else {
            backward_one(q + bh * N * Dk, k + bh * N * Dk, v + bh * N * Dv,
                         alpha ? alpha + bh * N : NULL,
                         s_init ? s_init + bh * Dk * Dv : NULL,
                         z_init ? z_init + bh * Dk : NULL, dout + bh * N * Dv,
                         dq + bh * N * Dk, dk + bh * N * Dk, dv + bh * N * Dv,
                         ds_init ? ds_init + bh * Dk * Dv : NULL,
                         dz_init ? dz_init + bh * Dk : NULL, N, Dk, Dv, mode,
                         eps, s, z, dy, dd, fq, fk, num);
        }
        free(s); free(z); free(dy); free(dd); free(fq); free(fk); free(num);
    }
    return err ? -1 : 0;
}

/* Delta rule ("Linear Attention: what happens when you change the product
 * order", section "The summary runs out of room"): before writing, the
 * summary is read with the key, and only the difference between the value
 * and that read is written, so that re-reading with the same key returns the
 * new value.  The same section's gated form (Gated DeltaNet: a global decay
 * combined with the selective overwrite) first decays the whole summary by
 * a_t.  Per token, for one (batch, head) pair:
 *   kh_t = phi(k_t) / |phi(k_t)|_2             (unit key; a zero key writes nothing)
 *   S'   = a_t S_{t-1}                         (a_t = 1 unless gated)
 *   u_t  = S'^T kh_t                           (read before the write)
 *   S_t  = S' + beta_t kh_t (v_t - u_t)^T      (write the difference; beta_t = 1 unless given)
 *   o_t  = S_t^T phi(q_t)                      (read with the query; no normalizer)
 * s holds the running state on entry and on exit. */
static void delta_one(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta, double *o,
                      double *s, int64_t N, int Dk, int Dv, int mode,
                      double *kh, double *u)
{
    for (int64_t t = 0; t < N; ++t) {
        if (alpha)
            for (int64_t e = 0; e < (int64_t)Dk * Dv; ++e)
                s[e] *= alpha[t];
        const double *qt = q + t * Dk, *kt = k + t * Dk, *vt = v + t * Dv;
        double nrm = 0.0;
        for (int i = 0; i < Dk; ++i) {
            kh[i] = phi(kt[i], mode);
            nrm += kh[i] * kh[i];
        }
        nrm = sqrt(nrm);
        for (int i = 0; i < Dk; ++i)
            kh[i] = nrm > 0.0 ? kh[i] / nrm : 0.0;
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i)
                acc += s[(int64_t)i * Dv + j] * kh[i];
            u[j] = acc;
        }
        const double b = beta ? beta[t] : 1.0;
        for (int i = 0; i < Dk; ++i)
            for (int j = 0; j < Dv; ++j)
                s[(int64_t)i * Dv + j] += b * kh[i] * (vt[j] - u[j]);
        if (o) {
            for (int j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < Dk; ++i)
                    acc += s[(int64_t)i * Dv + j] * phi(qt[i], mode);
                o[t * Dv + j] = acc;
            }
        }
    }
}

/* Delta-rule forward over BH pairs; alpha, beta [BH][N] or NULL (all ones);
 * s_init NULL for zero; o, s_final may be NULL. */
int oracle_delta(const double *q, const double *k, const double *v,
                 const double *alpha, const double *beta,
                 const double *s_init, double *o, double *s_final,
                 int64_t BH, int64_t N, int Dk, int Dv, int mode,
                 int nthreads)
{
    if (!q || !k || !v || BH < 0 || N < 0 || Dk < 1 || Dv < 1)
        return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double *s = calloc((size_t)Dk * Dv, sizeof(double));
        double *kh = malloc(sizeof(double) * Dk);
        double *u = malloc(sizeof(double) * Dv);
        if (!s || !kh || !u) {
#pragma omp atomic write
            err = 1;
        } else {
            if (s_init)
                memcpy(s, s_init + bh * Dk * Dv, sizeof(double) * Dk * Dv);
            delta_one(q + bh * N * Dk, k + bh * N * Dk, v + bh * N * Dv,
                      alpha ? alpha + bh * N : NULL, beta ? beta + bh * N : NULL,
                      o ? o + bh * N * Dv : NULL, s, N, Dk, Dv, mode, kh, u);
            if (s_final)
                memcpy(s_final + bh * Dk * Dv, s, sizeof(double) * Dk * Dv);
        }
        free(s); free(kh); free(u);
    }
    return err ? -1 : 0;
}

void oracle_phi(const double *x, double *y, int64_t n, int mode)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = phi(x[i], mode);
}
