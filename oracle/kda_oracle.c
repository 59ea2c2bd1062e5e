/*
 * kda_oracle.c -- plain, slow, sequential fp64 recurrence (TEST INFRASTRUCTURE).
 *
 * Each step follows the order the explainer "我终于看懂了 KDA…" gives in its
 * section 八: decay the old state with the gate, read the old answer with the
 * key, take the error against the new value, write the correction.  The read,
 * error and write are the delta rule of section 六 ("old_value = read(memory,
 * key); error = new_value - old_value; memory += learning_rate * write(key,
 * error)"), the learning rate being beta.  The gate is the per-channel alpha of
 * the Kimi Linear paragraph of "一个KimiK3装下22580个GPT-2…", alpha = exp(g).
 * The output is read from the state after the token's own write.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_last_threads = 1;

int kda_oracle_last_threads(void) { return g_last_threads; }

void kda_oracle_recurrent(int B, int T, int H, int dk, int dv,
                          const double *q, const double *k, const double *v,
                          const double *g, const double *beta,
                          const double *S0, double *o, double *ST,
                          int delta, double *u_out, int nthreads)
{
    const long BH = (long)B * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    g_last_threads = nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
    g_last_threads = 1;
#endif
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);

        if (S0) memcpy(S, S0 + bh * (long)dk * dv, sizeof(double) * (size_t)dk * dv);
        else    memset(S, 0, sizeof(double) * (size_t)dk * dv);

        for (long t = 0; t < T; ++t) {
            const long row = (b * T + t) * H + h;          /* (b,t,h) */
            const double *qt = q + row * dk;
            const double *kt = k + row * dk;
            const double *vt = v + row * dv;
            const double *gt = g + row * dk;
            const double  bt = beta[row];

            /* 1. decay: row c of S is scaled by alpha_c = exp(g_c) (exp(-inf) = 0) */
            for (int c = 0; c < dk; ++c) {
                const double a = exp(gt[c]);
                for (int j = 0; j < dv; ++j) S[(long)c * dv + j] *= a;
            }
            /* 2. read the decayed state with the key: r = S^T k */
            for (int j = 0; j < dv; ++j) r[j] = 0.0;
            if (delta) {
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) r[j] += kt[c] * S[(long)c * dv + j];
            }
            /* 3. error against the new value, scaled by beta */
            for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);
            /* 4. write the correction along the key: S += k u^T */
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) S[(long)c * dv + j] += kt[c] * u[j];
            /* 5. output from the updated state: o = S^T q */
            double *ot = o + row * dv;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) ot[j] += qt[c] * S[(long)c * dv + j];
            if (u_out) memcpy(u_out + row * dv, u, sizeof(double) * (size_t)dv);
        }
        if (ST) memcpy(ST + bh * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(r); free(u);
    }
}

/*
 * The adjoint of the recurrence.  For one token, with a = exp(g) per channel:
 *     S' = Diag(a) S,   r = S'^T k,   u = beta (v - r),   S+ = S' + k u^T,   o = S+^T q
 * and an incoming cotangent dS+ of S+ (plus dO of o), reverse mode gives, in this
 * order:
 *     dS+ += q dO^T            dq = S+ dO
 *     du   = dS+^T k           dk = dS+ u
 *     dbeta = du . (v - r)     dv = beta du        dr = -beta du
 *     dS'  = dS+ + k dr^T      dk += S' dr
 *     da_c = sum_j dS'_cj S_cj,  dg = da * a         dS = Diag(a) dS'
 * (dS is the cotangent handed to the previous token).
 */
static void step_forward(int dk, int dv, const double *qt, const double *kt, const double *vt,
                         const double *gt, double bt, const double *S, double *Sn,
                         double *r, double *u)
{
    (void)qt;
    for (int c = 0; c < dk; ++c) {
        const double a = exp(gt[c]);
        for (int j = 0; j < dv; ++j) Sn[(long)c * dv + j] = a * S[(long)c * dv + j];
    }
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) r[j] += kt[c] * Sn[(long)c * dv + j];
    for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) Sn[(long)c * dv + j] += kt[c] * u[j];
}

void kda_oracle_backward(int B, int T, int H, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *S0,
                         const double *dO, const double *dST,
                         double *dq, double *dk_out, double *dv_out, double *dg,
                         double *dbeta, double *dS0, int seg, int nthreads)
{
    const long BH = (long)B * H;
    const long SZ = (long)dk * dv;
    if (seg <= 0) seg = 64;
    const int nseg = (T + seg - 1) / seg;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    g_last_threads = nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
    g_last_threads = 1;
#endif
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *ck = (double *)malloc(sizeof(double) * (size_t)(nseg + 1) * SZ);  /* state before each segment */
        double *st = (double *)malloc(sizeof(double) * (size_t)(seg + 1) * SZ);   /* states inside a segment */
        double *dS = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *dSp = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dr = (double *)malloc(sizeof(double) * (size_t)dv);

        /* forward once, keeping the state at the start of every segment */
        if (S0) memcpy(ck, S0 + bh * SZ, sizeof(double) * (size_t)SZ);
        else    memset(ck, 0, sizeof(double) * (size_t)SZ);
        for (int s = 0; s < nseg; ++s) {
            memcpy(st, ck + (long)s * SZ, sizeof(double) * (size_t)SZ);
            const int t1 = (s + 1) * seg < T ? (s + 1) * seg : T;
            for (int t = s * seg; t < t1; ++t) {
                const long row = (b * T + t) * H + h;
                step_forward(dk, dv, q + row * dk, k + row * dk, v + row * dv, g + row * dk, beta[row],
                             st, st + SZ, r, u);
                memcpy(st, st + SZ, sizeof(double) * (size_t)SZ);
            }
            memcpy(ck + (long)(s + 1) * SZ, st, sizeof(double) * (size_t)SZ);
        }

        if (dST) memcpy(dS, dST + bh * SZ, sizeof(double) * (size_t)SZ);
        else     memset(dS, 0, sizeof(double) * (size_t)SZ);
        for (int s = nseg - 1; s >= 0; --s) {
            const int t0 = s * seg, t1 = (s + 1) * seg < T ? (s + 1) * seg : T;
            /* states st[i] before token t0 + i, for i = 0 .. t1 - t0 */
            memcpy(st, ck + (long)s * SZ, sizeof(double) * (size_t)SZ);
            for (int t = t0; t < t1; ++t) {
                const long row = (b * T + t) * H + h;
                step_forward(dk, dv, q + row * dk, k + row * dk, v + row * dv, g + row * dk, beta[row],
                             st + (long)(t - t0) * SZ, st + (long)(t - t0 + 1) * SZ, r, u);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const long row = (b * T + t) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv, *gt = g + row * dk;
                const double bt = beta[row];
                const double *S = st + (long)(t - t0) * SZ;        /* before the token */
                const double *Sn = st + (long)(t - t0 + 1) * SZ;   /* after the token  */
                const double *dot = dO ? dO + row * dv : NULL;
                /* recompute r, u of this token */
                for (int j = 0; j < dv; ++j) r[j] = 0.0;
                for (int c = 0; c < dk; ++c) {
                    const double a = exp(gt[c]);
                    for (int j = 0; j < dv; ++j) r[j] += kt[c] * a * S[(long)c * dv + j];
                }
                for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);
                /* o = S+^T q */
                if (dot) {
                    for (int c = 0; c < dk; ++c)
                        for (int j = 0; j < dv; ++j) dS[(long)c * dv + j] += qt[c] * dot[j];
                }
                if (dq) {
                    for (int c = 0; c < dk; ++c) {
                        double x = 0.0;
                        if (dot) for (int j = 0; j < dv; ++j) x += Sn[(long)c * dv + j] * dot[j];
                        dq[row * dk + c] = x;
                    }
                }
                /* S+ = S' + k u^T */
                for (int j = 0; j < dv; ++j) {
                    double x = 0.0;
                    for (int c = 0; c < dk; ++c) x += dS[(long)c * dv + j] * kt[c];
                    du[j] = x;
                }
                double dkc_acc;
                /* u = beta (v - r) */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    db += du[j] * (vt[j] - r[j]);
                    if (dv_out) dv_out[row * dv + j] = bt * du[j];
                    dr[j] = -bt * du[j];
                }
                if (dbeta) dbeta[row] = db;
                /* r = S'^T k ;  S' = Diag(a) S */
                for (int c = 0; c < dk; ++c) {
                    const double a = exp(gt[c]);
                    dkc_acc = 0.0;
                    double da = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const double sp = a * S[(long)c * dv + j];
                        dkc_acc += dS[(long)c * dv + j] * u[j] + sp * dr[j];
                        const double dsp = dS[(long)c * dv + j] + kt[c] * dr[j];
                        da += dsp * S[(long)c * dv + j];
                        dSp[(long)c * dv + j] = a * dsp;
                    }
                    if (dk_out) dk_out[row * dk + c] = dkc_acc;
                    if (dg) dg[row * dk + c] = da * a;
                }
                memcpy(dS, dSp, sizeof(double) * (size_t)SZ);
            }
        }
        if (dS0) memcpy(dS0 + bh * SZ, dS, sizeof(double) * (size_t)SZ);
        free(ck); free(st); free(dS); free(dSp); free(r); free(u); free(du); free(dr);
    }
}
