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
