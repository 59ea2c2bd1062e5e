/*
 * kda_oracle.h -- fp64 CPU oracle for the gated delta-rule (KDA) state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this code; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source with the GPU library.
 *
 * Sources (web pages on Kimi Delta Attention; cited by title and section):
 *  - "一个KimiK3装下22580个GPT-2，七年缩放真正改变的是记忆与检索"
 *    (pwwt.cn/news/3716252): delta-rule paragraph (S <- S + k^T (v - S k)),
 *    Gated DeltaNet paragraph (alpha in [0,1]: 1 = pure delta, 0 = clear),
 *    Kimi Linear paragraph (one alpha per channel).
 *  - "我终于看懂了 KDA：百万 Token 的关键，不是记得更多，而是会修改记忆"
 *    (pwwt.cn/news/3787313): section 五 (additive memory M = M + key x value),
 *    section 六 (read old value, error = new - old, memory += lr * write(key,
 *    error)), section 八 (order: decay -> read -> error -> write), section 十五
 *    (serial recurrence State_t = Update(State_{t-1}, Token_t)).
 *
 * Notation (fixed by reading the pages together; see the readings list in the
 * design notes): per (batch b, head h) the state S is d_k x d_v, key channels
 * are rows, value channels are columns.  Per token t:
 *     S'  = Diag(exp(g_t)) S                (decay, per key channel)
 *     u_t = beta_t (v_t - S'^T k_t)         (read with the key, error, scaled)
 *     S   = S' + k_t u_t^T                  (write the correction along k_t)
 *     o_t = S^T q_t                         (output read after the write)
 *
 * Layouts are contiguous row-major: q,k,g [B,T,H,dk]; v [B,T,H,dv]; beta
 * [B,T,H]; S0, ST [B,H,dk,dv]; o [B,T,H,dv]; u_out [B,T,H,dv].
 * All arrays are fp64; callers upcast stored inputs exactly (bf16/fp32 -> fp64).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Sequential recurrence over t for every (b,h).  S0 may be NULL (zeros).
 * delta = 1: gated delta rule; delta = 0: the read term is dropped, giving the
 * beta-scaled additive (linear-attention) memory of section 五.
 * u_out may be NULL; when given it receives u_t for every token.
 * Parallel over (b,h) with OpenMP; the loop over t is sequential.  nthreads <= 0
 * means the OpenMP default. */
void kda_oracle_recurrent(int B, int T, int H, int dk, int dv,
                          const double *q, const double *k, const double *v,
                          const double *g, const double *beta,
                          const double *S0, double *o, double *ST,
                          int delta, double *u_out, int nthreads);

/* Number of threads the last kda_oracle_recurrent call ran with. */
int kda_oracle_last_threads(void);

/* Reverse-mode derivative (the adjoint) of kda_oracle_recurrent (delta = 1) for
 * the scalar  L = sum(dO * o) + sum(dST * S_T):  given the output cotangents dO
 * [B,T,H,dv] and dST [B,H,dk,dv] (either may be NULL: zeros), returns dq, dk, dg
 * [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H] and dS0 [B,H,dk,dv] (any output may
 * be NULL).  It applies, token by token in reverse order, the derivative of each
 * step of the recurrence (output read, write, error, read, decay).  States are
 * kept at every `seg`-th token and the states inside a segment are recomputed
 * from it (seg <= 0 means 64).  Parallel over (b,h) like the forward. */
void kda_oracle_backward(int B, int T, int H, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *S0,
                         const double *dO, const double *dST,
                         double *dq, double *dk_out, double *dv_out, double *dg,
                         double *dbeta, double *dS0, int seg, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
