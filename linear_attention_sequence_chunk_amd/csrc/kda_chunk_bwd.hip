// kda_chunk_bwd.hip -- backward pass of the chunkwise forward: the gradients of
// L = sum(dO * o) + sum(dS_T * S_T) with respect to q, k, v, g, beta and S0.
//
// The forward of one chunk (kda_chunk.h), with S its start state and S' its end
// state:  W = U - Wk S,  O = Qt S + P W,  S' = Diag(gam) S + Kb^T W.
// Its adjoint, given dO and the cotangent dS' of the end state, is
//   dW = Kb dS' + P^T dO,          dS = Diag(gam) dS' - Wk^T dW + Qt^T dO,
// a recurrence backwards over the chunks (chunk_bwd_chain_kernel), followed by
// work that is independent per chunk (chunk_bwd_intra_kernel):
//   dQt = dO S^T,  dWk = -dW S^T,  dKb = W dS'^T,  dgam_c = sum_j dS'_cj S_cj,
//   dP = lower(dO W^T),  dT = dW (beta V)^T + dWk (beta Kt)^T,
//   dV = beta T^T dW,  dKt = beta T^T dWk,  dM = -strict_lower(T^T dT T^T),
//   dA = beta dM,  dbeta = rows of (T^T dW) V + (T^T dWk) Kt + dM A,
// then through the decays Kt = e^G K, Qt = e^G Q, Kb = e^{G_C - G} K, gam =
// e^{G_C}, the pairwise decays inside A and P, and the prefix sum G of g.
// The forward state S and W of every chunk, and T and A, are kept by the forward
// stages run in their generic format (fp32 checkpoints).  All gradient
// arithmetic is fp32.
#include "kda_chunk.h"

namespace kda {

// ================================================================ reverse chain
// One workgroup of 256 threads per (sequence, head, slice of 32 value columns).
// Thread t owns column t % 32 and rows 16 (t / 32) .. + 15 of the slice's dS.
template <typename T, int DK, int DV, int C>
struct BwdChainCfg {
    static constexpr int DVS = 32, NSL = DV / DVS;
    static constexpr size_t OFF_KB = size_t(DK) * DVS * 4;                 // sS [DK][DVS]
    static constexpr size_t OFF_P = OFF_KB + size_t(DK) * C * 4;           // sKb [DK][C]
    static constexpr size_t OFF_WK = OFF_P + size_t(C) * C * 4;            // sP [C][C]
    static constexpr size_t OFF_QT = OFF_WK + size_t(C) * DK * 4;          // sWk [C][DK]
    static constexpr size_t OFF_DO = OFF_QT + size_t(C) * DK * 4;          // sQt [C][DK]
    static constexpr size_t OFF_DW = OFF_DO + size_t(C) * DVS * 4;         // sdO [C][DVS]
    static constexpr size_t OFF_G = OFF_DW + size_t(C) * DVS * 4;          // sdW [C][DVS]
    static constexpr size_t TOTAL = OFF_G + size_t(DK) * 4;                // sG [DK]
    static constexpr bool FITS = TOTAL <= LDS_LIMIT && DK * DVS % 256 == 0 && C * DVS % 256 == 0;
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void chunk_bwd_chain_kernel(
    const T* __restrict__ ws_qt, const T* __restrict__ ws_wk, const T* __restrict__ ws_kb,
    const T* __restrict__ ws_p, const float* __restrict__ ws_gam, const float* __restrict__ dO,
    const float* __restrict__ dST, float* __restrict__ dS0, float* __restrict__ ck_dS,
    float* __restrict__ ck_dW, UnitMap um) {
    typedef BwdChainCfg<T, DK, DV, C> Cfg;
    constexpr int DVS = Cfg::DVS, NSL = Cfg::NSL, RPT = DK * DVS / 256, WPT = C * DVS / 256;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    float* sS = reinterpret_cast<float*>(smem);
    float* sKb = reinterpret_cast<float*>(smem + Cfg::OFF_KB);
    float* sP = reinterpret_cast<float*>(smem + Cfg::OFF_P);
    float* sWk = reinterpret_cast<float*>(smem + Cfg::OFF_WK);
    float* sQt = reinterpret_cast<float*>(smem + Cfg::OFF_QT);
    float* sdO = reinterpret_cast<float*>(smem + Cfg::OFF_DO);
    float* sdW = reinterpret_cast<float*>(smem + Cfg::OFF_DW);
    float* sG = reinterpret_cast<float*>(smem + Cfg::OFF_G);

    const int tid = threadIdx.x;
    const long bh = blockIdx.x / NSL;
    const int sl = blockIdx.x % NSL, j0 = sl * DVS;
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int NC = sr.nchunks;
    const int j = tid % DVS, rb = (tid / DVS) * RPT;       // this thread's column and first row

    float ds[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) ds[m] = dST ? dST[(bh * DK + rb + m) * (long)DV + j0 + j] : 0.f;

    for (int n = NC - 1; n >= 0; --n) {
        const long unit = unit_id(um, sq, h, n, sr.chunk0);
        // the cotangent of this chunk's end state
        float* cds = ck_dS + unit * (long)DK * DV;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            cds[(rb + m) * (long)DV + j0 + j] = ds[m];
            sS[(rb + m) * DVS + j] = ds[m];
        }
        const T* gkb = ws_kb + unit * (long)DK * C;
        const T* gp = ws_p + unit * (long)C * C;
        const T* gwk = ws_wk + unit * (long)C * DK;
        const T* gqt = ws_qt + unit * (long)C * DK;
        for (int u = tid; u < DK * C; u += 256) {
            sKb[u] = to_f32(gkb[u]);
            sWk[u] = to_f32(gwk[u]);
            sQt[u] = to_f32(gqt[u]);
        }
        for (int u = tid; u < C * C; u += 256) sP[u] = to_f32(gp[u]);
        if (tid < DK) sG[tid] = ws_gam[unit * DK + tid];
        const long t0 = sr.tok_begin + (long)n * C;
        for (int u = tid; u < C * DVS; u += 256) {
            const int r = u / DVS, jj = u % DVS;
            sdO[u] = t0 + r < sr.tok_end ? dO[((t0 + r) * H + h) * DV + j0 + jj] : 0.f;
        }
        __syncthreads();

        // dW = Kb dS' + P^T dO   (Kb[r][c] = sKb[c][r];  P^T[r][i] = sP[i][r], zero above the diagonal)
        float* cdw = ck_dW + unit * (long)C * DV;
        const int wr = (tid / DVS) * WPT;
#pragma unroll
        for (int m = 0; m < WPT; ++m) {
            const int r = wr + m;
            float acc = 0.f;
            for (int c = 0; c < DK; ++c) acc += sKb[c * C + r] * sS[c * DVS + j];
            for (int i = r; i < C; ++i) acc += sP[i * C + r] * sdO[i * DVS + j];
            sdW[r * DVS + j] = acc;
            cdw[r * (long)DV + j0 + j] = acc;
        }
        __syncthreads();

        // dS = Diag(gam) dS' - Wk^T dW + Qt^T dO
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int c = rb + m;
            float acc = sG[c] * ds[m];
            for (int r = 0; r < C; ++r) acc += sQt[r * DK + c] * sdO[r * DVS + j] - sWk[r * DK + c] * sdW[r * DVS + j];
            ds[m] = acc;
        }
        __syncthreads();
    }
    if (dS0) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) dS0[(bh * DK + rb + m) * (long)DV + j0 + j] = ds[m];
    }
}

// ================================================================ per-chunk gradients
// One workgroup of 256 threads per chunk unit.  C x C matrices live in LDS; the
// C x DK intermediates go through per-unit scratch in the workspace.
template <int DK, int DV, int C>
struct BwdIntraCfg {
    static constexpr int NB = C / 16;
    static constexpr int DKT = 16;                                          // channels per tile (phase 5)
    static constexpr size_t SZ_CC = size_t(C) * C * 4;
    static constexpr size_t OFF_T = 0, OFF_A = SZ_CC, OFF_DP = 2 * SZ_CC, OFF_DT = 3 * SZ_CC;
    static constexpr size_t OFF_G = 4 * SZ_CC;                             // sG [C][DK]: prefix sums
    static constexpr size_t OFF_ST = OFF_G + size_t(C) * DK * 4;          // staging
    static constexpr int DM = DK > DV ? DK : DV;
    static constexpr size_t ST_FLOATS = size_t(C) * DM > size_t(6) * C * DKT ? size_t(C) * DM : size_t(6) * C * DKT;
    static constexpr size_t OFF_BETA = OFF_ST + ST_FLOATS * 4;
    static constexpr size_t OFF_DB = OFF_BETA + size_t(C) * 4;            // dbeta accumulators [C]
    static constexpr size_t OFF_DGM = OFF_DB + size_t(C) * 4;             // dgam [DK]
    static constexpr size_t TOTAL = OFF_DGM + size_t(DK) * 4;
    static constexpr bool FITS = TOTAL <= LDS_LIMIT;
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void chunk_bwd_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ dO,
    const float* __restrict__ ck_state, const float* __restrict__ ck_dS, const float* __restrict__ ck_w,
    const float* __restrict__ ck_dW, const float* __restrict__ ck_t, const float* __restrict__ ck_a,
    float* __restrict__ scr, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta, UnitMap um, int gate) {
    typedef BwdIntraCfg<DK, DV, C> Cfg;
    constexpr int NB = Cfg::NB, DKT = Cfg::DKT;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    float* sT = reinterpret_cast<float*>(smem + Cfg::OFF_T);
    float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
    float* sdP = reinterpret_cast<float*>(smem + Cfg::OFF_DP);
    float* sdT = reinterpret_cast<float*>(smem + Cfg::OFF_DT);
    float* sG = reinterpret_cast<float*>(smem + Cfg::OFF_G);
    float* sSt = reinterpret_cast<float*>(smem + Cfg::OFF_ST);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);
    float* sDb = reinterpret_cast<float*>(smem + Cfg::OFF_DB);
    float* sDgm = reinterpret_cast<float*>(smem + Cfg::OFF_DGM);

    const int tid = threadIdx.x;
    const long unit = blockIdx.x;
    UnitPos up;
    if (!unit_pos(um, unit, up)) return;
    const int H = um.H, h = up.h, cnt = up.count;
    const long tok0 = up.tok0;
    auto grow = [&](int t) -> long { return (tok0 + t) * H + h; };
    auto valid = [&](int t) -> bool { return t < cnt; };

    const float* S = ck_state + unit * (long)DK * DV;      // start state [DK][DV]
    const float* dSn = ck_dS + unit * (long)DK * DV;       // cotangent of the end state
    const float* W = ck_w + unit * (long)C * DV;
    const float* dW = ck_dW + unit * (long)C * DV;
    float* xdQt = scr + unit * (long)4 * C * DK;            // scratch: dQt, dWk, dKb, T^T dWk  [C][DK] each
    float* xdWk = xdQt + C * DK;
    float* xdKb = xdWk + C * DK;
    float* xTdWk = xdKb + C * DK;
    auto dOat = [&](int r, int jj) -> float { return valid(r) ? dO[grow(r) * DV + jj] : 0.f; };

    // ---- load T, A, beta; prefix sums G of the clamped log-gate (chunk-local)
    for (int u = tid; u < C * C; u += 256) {
        sT[u] = ck_t[unit * (long)C * C + u];
        sA[u] = ck_a[unit * (long)C * C + u];
    }
    if (tid < C) { sBeta[tid] = valid(tid) ? beta[grow(tid)] : 0.f; sDb[tid] = 0.f; }
    for (int c = tid; c < DK; c += 256) {
        float s = 0.f;
        for (int r = 0; r < C; ++r) {
            if (valid(r)) s += clamp_g(gate_at(g, gate, grow(r), DK, c));
            sG[r * DK + c] = s;
        }
    }
    __syncthreads();

    // ---- phase 1: contractions over the value channels
    // dP = lower(dO W^T);  dT = dW (beta V)^T (the dWk part is added in phase 3)
    for (int u = tid; u < C * C; u += 256) {
        const int r = u / C, i = u % C;
        float p = 0.f, t = 0.f;
        if (i <= r) {
            for (int jj = 0; jj < DV; ++jj) p += dOat(r, jj) * W[i * DV + jj];
            if (valid(i)) {
                for (int jj = 0; jj < DV; ++jj) t += dW[r * DV + jj] * to_f32(v[grow(i) * DV + jj]);
                t *= sBeta[i];
            }
        }
        sdP[u] = p;
        sdT[u] = t;
    }
    // dV = beta T^T dW;  dbeta += rows of (T^T dW) V (row sums in a fixed order)
    for (int u = tid; u < C * DV; u += 256) {
        const int r = u / DV, jj = u % DV;
        float x = 0.f;
        for (int i = r; i < C; ++i) x += sT[i * C + r] * dW[i * DV + jj];
        float pr = 0.f;
        if (valid(r)) {
            dv[grow(r) * DV + jj] = sBeta[r] * x;
            pr = x * to_f32(v[grow(r) * DV + jj]);
        }
        sSt[u] = pr;
    }
    __syncthreads();
    if (tid < C) {
        float x = 0.f;
        for (int jj = 0; jj < DV; ++jj) x += sSt[tid * DV + jj];
        sDb[tid] = x;
    }
    __syncthreads();
    // ---- phase 2: dQt = dO S^T, dWk = -dW S^T, dKb = W dS'^T, dgam = rows of dS' * S
    for (int u = tid; u < C * DK; u += 256) {
        const int r = u / DK, c = u % DK;
        float a = 0.f, b = 0.f, e = 0.f;
        for (int jj = 0; jj < DV; ++jj) {
            const float s = S[c * DV + jj];
            a += dOat(r, jj) * s;
            b += dW[r * DV + jj] * s;
            e += W[r * DV + jj] * dSn[c * DV + jj];
        }
        xdQt[u] = a;
        xdWk[u] = -b;
        xdKb[u] = e;
    }
    for (int c = tid; c < DK; c += 256) {
        float x = 0.f;
        for (int jj = 0; jj < DV; ++jj) x += dSn[c * DV + jj] * S[c * DV + jj];
        sDgm[c] = x;
    }
    // Kt = e^G K into the staging area
    for (int u = tid; u < C * DK; u += 256) {
        const int r = u / DK, c = u % DK;
        sSt[u] = valid(r) ? __expf(sG[u]) * to_f32(k[grow(r) * DK + c]) : 0.f;
    }
    __syncthreads();                                        // scratch, sdT, sSt complete

    // ---- phase 3: dT += dWk (beta Kt)^T;  T^T dWk;  dbeta += rows of (T^T dWk) Kt
    for (int u = tid; u < C * C; u += 256) {
        const int r = u / C, i = u % C;
        if (i <= r) {
            float t = 0.f;
            for (int c = 0; c < DK; ++c) t += xdWk[r * DK + c] * sSt[i * DK + c];
            sdT[u] += sBeta[i] * t;
        }
    }
    for (int u = tid; u < C * DK; u += 256) {
        const int r = u / DK, c = u % DK;
        float x = 0.f;
        for (int i = r; i < C; ++i) x += sT[i * C + r] * xdWk[i * DK + c];
        xTdWk[u] = x;
    }
    __syncthreads();
    if (tid < C) {                                          // dbeta += rows of (T^T dWk) Kt
        float x = 0.f;
        for (int c = 0; c < DK; ++c) x += xTdWk[tid * DK + c] * sSt[tid * DK + c];
        sDb[tid] += x;
    }
    __syncthreads();

    // ---- phase 4: dM = -strict_lower(T^T dT T^T);  X = T^T dT into the staging area
    for (int u = tid; u < C * C; u += 256) {
        const int r = u / C, i = u % C;
        float x = 0.f;
        for (int m = r; m < C; ++m) x += sT[m * C + r] * sdT[m * C + i];   // T lower: T^T[r][m] = T[m][r], m >= r
        sSt[u] = x;
    }
    __syncthreads();
    for (int u = tid; u < C * C; u += 256) {
        const int r = u / C, i = u % C;
        float x = 0.f;
        if (i < r) {
            for (int m = 0; m <= i; ++m) x += sSt[r * C + m] * sT[i * C + m];  // (X T^T)[r][i]: T[i][m], m <= i
        }
        sdT[u] = -x;                                                          // dM (strictly lower)
    }
    __syncthreads();
    // dbeta += rows of dM A;  dA = Diag(beta) dM (in place)
    if (tid < C) {
        float x = 0.f;
        for (int i = 0; i < C; ++i) x += sdT[tid * C + i] * sA[tid * C + i];
        sDb[tid] += x;
    }
    __syncthreads();
    for (int u = tid; u < C * C; u += 256) sdT[u] *= sBeta[u / C];
    __syncthreads();

    // ---- phase 5: per tile of DKT channels: decays, pairwise decays, prefix-sum adjoint.
    // Pairwise factors e^{G_r - G_i} (i <= r) are split at 16-row block boundaries
    // so that every stored factor is <= 1: with Gs(R) the prefix sum before block R
    // and Gm(I) the one at the end of block I,
    //   Er_r = e^{G_r - Gs(R(r))},  Ei_r = e^{Gm(R(r)) - G_r},  B_RI = e^{Gs(R) - Gm(I)} (I < R).
    // Inside one block, e^{G_r - G_i} = Er_r / Er_i, exact while the block's log-gate
    // sum stays above -SAFE_SPAN; otherwise that channel's block is done term by term.
    constexpr int NTILE = C * DKT;
    float* sEr = sSt;                      // [C][DKT] each
    float* sKm = sEr + NTILE;              // K Ei   (K scaled to its block end)
    float* sKs = sKm + NTILE;              // K Er
    float* sQs = sKs + NTILE;              // Q Er
    float* sKi = sQs + NTILE;              // K / Er (safe blocks)
    float* sdG = sKi + NTILE;              // dG, then dg
    static_assert(6 * NTILE <= Cfg::ST_FLOATS, "phase 5 staging");
    static_assert(NTILE % 256 == 0, "phase 5 thread mapping");
    for (int c0 = 0; c0 < DK; c0 += DKT) {
        for (int u = tid; u < NTILE; u += 256) {
            const int r = u / DKT, c = c0 + u % DKT, R = r / 16;
            const float G = sG[r * DK + c];
            const float Gs = R ? sG[(16 * R - 1) * DK + c] : 0.f, Gm = sG[(16 * R + 15) * DK + c];
            const float er = __expf(G - Gs), ei = __expf(Gm - G);
            const float kk = valid(r) ? to_f32(k[grow(r) * DK + c]) : 0.f;
            const float qq = valid(r) ? to_f32(q[grow(r) * DK + c]) : 0.f;
            sEr[u] = er;
            sKm[u] = kk * ei;
            sKs[u] = kk * er;
            sQs[u] = qq * er;
            sKi[u] = Gm - Gs >= -SAFE_SPAN ? kk / er : 0.f;
        }
        __syncthreads();
        {
            constexpr int RPT = NTILE / 256;
            const int cc = tid % DKT, c = c0 + cc, rq = (tid / DKT) * RPT;
            const float GC = sG[(C - 1) * DK + c];
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int r = rq + m, R = r / 16, u = r * DKT + cc;
                const float G = sG[r * DK + c], E = __expf(G), F = __expf(GC - G);
                const float Gs_R = R ? sG[(16 * R - 1) * DK + c] : 0.f, Gm_R = sG[(16 * R + 15) * DK + c];
                const float er = sEr[u];
                const float kc = valid(r) ? to_f32(k[grow(r) * DK + c]) : 0.f;
                const float qc = valid(r) ? to_f32(q[grow(r) * DK + c]) : 0.f;
                const float dKt = sBeta[r] * xTdWk[r * DK + c], dQt = xdQt[r * DK + c], dKb = xdKb[r * DK + c];
                float dK = E * dKt + F * dKb, dQ = E * dQt;
                float dG = E * kc * dKt + E * qc * dQt - F * kc * dKb;
                float XA = 0.f, XP = 0.f, YA = 0.f, YP = 0.f;
                for (int I = 0; I < R; ++I) {                      // earlier column blocks
                    const float Gm_I = sG[(16 * I + 15) * DK + c];
                    float xa = 0.f, xp = 0.f;
                    for (int i = 16 * I; i < 16 * I + 16; ++i) {
                        xa += sdT[r * C + i] * sKm[i * DKT + cc];
                        xp += sdP[r * C + i] * sKm[i * DKT + cc];
                    }
                    const float f = __expf(Gs_R - Gm_I);
                    XA += f * xa; XP += f * xp;
                }
                XA *= er; XP *= er;
                for (int I = R + 1; I < NB; ++I) {                 // later row blocks
                    const float Gs_I = sG[(16 * I - 1) * DK + c];
                    float ya = 0.f, yp = 0.f;
                    for (int rr = 16 * I; rr < 16 * I + 16; ++rr) {
                        ya += sdT[rr * C + r] * sKs[rr * DKT + cc];
                        yp += sdP[rr * C + r] * sQs[rr * DKT + cc];
                    }
                    const float f = __expf(Gs_I - Gm_R);
                    YA += f * ya; YP += f * yp;
                }
                YA *= __expf(Gm_R - G);
                YP *= __expf(Gm_R - G);
                // the diagonal block
                if (Gm_R - Gs_R >= -SAFE_SPAN) {
                    float xa = 0.f, xp = 0.f, ya = 0.f, yp = 0.f;
                    for (int i = 16 * R; i < 16 * R + 16; ++i) {
                        if (i < r) xa += sdT[r * C + i] * sKi[i * DKT + cc];
                        if (i <= r) xp += sdP[r * C + i] * sKi[i * DKT + cc];
                        if (i > r) ya += sdT[i * C + r] * sKs[i * DKT + cc];
                        if (i >= r) yp += sdP[i * C + r] * sQs[i * DKT + cc];
                    }
                    XA += er * xa; XP += er * xp;
                    YA += ya / er; YP += yp / er;
                } else {                                           // term by term
                    for (int i = 16 * R; i < 16 * R + 16; ++i) {
                        const float ki = valid(i) ? to_f32(k[grow(i) * DK + c]) : 0.f;
                        const float qi = valid(i) ? to_f32(q[grow(i) * DK + c]) : 0.f;
                        const float wd = __expf(G - sG[i * DK + c]), wu = __expf(sG[i * DK + c] - G);
                        if (i < r) XA += sdT[r * C + i] * ki * wd;
                        if (i <= r) XP += sdP[r * C + i] * ki * wd;
                        if (i > r) YA += sdT[i * C + r] * ki * wu;
                        if (i >= r) YP += sdP[i * C + r] * qi * wu;
                    }
                }
                dK += XA + YA + YP;
                dQ += XP;
                dG += kc * XA - kc * YA + qc * XP - kc * YP;
                if (valid(r)) {
                    dq[grow(r) * DK + c] = dQ;
                    dk[grow(r) * DK + c] = dK;
                }
                sdG[u] = dG;
            }
        }
        __syncthreads();
        // prefix-sum adjoint: dg_t = dG_C + sum_{r >= t} dG_r (G_C is the last row's
        // prefix sum; rows past the end of the sequence have g = 0 and add nothing)
        if (tid < DKT) {
            const int c = c0 + tid;
            const float GC = sG[(C - 1) * DK + c];
            float dGC = sDgm[c] * __expf(GC);                  // gam = e^{G_C}
            for (int r = 0; r < C; ++r) {                      // Kb = e^{G_C - G} K
                const float kr = valid(r) ? to_f32(k[grow(r) * DK + c]) : 0.f;
                dGC += __expf(GC - sG[r * DK + c]) * kr * xdKb[r * DK + c];
            }
            float run = dGC;
            for (int r = C - 1; r >= 0; --r) {
                run += sdG[r * DKT + tid];
                float gr = run;
                if (valid(r) && gate != GATE_NONE && gate_at(g, gate, grow(r), DK, c) < G_FLOOR) gr = 0.f;
                sdG[r * DKT + tid] = gr;                       // the forward floors the log-gate
            }
        }
        __syncthreads();
        if (gate == GATE_CHANNEL) {
            for (int u = tid; u < NTILE; u += 256) {
                const int r = u / DKT, c = c0 + u % DKT;
                if (valid(r)) dg[grow(r) * DK + c] = sdG[u];
            }
        } else if (gate == GATE_HEAD) {
            if (tid < C && valid(tid)) {
                float sum = 0.f;
                for (int cc = 0; cc < DKT; ++cc) sum += sdG[tid * DKT + cc];
                if (c0 == 0) dg[grow(tid)] = sum;
                else dg[grow(tid)] += sum;
            }
        }
        __syncthreads();
    }
    if (tid < C && valid(tid)) dbeta[grow(tid)] = sDb[tid];
}

// ================================================================ host side
template <typename T, int DK, int DV, int C>
static hipError_t launch_bwd(const BwdArgs& b) {
    typedef BwdChainCfg<T, DK, DV, C> CC;
    typedef BwdIntraCfg<DK, DV, C> IC;
    if constexpr (!CC::FITS || !IC::FITS) {
        return hipErrorInvalidValue;
    } else {
        const ChunkArgs& a = b.fwd;
        const WsLayout w = ws_layout_of(a);
        char* ws = (char*)a.ws;
        const long units = unit_count(a);
        const long nsh = seq_head_count(a);
        if (nsh == 0) return hipSuccess;
        hipLaunchKernelGGL((chunk_bwd_chain_kernel<T, DK, DV, C>), dim3((unsigned)(nsh * CC::NSL)), dim3(256), 0,
                           a.stream, (const T*)(ws + w.qt), (const T*)(ws + w.wk), (const T*)(ws + w.kb),
                           (const T*)(ws + w.p), (const float*)(ws + w.gam), b.dO, b.dST, b.dS0, b.ck_dS,
                           b.ck_dW, unit_map(a));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || units == 0) return e;
        hipLaunchKernelGGL((chunk_bwd_intra_kernel<T, DK, DV, C>), dim3((unsigned)units), dim3(256), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, b.dO, a.ck_state, b.ck_dS,
                           a.ck_w, b.ck_dW, a.ck_t, a.ck_a, b.scratch, b.dq, b.dk, b.dv, b.dg, b.dbeta,
                           unit_map(a), a.gate);
        return hipGetLastError();
    }
}

template <typename T, int DK, int DV>
static hipError_t bwd_c(const BwdArgs& b) {
    switch (b.fwd.C) {
        case 16: return launch_bwd<T, DK, DV, 16>(b);
        case 32: return launch_bwd<T, DK, DV, 32>(b);
        case 64: return launch_bwd<T, DK, DV, 64>(b);
        default: return hipErrorInvalidValue;
    }
}
template <typename T>
static hipError_t bwd_dims(const BwdArgs& b) {
    const ChunkArgs& a = b.fwd;
    if (a.dk == 64) return a.dv == 64 ? bwd_c<T, 64, 64>(b) : bwd_c<T, 64, 128>(b);
    return a.dv == 64 ? bwd_c<T, 128, 64>(b) : bwd_c<T, 128, 128>(b);
}

BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, bool in_bf16, int C) {
    BwdLayout L{};
    L.fwd = ws_layout(B, T, H, dk, dv, in_bf16, C, true);
    const size_t units = (size_t)B * H * (size_t)((T + C - 1) / C);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t off = al(L.fwd.total);
    L.t = off;     off = al(off + units * C * C * 4);
    L.a = off;     off = al(off + units * C * C * 4);
    L.state = off; off = al(off + units * dk * dv * 4);
    L.w = off;     off = al(off + units * C * dv * 4);
    L.dS = off;    off = al(off + units * dk * dv * 4);
    L.dW = off;    off = al(off + units * C * dv * 4);
    L.scr = off;   off = al(off + units * 4 * C * dk * 4);
    L.total = off;
    return L;
}

hipError_t run_chunk_bwd_stages(const BwdArgs& b) {
    return b.fwd.in_bf16 ? bwd_dims<bf16>(b) : bwd_dims<float>(b);
}

bool bwd_supported(int dk, int dv, int C, bool in_bf16) {
    (void)in_bf16;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return false;
    if (C != 16 && C != 32 && C != 64) return false;
#define KDA_BFIT(DK, DV, CC) if (dk == DK && dv == DV && C == CC) return BwdChainCfg<float, DK, DV, CC>::FITS && BwdIntraCfg<DK, DV, CC>::FITS;
    KDA_BFIT(64, 64, 16) KDA_BFIT(64, 64, 32) KDA_BFIT(64, 64, 64)
    KDA_BFIT(64, 128, 16) KDA_BFIT(64, 128, 32) KDA_BFIT(64, 128, 64)
    KDA_BFIT(128, 64, 16) KDA_BFIT(128, 64, 32) KDA_BFIT(128, 64, 64)
    KDA_BFIT(128, 128, 16) KDA_BFIT(128, 128, 32) KDA_BFIT(128, 128, 64)
#undef KDA_BFIT
    return false;
}

}  // namespace kda
