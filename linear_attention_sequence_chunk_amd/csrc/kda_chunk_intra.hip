// kda_chunk_intra.hip -- stage 1 of the chunkwise forward (every chunk in
// parallel) and the host-side dispatch of both stages.  The method and the
// exponent-safety scheme are described in kda_chunk.h.
#include "kda_chunk.h"

namespace kda {

// Eight consecutive values of T as loaded; converted to fp32 (times a scale) where
// used, so that all of a thread's loads can be in flight at once.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    u32x4 x;
    __device__ __forceinline__ void load(const bf16* p) { x = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void get(float* o, float s) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(x[i] << 16) * s;
            o[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u) * s;
        }
    }
};
template <> struct Raw8<float> {
    floatx4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const floatx4*>(p);
        b = *reinterpret_cast<const floatx4*>(p + 4);
    }
    __device__ __forceinline__ void get(float* o, float s) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[i] = a[i] * s; o[4 + i] = b[i] * s; }
    }
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void chunk_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    T* __restrict__ ws_qt, T* __restrict__ ws_wk, T* __restrict__ ws_kb, T* __restrict__ ws_p,
    float* __restrict__ ws_u, float* __restrict__ ws_gam, UnitMap um, int gate,
    float* __restrict__ ck_t, float* __restrict__ ck_a) {
    // ck_t / ck_a (NULL in the forward pass): per unit, T and A in fp32 [C][C],
    // kept for the backward pass
    typedef IntraCfg<T, DK, DV, C> Cfg;
    constexpr int NB = Cfg::NB, NP = Cfg::NP, HR = Cfg::HR, LDK = Cfg::LDK, LDA = Cfg::LDA,
                  LDT = Cfg::LDT, CK = Cfg::CK;
    constexpr int KSTEP = Mma<T>::KSTEP;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    float* sL = reinterpret_cast<float*>(smem);
    T* sKrow = reinterpret_cast<T*>(smem + Cfg::SZ_L);
    T* sQrow = sKrow + HR * LDK;
    T* sKcol = sQrow + HR * LDK;
    float* sTot = reinterpret_cast<float*>(smem + Cfg::OFF_TOT);
    float* sOff = reinterpret_cast<float*>(smem + Cfg::OFF_OFF);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);
    int* sFlag = reinterpret_cast<int*>(smem + Cfg::OFF_FLAG);
    float* sQn = reinterpret_cast<float*>(smem + Cfg::OFF_QN);   // 1/||q_t||, 1/||k_t|| (or 1)
    float* sKn = sQn + C;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // chunk-major order (fixed-length batches): workgroups running together cover
    // all heads of the same tokens, so every token row of q, k, v, g is read whole
    const long ch = blockIdx.x;
    UnitPos up;
    if (!unit_pos(um, ch, up)) return;             // past the last chunk of a packed batch
    const int H = um.H, h = up.h, cnt = up.count;
    const long tok0 = up.tok0;
    auto grow = [&](int t) -> long { return (tok0 + t) * H + h; };
    auto valid = [&](int t) -> bool { return t < cnt; };
    // a row past the sequence end reads row 0 (the value is then dropped), so that
    // loads need no branch and can all be in flight together
    auto crow = [&](int t) -> long { return grow(t < cnt ? t : 0); };

    // ---------------------------------------------------------------- phase 0
    // Block-local inclusive prefix sums of the clamped log-gate (a1), block totals.
    if (tid < NB) sFlag[tid] = 0;
    if (tid < C) sBeta[tid] = valid(tid) ? beta[grow(tid)] : 0.f;
    if (gate & MODE_QK_L2NORM) {
        // inverse L2 norms of the q and k rows: 256 / C threads per row
        constexpr int TPR = 256 / C, CPT = DK / TPR;
        const int r = tid / TPR, c0 = (tid % TPR) * CPT;
        float sq = 0.f, sk = 0.f;
        if (valid(r)) {
            for (int c = c0; c < c0 + CPT; c += 2) {
                float q0, q1, k0, k1;
                Pair2<T>::load(q + grow(r) * DK + c, q0, q1);
                Pair2<T>::load(k + grow(r) * DK + c, k0, k1);
                sq += q0 * q0 + q1 * q1;
                sk += k0 * k0 + k1 * k1;
            }
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) { sq += __shfl_xor(sq, off); sk += __shfl_xor(sk, off); }
        if (tid % TPR == 0) { sQn[r] = inv_norm(sq); sKn[r] = inv_norm(sk); }
    } else if (tid < C) {
        sQn[tid] = 1.f;
        sKn[tid] = 1.f;
    }
    __syncthreads();
    for (int u = tid; u < NB * (DK / 2); u += 256) {
        const int R = u / (DK / 2), c = 2 * (u % (DK / 2));
        long rows[16];
        float2 gg[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) rows[rr] = crow(R * 16 + rr);
        gate_pair_rows<16>(g, gate, rows, DK, c, gg);
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int t = R * 16 + rr;
            if (valid(t)) {
                l0 += clamp_g(gg[rr].x);
                l1 += clamp_g(gg[rr].y);
            }
            *reinterpret_cast<float2*>(sL + t * DK + c) = make_float2(l0, l1);
        }
        sTot[R * DK + c] = l0;
        sTot[R * DK + c + 1] = l1;
        if (l0 < -SAFE_SPAN || l1 < -SAFE_SPAN) sFlag[R] = 1;
    }
    __syncthreads();

    floatx4 accA[Cfg::NSLOT], accP[Cfg::NSLOT];
#pragma unroll
    for (int s = 0; s < Cfg::NSLOT; ++s) { accA[s] = zero4(); accP[s] = zero4(); }

    // ---------------------------------------------------------------- phase S
    // This thread's q and k units (row t, 8 channels) for every level below, loaded
    // once: unit it is u = tid + 256 it of the C x (DK/8) units.
    constexpr int NU8 = C * (DK / 8), NIT8 = (NU8 + 255) / 256;
    Raw8<T> kraw[NIT8], qraw[NIT8];
#pragma unroll
    for (int it = 0; it < NIT8; ++it) {
        const int u = tid + 256 * it, uu = u < NU8 ? u : 0, t = uu / (DK / 8), c = 8 * (uu % (DK / 8));
        kraw[it].load(k + crow(t) * DK + c);
        qraw[it].load(q + crow(t) * DK + c);
    }
    // Cross levels: segment length n, split point in the middle.
    static_for<Cfg::NLV>([&](auto LV) {
        constexpr int SEG = C >> LV;
        constexpr int HALF = SEG / 2;
        // exponent offsets per (block, channel) relative to the split point
        for (int u = tid; u < NB * DK; u += 256) {
            const int R = u / DK, c = u % DK;
            const int seg = (R * 16) / SEG, M = (seg * SEG + HALF) / 16;
            float s = 0.f;
            if (R >= M) { for (int J = M; J < R; ++J) s += sTot[J * DK + c]; }
            else        { for (int J = R; J < M; ++J) s += sTot[J * DK + c]; }
            sOff[u] = s;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NIT8; ++it) {
            const int u = tid + 256 * it;
            if (NU8 % 256 != 0 && u >= NU8) continue;
            const int t = u / (DK / 8), c = 8 * (u % (DK / 8));
            const int R = t / 16, seg = t / SEG, w = t - seg * SEG;
            float L8[8], o8[8], kv[8], x[8];
            Vec8<float>::load(sL + t * DK + c, L8);
            Vec8<float>::load(sOff + R * DK + c, o8);
            kraw[it].get(kv, valid(t) ? sKn[t] : 0.f);
            if (w >= HALF) {                      // row side: e^{G_r - G_{m-1}} <= 1
                const int ri = seg * HALF + (w - HALF);
                float qv[8];
                qraw[it].get(qv, valid(t) ? sQn[t] : 0.f);
#pragma unroll
                for (int m = 0; m < 8; ++m) { const float e = __expf(o8[m] + L8[m]); x[m] = kv[m] * e; qv[m] *= e; }
                Vec8<T>::store(sKrow + ri * LDK + c, x);
                Vec8<T>::store(sQrow + ri * LDK + c, qv);
            } else {                              // column side: e^{G_{m-1} - G_i} <= 1
                const int ci = seg * HALF + w;
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = kv[m] * __expf(o8[m] - L8[m]);
                Vec8<T>::store(sKcol + ci * LDK + c, x);
            }
        }
        __syncthreads();
        static_for<NP>([&](auto PI) {
            constexpr int p = PI;
            if constexpr (pair_level(p) == SEG) {
                if (wave == p % 4) {
                    constexpr int R = pair_R(p), I = pair_I(p);
                    constexpr int segR = (R * 16) / SEG, segI = (I * 16) / SEG;
                    constexpr int ri0 = segR * HALF + (R * 16 - segR * SEG - HALF);
                    constexpr int ci0 = segI * HALF + (I * 16 - segI * SEG);
                    mma_tile2<T>(accA[p / 4], accP[p / 4], sKrow + ri0 * LDK, sQrow + ri0 * LDK, LDK,
                                 sKcol + ci0 * LDK, LDK, DK, lane);
                }
            }
        });
        __syncthreads();
    });

    // Diagonal sub-blocks, block start as reference, in passes of HR rows.
    static_for<Cfg::NPASS>([&](auto PS) {
        constexpr int r0 = PS * HR;
#pragma unroll
        for (int it = 0; it < NIT8; ++it) {           // this thread's units whose row is in the pass
            const int u = tid + 256 * it, t = u / (DK / 8), c = 8 * (u % (DK / 8));
            if (u >= NU8 || t < r0 || t >= r0 + HR) continue;
            const int tl = t - r0, R = t / 16;
            float L8[8], kv[8], qv[8], x[8];
            Vec8<float>::load(sL + t * DK + c, L8);
            kraw[it].get(kv, valid(t) ? sKn[t] : 0.f);
            qraw[it].get(qv, valid(t) ? sQn[t] : 0.f);
            float y[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) { const float e = __expf(L8[m]); x[m] = kv[m] * e; y[m] = qv[m] * e; }
            Vec8<T>::store(sKrow + tl * LDK + c, x);
            Vec8<T>::store(sQrow + tl * LDK + c, y);
            if (!sFlag[R]) {
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = kv[m] * __expf(-L8[m]);
                Vec8<T>::store(sKcol + tl * LDK + c, x);
            }
        }
        __syncthreads();
        static_for<NP>([&](auto PI) {
            constexpr int p = PI;
            constexpr int R = pair_R(p);
            if constexpr (pair_level(p) == 0 && R * 16 >= r0 && R * 16 < r0 + HR) {
                if (wave == p % 4) {
                    constexpr int rl = R * 16 - r0;
                    if (!sFlag[R]) {
                        mma_tile2<T>(accA[p / 4], accP[p / 4], sKrow + rl * LDK, sQrow + rl * LDK, LDK,
                                     sKcol + rl * LDK, LDK, DK, lane);
                    } else {
                        // term-by-term: e^{L_r - L_i} with both sums block-local, r >= i
                        const int i = R * 16 + (lane & 15);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = R * 16 + 4 * (lane >> 4) + e;
                            float sa = 0.f, sp = 0.f;
                            if (i <= r && valid(r)) {
                                for (int c = 0; c < DK; ++c) {
                                    const float w = __expf(sL[r * DK + c] - sL[i * DK + c]);
                                    const float ki = to_f32(k[grow(i) * DK + c]);
                                    sa += to_f32(k[grow(r) * DK + c]) * ki * w;
                                    sp += to_f32(q[grow(r) * DK + c]) * ki * w;
                                }
                            }
                            accA[p / 4][e] = i <= r && valid(r) ? sa * sKn[r] * sKn[i] : 0.f;
                            accP[p / 4][e] = i <= r && valid(r) ? sp * sQn[r] * sKn[i] : 0.f;
                        }
                    }
                }
            }
        });
        __syncthreads();
    });

    // ---------------------------------------------------------------- write A (as M = beta A) and P
    float* sA = reinterpret_cast<float*>(smem + Cfg::SZ_TB);
    T* gP = ws_p + ch * (long)C * C;
    for (int u = tid; u < C * C; u += 256) {
        const int r = u / C, i = u % C;
        if (r / 16 < i / 16) {
            sA[r * LDA + i] = 0.f; gP[u] = from_f32<T>(0.f);
            if (ck_a) ck_a[ch * (long)C * C + u] = 0.f;
        }
    }
    static_for<NP>([&](auto PI) {
        constexpr int p = PI;
        if (wave == p % 4) {
            constexpr int R = pair_R(p), I = pair_I(p);
            const int i = I * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = R * 16 + 4 * (lane >> 4) + e;
                float av = accA[p / 4][e], pv = accP[p / 4][e];
                if (R == I) { if (i >= r) av = 0.f; if (i > r) pv = 0.f; }
                sA[r * LDA + i] = sBeta[r] * av;
                gP[r * C + i] = from_f32<T>(pv);
                if (ck_a) ck_a[ch * (long)C * C + r * C + i] = av;
            }
        }
    });
    __syncthreads();

    // ---------------------------------------------------------------- phase T
    // T = (I + M)^-1 in place.  16x16 diagonal blocks by forward substitution (one
    // lane per column), then doubling: T21 = -T22 M21 T11 on fp32 MFMA.
    {
        const int bd = wave * 4 + (lane >> 4), j = lane & 15;
        if (bd < NB) {
            float* Mb = sA + (bd * 16) * LDA + bd * 16;
            float x[16];                 // right-looking: 15 dependent steps
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
                for (int r = i + 1; r < 16; ++r) x[r] -= Mb[r * LDA + i] * x[i];
#pragma unroll
            for (int r = 0; r < 16; ++r) Mb[r * LDA + j] = x[r];
        }
    }
    __syncthreads();
    float* sX = reinterpret_cast<float*>(smem);
    static_for<Cfg::NLV>([&](auto LH) {
        constexpr int HH = 16 << LH;             // size of the blocks being merged
        constexpr int NM = C / (2 * HH);
        constexpr int HT = HH / 16;
        constexpr int NTL = NM * HT * HT;
        constexpr int LDX = HH + 4;
        for (int tt = wave; tt < NTL; tt += 4) {
            const int m = tt / (HT * HT), a = (tt / HT) % HT, bc = tt % HT, base = m * 2 * HH;
            floatx4 acc = mma_f32_rowB(zero4(), sA + (base + HH + a * 16) * LDA + base, LDA,
                                       sA + base * LDA + base + bc * 16, LDA, HH, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sX[m * HH * LDX + (a * 16 + 4 * (lane >> 4) + e) * LDX + bc * 16 + (lane & 15)] = acc[e];
        }
        __syncthreads();
        for (int tt = wave; tt < NTL; tt += 4) {
            const int m = tt / (HT * HT), a = (tt / HT) % HT, bc = tt % HT, base = m * 2 * HH;
            floatx4 acc = mma_f32_rowB(zero4(), sA + (base + HH + a * 16) * LDA + base + HH, LDA,
                                       sX + m * HH * LDX + bc * 16, LDX, HH, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sA[(base + HH + a * 16 + 4 * (lane >> 4) + e) * LDA + base + bc * 16 + (lane & 15)] = -acc[e];
        }
        __syncthreads();
    });
    if (ck_t) {
        for (int u = tid; u < C * C; u += 256) ck_t[ch * (long)C * C + u] = sA[(u / C) * LDA + u % C];
    }

    // ---------------------------------------------------------------- phase W
    T* sTb = reinterpret_cast<T*>(smem);
    for (int u = tid; u < C * CK; u += 256) {
        const int r = u / CK, i = u % CK;
        sTb[r * LDT + i] = from_f32<T>(i < C ? sA[r * LDA + i] : 0.f);
    }
    __syncthreads();
    T* sVt = reinterpret_cast<T*>(smem + Cfg::SZ_TB);     // [DV][LDT]: beta_i v_ij
    T* sKt = sVt + DV * LDT;                                // [DK][LDT]: beta_i e^{G_i} k_i
    {
        constexpr int NUV = C * (DV / 8), NITV = (NUV + 255) / 256;
        Raw8<T> vraw[NITV];
#pragma unroll
        for (int it = 0; it < NITV; ++it) {
            const int u = tid + 256 * it, uu = u < NUV ? u : 0;
            vraw[it].load(v + crow(uu / (DV / 8)) * DV + 8 * (uu % (DV / 8)));
        }
#pragma unroll
        for (int it = 0; it < NITV; ++it) {
            const int u = tid + 256 * it;
            if (NUV % 256 != 0 && u >= NUV) continue;
            const int i = u / (DV / 8), j = 8 * (u % (DV / 8));
            float vv[8];
            vraw[it].get(vv, valid(i) ? sBeta[i] : 0.f);     // beta_i v_i (0 past the end)
#pragma unroll
            for (int m = 0; m < 8; ++m) sVt[(j + m) * LDT + i] = from_f32<T>(vv[m]);
        }
    }
    if constexpr (CK > C) {
        for (int u = tid; u < (DV + DK) * (CK - C); u += 256) {
            const int row = u / (CK - C), i = C + u % (CK - C);
            sVt[row * LDT + i] = from_f32<T>(0.f);
        }
    }
    T* gQt = ws_qt + ch * (long)C * DK;
    T* gKb = ws_kb + ch * (long)C * DK;
    for (int u = tid; u < NB * (DK / 2); u += 256) {
        const int R = u / (DK / 2), c = 2 * (u % (DK / 2));
        float in0 = 0.f, in1 = 0.f, out0 = 0.f, out1 = 0.f;   // G_{R,start} and G_last - G_{R,start}
        for (int J = 0; J < NB; ++J) {
            const float t0v = sTot[J * DK + c], t1v = sTot[J * DK + c + 1];
            if (J < R) { in0 += t0v; in1 += t1v; } else { out0 += t0v; out1 += t1v; }
        }
        long rows[16];
        float2 gg[16], kp[16], qp[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) rows[rr] = crow(R * 16 + rr);
        gate_pair_rows<16>(g, gate, rows, DK, c, gg);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            Pair2<T>::load(k + rows[rr] * DK + c, kp[rr].x, kp[rr].y);
            Pair2<T>::load(q + rows[rr] * DK + c, qp[rr].x, qp[rr].y);
        }
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int t = R * 16 + rr;
            float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f;
            if (valid(t)) {
                l0 += clamp_g(gg[rr].x); l1 += clamp_g(gg[rr].y);
                k0 = kp[rr].x * sKn[t]; k1 = kp[rr].y * sKn[t];
                q0 = qp[rr].x * sQn[t]; q1 = qp[rr].y * sQn[t];
            }
            const float ei0 = __expf(in0 + l0), ei1 = __expf(in1 + l1);
            const float eo0 = __expf(out0 - l0), eo1 = __expf(out1 - l1);
            const float bt = sBeta[t];
            sKt[c * LDT + t] = from_f32<T>(bt * k0 * ei0);
            sKt[(c + 1) * LDT + t] = from_f32<T>(bt * k1 * ei1);
            Pair2<T>::store(gQt + t * DK + c, q0 * ei0, q1 * ei1);
            gKb[c * C + t] = from_f32<T>(k0 * eo0);            // Kb stored transposed: [dk][C]
            gKb[(c + 1) * C + t] = from_f32<T>(k1 * eo1);
        }
    }
    if (tid < DK) {
        float s = 0.f;
        for (int J = 0; J < NB; ++J) s += sTot[J * DK + tid];
        ws_gam[ch * DK + tid] = __expf(s);
    }
    __syncthreads();
    constexpr int NTU = NB * (DV / 16), NTW = NB * (DK / 16);
    float* gU = ws_u + ch * (long)C * DV;
    T* gWk = ws_wk + ch * (long)C * DK;
    for (int tt = wave; tt < NTU + NTW; tt += 4) {
        const bool isU = tt < NTU;
        const int t2 = isU ? tt : tt - NTU;
        const int ncol = isU ? DV / 16 : DK / 16;
        const int R = t2 / ncol, J = t2 % ncol;
        const int K = ((16 * (R + 1) + KSTEP - 1) / KSTEP) * KSTEP;
        const T* bsrc = isU ? sVt + J * 16 * LDT : sKt + J * 16 * LDT;
        floatx4 acc = mma_tile<T>(zero4(), sTb + R * 16 * LDT, LDT, bsrc, LDT, K, lane);
        const int col = J * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = R * 16 + 4 * (lane >> 4) + e;
            if (isU) gU[row * DV + col] = acc[e];
            else gWk[row * DK + col] = from_f32<T>(acc[e]);
        }
    }
}

// ================================================================ stage 1, bf16 / C = 64 / dk = 128
// The hot configuration.  Same workspace contents as chunk_intra_kernel, stored in
// the MFMA fragment order that chunk_chain64_kernel reads (kda_chunk_chain64.hip).
//  - Inside each 16-token block the inclusive prefix sum L of the (floored)
//    log-gate is formed in registers with DPP row shifts: the 16 tokens of a
//    block sit in the 16 lanes of one DPP row.  E = e^{L} and F = e^{tot - L}
//    (tot the block sum) are both <= 1; every other decay factor is e^{sum of
//    block totals} <= 1, except e^{-L} which is only formed for blocks whose
//    total stays above -SAFE_SPAN.
//  - The sums are kept in base 2 (the log-gate scaled by log2 e as it enters the
//    prefix sum), so that every decay factor is a single v_exp_f32.
//  - The block index is uniform per wave; code that depends on it is
//    instantiated per block so that nothing indexes registers at run time.
//  - Two passes over halves of the key channels keep LDS under 80 KB so that
//    two workgroups share a CU; A and P accumulate across the passes.
//  - MFMA operand fragments are shared across the tiles a wave computes.
//  - The workspace goes out with streaming (nontemporal) stores: only a later
//    launch reads it, and dirty lines left in L2 would otherwise be written back
//    while the chain runs (mid workload: chain 0.205 -> 0.194 ms).
// Block pairs (R, I) and operands (Kr = k E, Kf = k F, Kd = k e^{-L}; b_J = e^{tot_J}):
//   (1,0) (3,2): Kr_R . Kf_I      (2,1): Kr_2 . Kf_1      (2,0): Kr_2 . (b_1 Kf_0)
//   (3,1): (b_2 Kr_3) . Kf_1      (3,0): (b_2 Kr_3) . (b_1 Kf_0)      (R,R): Kr_R . Kd_R
constexpr float LOG2E = 1.44269504088896341f;
constexpr float SAFE_SPAN2 = SAFE_SPAN * LOG2E;      // SAFE_SPAN in base-2 units
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), CTRL, 0xF, 0xF, true));
}
// lane N of each row of 16 lanes, to the whole row (DPP row_newbcast)
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}
// inclusive prefix sum within each row of 16 lanes (fuses into v_add_f32_dpp)
__device__ __forceinline__ float row_prefix_sum(float x) {
    x += dpp_or_zero<0x111>(x);   // row_shr:1
    x += dpp_or_zero<0x112>(x);   // row_shr:2
    x += dpp_or_zero<0x114>(x);   // row_shr:4
    x += dpp_or_zero<0x118>(x);   // row_shr:8
    return x;
}

// The transposed LDS arrays (rows of 64 positions, 16-byte units of 8) keep unit
// u of row r at unit u ^ swz8(r): lanes whose rows sit a multiple of 32 banks
// apart (rows 8 apart) then write different banks, with no data moved between
// registers.  Readers apply the same swizzle.
__device__ __forceinline__ int swz8(int row) { return 2 * ((row >> 3) & 3); }
// Writes the 8 bf16 of x to rows row0 .. row0+7 (row0 a multiple of 8) of column
// col of such an array (a transpose).
__device__ __forceinline__ void store_column8(bf16* base, int ld, int row0, int col, u32x4 x) {
    const int cs = (((col >> 3) ^ swz8(row0)) << 3) | (col & 7);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const unsigned int pr = x[m >> 1];
        const unsigned short hv = (unsigned short)((m & 1) ? (pr >> 16) : (pr & 0xFFFFu));
        *reinterpret_cast<unsigned short*>(base + (row0 + m) * ld + cs) = hv;
    }
}
__device__ __forceinline__ u32x4 pack_bf16x8(const float* x) {
    bf16x8 b;
#pragma unroll
    for (int m = 0; m < 8; ++m) b[m] = (bf16)x[m];
    return __builtin_bit_cast(u32x4, b);
}

template <int DV>
struct Intra64Cfg {
    static constexpr int C = 64, NB = 4, DK = 128, NT = 512, NW = 8, HALF = 64;
    static constexpr int LDH = HALF + 8;             // bf16 operand rows (one channel half)
    static constexpr int LDT = C + 8;                // bf16 rows over positions
    static constexpr int LDA = C + 8;                // fp32 rows of the C x C matrices
    static constexpr int NITV = C * DV / 8 / NT;     // v units per thread
    static constexpr size_t BLK = size_t(16) * LDH * 2;                 // one 16-row operand block
    // operand blocks: Kr 0-3, Qr 4-7, Kf 8-10 (blocks 0..2), Kd 11-14, Kr3' 15, Qr3' 16, Kf0' 17
    static constexpr size_t SZ_S = 18 * BLK;
    // after the score matrices (aliasing the operand blocks): M then T (fp32), later V^T
    static constexpr size_t OFF_A = 0;
    static constexpr size_t OFF_VT = 0;
    static constexpr size_t OFF_TB = size_t(C) * LDA * 4;
    static constexpr int LDP = C + 8;                // bf16 rows of the P / Kb^T / Wk staging
    static constexpr int LDW = DK + 8;
    static constexpr size_t OFF_PB = OFF_TB + size_t(C) * LDT * 2;      // P staging, then the T temp
    static constexpr size_t SZ_W = OFF_PB + size_t(C) * LDP * 2;
    static constexpr size_t OFF_KT = SZ_S > SZ_W ? SZ_S : SZ_W;         // (e^G k)^T [DK][LDT]
    static constexpr size_t OFF_KB = OFF_KT + size_t(DK) * LDT * 2;     // Kb^T staging [DK][LDP]
    static constexpr size_t OFF_TOT = OFF_KB + size_t(DK) * LDP * 2;
    static constexpr size_t OFF_BETA = OFF_TOT + size_t(NB) * DK * 4;
    static constexpr size_t OFF_NP = OFF_BETA + size_t(C) * 4;          // q, k sums of squares [2][2][C]
    static constexpr size_t TOTAL = OFF_NP + size_t(4) * C * 4;
    static_assert(size_t(DV) * LDT * 2 <= size_t(C) * LDA * 4, "V^T fits over M");
    static_assert(size_t(C / 2) * (C / 2 + 4) * 4 <= size_t(C) * LDP * 2, "T temp fits the P staging");
    static_assert(TOTAL <= 80 * 1024, "two workgroups per CU");
    static_assert(size_t(C) * LDW * 2 <= OFF_KT, "Wk staging");
    static_assert(NITV >= 1 && (C * DV / 8) % NT == 0 && (DV / 8) % 4 == 0, "v unit mapping");
};

// GEN: the backward pass's forward stage: the same workspace, plus the fp32
// checkpoints T and A per unit.
template <int DV, bool GEN, bool QKN>
__global__ __launch_bounds__(512, 4) void chunk_intra64_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    bf16* __restrict__ ws_qt, bf16* __restrict__ ws_wk, bf16* __restrict__ ws_kb, bf16* __restrict__ ws_p,
    void* __restrict__ ws_u, float* __restrict__ ws_gam, UnitMap um, int gate,
    float* __restrict__ ck_t, float* __restrict__ ck_a) {
    typedef Intra64Cfg<DV> Cfg;
    constexpr int C = 64, NB = 4, DK = 128, NT = 512, NW = 8, HALF = 64;
    constexpr int LDH = Cfg::LDH, LDT = Cfg::LDT, LDA = Cfg::LDA;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    bf16* sOp = reinterpret_cast<bf16*>(smem);
    bf16* sKtT = reinterpret_cast<bf16*>(smem + Cfg::OFF_KT);
    bf16* sKbT = reinterpret_cast<bf16*>(smem + Cfg::OFF_KB);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::OFF_TOT);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);
    float* sNp = reinterpret_cast<float*>(smem + Cfg::OFF_NP);   // [q|k][channel half][row]
    auto blk = [&](int b) { return sOp + b * 16 * LDH; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // chunk-major order (fixed-length batches): workgroups running together cover
    // all heads of the same tokens, so every token row of q, k, v, g is read whole
    const long ch = blockIdx.x;
    UnitPos up;
    if (!unit_pos(um, ch, up)) return;             // past the last chunk of a packed batch
    const int H = um.H, h = up.h, cnt = up.count;
    const long tok0 = up.tok0;
    auto grow = [&](int t) -> long { return (tok0 + t) * H + h; };
    auto valid = [&](int t) -> bool { return t < cnt; };

    // unit of pass p: wave -> (16-row block R, 32-channel group), lane -> (row, 8 channels)
    const int R = wave >> 1, rr = lane & 15, t = R * 16 + rr;
    auto chan = [&](int p) { return 64 * p + 32 * (wave & 1) + 8 * (lane >> 4); };

    // ---------------------------------------------------------------- loads
    // Every load is issued before any value is used, channel half 0 first: a row
    // past the sequence end reads row 0 and is zeroed afterwards, and the gate's
    // layout and storage are decided once per half.  Half 1 is decoded and masked
    // only when pass 0 is done with half 0, so its loads stay in flight meanwhile.
    const bool tok_ok = valid(t);
    const long trow = grow(tok_ok ? t : 0);
    const int glay = gate_layout(gate);
    bf16x8 qv[2], kv[2], vv[Cfg::NITV], g8[2];
    floatx4 ga[2], gb[2];
    // the per-head gate value, raw (no default value: a register written on one
    // path while a load into it is in flight on another makes the compiler wait)
    float gh32;
    bf16 gh16;
    auto load_half = [&](auto PI) {
        constexpr int p = PI;
        if (glay == GATE_CHANNEL && (gate & MODE_GATE_BF16)) {
            g8[p] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(g) + trow * DK + chan(p));
        } else if (glay == GATE_CHANNEL) {
            ga[p] = *reinterpret_cast<const floatx4*>(g + trow * DK + chan(p));
            gb[p] = *reinterpret_cast<const floatx4*>(g + trow * DK + chan(p) + 4);
        } else if (glay == GATE_HEAD && (gate & MODE_GATE_BF16)) {
            if constexpr (p == 0) gh16 = reinterpret_cast<const bf16*>(g)[trow];
        } else if (glay == GATE_HEAD) {
            if constexpr (p == 0) gh32 = g[trow];
        }
        qv[p] = *reinterpret_cast<const bf16x8*>(q + trow * DK + chan(p));
        kv[p] = *reinterpret_cast<const bf16x8*>(k + trow * DK + chan(p));
    };
    load_half(std::integral_constant<int, 0>{});
    load_half(std::integral_constant<int, 1>{});
    // v unit mapping: each group of 64 units covers 16 tokens x 4 groups of 8 channels
    auto vunit = [&](int it, int& tv, int& j) {
        const int u = tid + NT * it, w = u >> 6, l = u & 63;
        tv = (w & 3) * 16 + (l & 15);
        j = 8 * ((w >> 2) * 4 + (l >> 4));
    };
#pragma unroll
    for (int it = 0; it < Cfg::NITV; ++it) {
        int tv, j;
        vunit(it, tv, j);
        vv[it] = *reinterpret_cast<const bf16x8*>(v + grow(valid(tv) ? tv : 0) * DV + j);
    }
    const float bt = beta[grow(tid < C && valid(tid) ? tid : 0)];
    // decode and mask channel half p (just before its values are first used)
    auto prep_half = [&](auto PI) {
        constexpr int p = PI;
        if (glay == GATE_CHANNEL && (gate & MODE_GATE_BF16)) {
            ga[p] = floatx4{(float)g8[p][0], (float)g8[p][1], (float)g8[p][2], (float)g8[p][3]};
            gb[p] = floatx4{(float)g8[p][4], (float)g8[p][5], (float)g8[p][6], (float)g8[p][7]};
        } else if (glay == GATE_HEAD) {
            const float gh = (gate & MODE_GATE_BF16) ? (float)gh16 : gh32;
            ga[p] = floatx4{gh, gh, gh, gh};
            gb[p] = ga[p];
        } else if (glay != GATE_CHANNEL) {
            ga[p] = zero4();
            gb[p] = zero4();
        }
        if (glay != GATE_NONE && (gate & MODE_GATE_SOFTPLUS)) {
#pragma unroll
            for (int m = 0; m < 4; ++m) { ga[p][m] = neg_softplus(ga[p][m]); gb[p][m] = neg_softplus(gb[p][m]); }
        }
        if (!tok_ok) {
#pragma unroll
            for (int m = 0; m < 8; ++m) { qv[p][m] = (bf16)0.f; kv[p][m] = (bf16)0.f; }
            ga[p] = zero4();
            gb[p] = zero4();
        }
    };
    prep_half(std::integral_constant<int, 0>{});
    // q and k row norms (pre-processing): a token's 128 channels are spread over the
    // four lane groups of this wave and the partner wave (wave ^ 1)
    constexpr bool qknorm = QKN;                      // the MODE_QK_L2NORM flag, as a constant
    if (qknorm) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float a = (float)qv[p][m], b = (float)kv[p][m];
                sq += a * a;
                sk += b * b;
            }
        if (!tok_ok) { sq = 0.f; sk = 0.f; }            // half 1 is masked later
        sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
        sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
        if (lane < 16) {
            sNp[(wave & 1) * C + t] = sq;
            sNp[2 * C + (wave & 1) * C + t] = sk;
        }
    }

    // ---------------------------------------------------------------- a1: block-local log-gate sums
    float Lg[2][8];
    auto a1_half = [&](int p) {
#pragma unroll
        for (int m = 0; m < 8; ++m) Lg[p][m] = row_prefix_sum(clamp_g(m < 4 ? ga[p][m] : gb[p][m - 4]) * LOG2E);
        if (rr == 15) {
#pragma unroll
            for (int m = 0; m < 8; ++m) sTot[R * DK + chan(p) + m] = Lg[p][m];
        }
    };
    a1_half(0);                                        // half 1 follows pass 0's a2
    __syncthreads();
    auto qn = [&](int r) { return inv_norm(sNp[r] + sNp[C + r]); };          // 1/||q_r||
    auto kn = [&](int r) { return inv_norm(sNp[2 * C + r] + sNp[3 * C + r]); };  // 1/||k_r||
    const float iqn = qknorm ? qn(t) : 1.f, ikn = qknorm ? kn(t) : 1.f;

    // ---------------------------------------------------------------- a2 + a3 per channel half
    bf16* gQt = ws_qt + ch * (long)C * DK;
    bf16* gKb = ws_kb + ch * (long)DK * C;
    floatx4 accA[2], accP[2];
    accA[0] = accA[1] = accP[0] = accP[1] = zero4();
    // pair assignment: w0 (0,0); w1 (1,0)(1,1); w2 (2,0)(2,1); w3 (2,2); w4 (3,0)(3,1); w5 (3,2)(3,3)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = chan(p), cl = c - 64 * p;
        static_for<NB>([&](auto RI) {
            constexpr int RB = RI;                     // this wave's block, as a constant
            if (R != RB) return;
            float tR[8], kr[8], qr[8], kf[8], o1[8], o2[8];
            Vec8<float>::load(sTot + RB * DK + c, tR);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float E = exp2_fast(Lg[p][m]), F = exp2_fast(tR[m] - Lg[p][m]);
                const float kk = (float)kv[p][m] * ikn, qq = (float)qv[p][m] * iqn;
                kr[m] = kk * E; qr[m] = qq * E; kf[m] = kk * F;
            }
            Vec8<bf16>::store(blk(RB) + rr * LDH + cl, kr);
            Vec8<bf16>::store(blk(4 + RB) + rr * LDH + cl, qr);
            if constexpr (RB < 3) Vec8<bf16>::store(blk(8 + RB) + rr * LDH + cl, kf);
            // Factors that depend on the channel only, shared by the block's 16 rows:
            //   D = e^{-tot_RB} (0 where the block is unsafe),
            //   X = e^{sum_{J<RB} tot_J}, or e^{tot_1} for RB = 0,
            //   Y = e^{sum_{J>RB} tot_J}, or e^{tot_2} for RB = 3.
            // Lane rr of each 16-lane row forms two of the row's 24 (channel rr % 8):
            // fa holds D (lanes 0-7) or X (lanes 8-15), fb holds Y; DPP row
            // broadcasts hand each lane the ones it needs where it needs them.
            float fa, fb;
            {
                const int cm = c + (rr & 7);
                const float t0 = sTot[cm], t1 = sTot[DK + cm], t2 = sTot[2 * DK + cm], t3 = sTot[3 * DK + cm];
                const float tb = RB == 0 ? t0 : RB == 1 ? t1 : RB == 2 ? t2 : t3;
                const float ax = RB == 0 ? t1 : RB == 1 ? t0 : RB == 2 ? t0 + t1 : t0 + t1 + t2;
                const float ay = RB == 0 ? t1 + t2 + t3 : RB == 1 ? t2 + t3 : RB == 2 ? t3 : t2;
                const float ad = tb >= -SAFE_SPAN2 ? -tb : -INFINITY;
                fa = exp2_fast(rr < 8 ? ad : ax);
                fb = exp2_fast(ay);
            }
            static_for<8>([&](auto MI) {                                 // k e^{-L}, safe blocks only
                constexpr int M = MI;
                o1[M] = kf[M] * row_bcast<M>(fa);
            });
            Vec8<bf16>::store(blk(11 + RB) + rr * LDH + cl, o1);
            if constexpr (RB == 3) {
                static_for<8>([&](auto MI) {
                    constexpr int M = MI;
                    const float y = row_bcast<M>(fb);
                    o1[M] = kr[M] * y;
                    o2[M] = qr[M] * y;
                });
                Vec8<bf16>::store(blk(15) + rr * LDH + cl, o1);
                Vec8<bf16>::store(blk(16) + rr * LDH + cl, o2);
            }
            if constexpr (RB == 0) {
                static_for<8>([&](auto MI) {
                    constexpr int M = MI;
                    o1[M] = kf[M] * row_bcast<8 + M>(fa);
                });
                Vec8<bf16>::store(blk(17) + rr * LDH + cl, o1);
            }
            // e^G = E e^{sum_{J<R} tot_J};  e^{G_last - G} = F e^{sum_{J>R} tot_J}
            static_for<8>([&](auto MI) {
                constexpr int M = MI;
                const float eb = RB > 0 ? row_bcast<8 + M>(fa) : 1.f, er = RB < 3 ? row_bcast<M>(fb) : 1.f;
                o1[M] = qr[M] * eb;
                kr[M] *= eb;
                kf[M] *= er;
            });
            store_column8(sKtT, LDT, c, t, pack_bf16x8(kr));
            store_column8(sKbT, Cfg::LDP, c, t, pack_bf16x8(kf));
            // fragment order: unit (row tile R, k-step c/32), lane = row%16 + 16 * ((c%32)/8)
            Vec8<bf16>::store_nt(gQt + ((R * 4 + (c >> 5)) * 64 + lane) * 8, o1);
        });
        if (p == 0) {                                  // channel half 1, and beta
            prep_half(std::integral_constant<int, 1>{});
            a1_half(1);
            if (tid < C) sBeta[tid] = valid(tid) ? bt : 0.f;
        }
        if (p == 1 && tid < DK) {
            float lg = 0.f;
#pragma unroll
            for (int J = 0; J < NB; ++J) lg += sTot[J * DK + tid];
            ws_gam[ch * DK + tid] = exp2_fast(lg);
        }
        __syncthreads();

        if (p == 1) {                                  // Kb^T complete: to the workspace in fragment order
            for (int u = tid; u < DK * C / 8; u += NT) {
                const int ctile = u >> 7, ks = (u >> 6) & 1, lf = u & 63;
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(
                    sKbT + (ctile * 16 + (lf & 15)) * Cfg::LDP + 8 * ((ks * 4 + (lf >> 4)) ^ swz8(ctile * 16 + (lf & 15)))),
                    reinterpret_cast<u32x4*>(gKb) + u);
            }
        }
        // A and P over this channel half (K = 64: two MFMA steps)
        if (wave < 6) {
            const int Rw = wave == 0 ? 0 : (wave <= 2 ? wave : (wave == 3 ? 2 : 3));
            const int npair = (wave == 0 || wave == 3) ? 1 : 2;
            // operands
            const bf16 *rk0, *rq0, *ck0, *ck1 = nullptr, *rk1 = nullptr, *rq1 = nullptr;
            if (wave == 0)      { rk0 = blk(0);  rq0 = blk(4);  ck0 = blk(11); }
            else if (wave == 1) { rk0 = blk(1);  rq0 = blk(5);  ck0 = blk(8);  ck1 = blk(12); }
            else if (wave == 2) { rk0 = blk(2);  rq0 = blk(6);  ck0 = blk(17); ck1 = blk(9); }
            else if (wave == 3) { rk0 = blk(2);  rq0 = blk(6);  ck0 = blk(13); }
            else if (wave == 4) { rk0 = blk(15); rq0 = blk(16); ck0 = blk(17); ck1 = blk(9); }
            else                { rk0 = blk(3);  rq0 = blk(7);  ck0 = blk(10); ck1 = blk(14); }
            (void)Rw; (void)rk1; (void)rq1;
            // a diagonal tile whose block total underflows is done term by term below
            const int dslot = (wave == 0 || wave == 3) ? 0 : ((wave == 1 || wave == 5) ? 1 : -1);
            const int dR = wave == 0 ? 0 : wave == 1 ? 1 : wave == 3 ? 2 : 3;
            bool uns = false;
            if (dslot >= 0) {
                uns = sTot[dR * DK + lane] < -SAFE_SPAN2 || sTot[dR * DK + 64 + lane] < -SAFE_SPAN2;
                uns = __any(uns);
            }
            const int r = lane & 15, kg = lane >> 4;
#pragma unroll
            for (int k0 = 0; k0 < HALF; k0 += 32) {
                const int o = r * LDH + k0 + 8 * kg;
                const bf16x8 fk = *reinterpret_cast<const bf16x8*>(rk0 + o);
                const bf16x8 fq = *reinterpret_cast<const bf16x8*>(rq0 + o);
                const bf16x8 fc0 = *reinterpret_cast<const bf16x8*>(ck0 + o);
                if (!(uns && dslot == 0)) {
                    accA[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk, fc0, accA[0], 0, 0, 0);
                    accP[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq, fc0, accP[0], 0, 0, 0);
                }
                if (npair == 2) {
                    const bf16x8 fc1 = *reinterpret_cast<const bf16x8*>(ck1 + o);
                    if (!(uns && dslot == 1)) {
                        accA[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk, fc1, accA[1], 0, 0, 0);
                        accP[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq, fc1, accP[1], 0, 0, 0);
                    }
                }
            }
            if (uns && p == 1) {
                // term by term over all channels: prod_{j=i+1..r} alpha_j, from global memory
                const int i = dR * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rw = dR * 16 + 4 * (lane >> 4) + e;
                    float sa = 0.f, sp = 0.f;
                    if (i <= rw && valid(rw)) {
                        for (int cc = 0; cc < DK; ++cc) {
                            float w = 1.f;
                            for (int j = i + 1; j <= rw; ++j) w *= __expf(clamp_g(gate_at(g, gate, grow(j), DK, cc)));
                            const float ki = (float)k[grow(i) * DK + cc];
                            sa += (float)k[grow(rw) * DK + cc] * ki * w;
                            sp += (float)q[grow(rw) * DK + cc] * ki * w;
                        }
                        if (qknorm) { sa *= kn(rw) * kn(i); sp *= qn(rw) * kn(i); }
                    }
                    if (dslot == 0) { accA[0][e] = sa; accP[0][e] = sp; }
                    else            { accA[1][e] = sa; accP[1][e] = sp; }
                }
            }
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- M = Diag(beta) A, P
    float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
    bf16* sPb = reinterpret_cast<bf16*>(smem + Cfg::OFF_PB);
    for (int u = tid; u < 6 * 256; u += NT) {          // the six strictly-upper 16x16 blocks
        const int bi = u >> 8, e = u & 255;
        const int br = bi < 3 ? 0 : (bi < 5 ? 1 : 2);
        const int bc = bi < 3 ? bi + 1 : (bi < 5 ? bi - 1 : 3);
        const int r = br * 16 + (e >> 4), i = bc * 16 + (e & 15);
        sA[r * LDA + i] = 0.f;
        sPb[r * Cfg::LDP + i] = (bf16)0.f;                // (A's checkpoint: only the lower blocks are read)
    }
    if (wave < 6) {
        const int np = (wave == 0 || wave == 3) ? 1 : 2;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s >= np) break;
            int PR, PI;
            if (wave == 0) { PR = 0; PI = 0; }
            else if (wave == 1) { PR = 1; PI = s; }
            else if (wave == 2) { PR = 2; PI = s; }
            else if (wave == 3) { PR = 2; PI = 2; }
            else if (wave == 4) { PR = 3; PI = s; }
            else { PR = 3; PI = 2 + s; }
            const int i = PI * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = PR * 16 + 4 * (lane >> 4) + e;
                float av = accA[s][e], pv = accP[s][e];
                if (PR == PI) { if (i >= r) av = 0.f; if (i > r) pv = 0.f; }
                sA[r * LDA + i] = sBeta[r] * av;
                sPb[r * Cfg::LDP + i] = (bf16)pv;
                if constexpr (GEN) ck_a[ch * (long)(C * C) + r * C + i] = av;
            }
        }
    }
    __syncthreads();
    {
        u32x4* gP = reinterpret_cast<u32x4*>(ws_p + ch * (long)C * C);
        // fragment order; the two blocks above the diagonal (row tiles 0, 1 at k-step 1) are not stored
        if (tid < 6 * 64) {
            const int bi = tid >> 6, lf = tid & 63;
            const int Rt = bi < 2 ? bi : 2 + (bi - 2) / 2, ks = bi < 2 ? 0 : (bi - 2) % 2;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(
                sPb + (Rt * 16 + (lf & 15)) * Cfg::LDP + ks * 32 + 8 * (lf >> 4)), gP + (Rt * 2 + ks) * 64 + lf);
        }
    }

    // ---------------------------------------------------------------- a4: T = (I + M)^-1
    if (wave == 0) {
        // column j of one diagonal block's inverse by forward substitution, in the
        // right-looking order: once x_i is final it updates every later row, so
        // the updates of one step are independent (15 dependent steps, not 120)
        const int bd = lane >> 4, j = lane & 15;
        float* Mb = sA + (bd * 16) * LDA + bd * 16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 15; ++i)
#pragma unroll
            for (int r = i + 1; r < 16; ++r) x[r] -= Mb[r * LDA + i] * x[i];
#pragma unroll
        for (int r = 0; r < 16; ++r) Mb[r * LDA + j] = x[r];
    }
    __syncthreads();
    float* sX = reinterpret_cast<float*>(smem + Cfg::OFF_PB);
    static_for<2>([&](auto LH) {
        constexpr int HH = 16 << LH, NM = C / (2 * HH), HT = HH / 16, NTL = NM * HT * HT, LDX = HH + 4;
        if (wave < NTL) {
            const int tt2 = wave;
            const int m = tt2 / (HT * HT), a = (tt2 / HT) % HT, bc = tt2 % HT, base = m * 2 * HH;
            floatx4 acc = mma_f32_rowB(zero4(), sA + (base + HH + a * 16) * LDA + base, LDA,
                                       sA + base * LDA + base + bc * 16, LDA, HH, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sX[m * HH * LDX + (a * 16 + 4 * (lane >> 4) + e) * LDX + bc * 16 + (lane & 15)] = acc[e];
        }
        __syncthreads();
        if (wave < NTL) {
            const int tt2 = wave;
            const int m = tt2 / (HT * HT), a = (tt2 / HT) % HT, bc = tt2 % HT, base = m * 2 * HH;
            floatx4 acc = mma_f32_rowB(zero4(), sA + (base + HH + a * 16) * LDA + base + HH, LDA,
                                       sX + m * HH * LDX + bc * 16, LDX, HH, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sA[(base + HH + a * 16 + 4 * (lane >> 4) + e) * LDA + base + bc * 16 + (lane & 15)] = -acc[e];
        }
        __syncthreads();
    });

    if constexpr (GEN) {                               // T, for the backward pass: its lower blocks
        for (int u = tid; u < C * C; u += NT)
            if (((u & 63) >> 4) <= (u >> 10)) ck_t[ch * (long)(C * C) + u] = sA[(u >> 6) * LDA + (u & 63)];
    }

    // ---------------------------------------------------------------- U = (T Diag(beta)) V, Wk = (T Diag(beta)) e^G K
    bf16* sTb = reinterpret_cast<bf16*>(smem + Cfg::OFF_TB);
    bf16* sVt = reinterpret_cast<bf16*>(smem + Cfg::OFF_VT);
    for (int u = tid; u < C * C / 2; u += NT) {
        const int r = u / (C / 2), i = 2 * (u % (C / 2));
        bf16x2 pr;
        pr[0] = (bf16)(sA[r * LDA + i] * sBeta[i]);
        pr[1] = (bf16)(sA[r * LDA + i + 1] * sBeta[i + 1]);
        *reinterpret_cast<bf16x2*>(sTb + r * LDT + i) = pr;
    }
    __syncthreads();                                   // M / T dead: V^T goes over it
#pragma unroll
    for (int it = 0; it < Cfg::NITV; ++it) {
        int tv, j;
        vunit(it, tv, j);
        if (!valid(tv)) {
#pragma unroll
            for (int m = 0; m < 8; ++m) vv[it][m] = (bf16)0.f;
        }
        store_column8(sVt, LDT, j, tv, __builtin_bit_cast(u32x4, vv[it]));
    }
    __syncthreads();
    {
        constexpr int NUT = DV / 16, NCT = NUT + DK / 16;        // column tiles: U then Wk
        bf16* gU = reinterpret_cast<bf16*>(ws_u) + ch * (long)C * DV;
        bf16* gW = ws_wk + ch * (long)C * DK;
        const int r = lane & 15, kg = lane >> 4;
        constexpr int NTPW = (NCT + NW - 1) / NW;                  // column tiles per wave
        floatx4 acc[NTPW][4];
#pragma unroll
        for (int sct = 0; sct < NTPW; ++sct) {
            const int ct = wave + NW * sct;
#pragma unroll
            for (int R2 = 0; R2 < 4; ++R2) acc[sct][R2] = zero4();
            if (ct < NCT) {
                const bool isU = ct < NUT;
                const int brow = (isU ? ct : ct - NUT) * 16 + r;      // row of V^T or (e^G k)^T
                const bf16* bsrc = (isU ? sVt : sKtT) + brow * LDT;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += 32) {
                    const bf16x8 fb = *reinterpret_cast<const bf16x8*>(bsrc + 8 * (((k0 >> 3) + kg) ^ swz8(brow)));
#pragma unroll
                    for (int R2 = 0; R2 < 4; ++R2) {
                        if (k0 >= 16 * (R2 + 1)) continue;              // T is lower triangular
                        const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sTb + (R2 * 16 + r) * LDT + k0 + 8 * kg);
                        acc[sct][R2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[sct][R2], 0, 0, 0);
                    }
                }
            }
        }
        // U goes out straight from the accumulators, in bf16: tile (row tile, column
        // tile) as [64 lanes][4]
#pragma unroll
        for (int sct = 0; sct < NTPW; ++sct) {
            const int ct = wave + NW * sct;
            if (ct < NUT) {
#pragma unroll
                for (int R2 = 0; R2 < 4; ++R2) {
                    bf16x4 u4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) u4[e] = (bf16)acc[sct][R2][e];
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, u4), reinterpret_cast<u32x2*>(gU) + (R2 * (DV / 16) + ct) * 64 + lane);
                }
            }
        }
        __syncthreads();                               // operands read by every wave: staging may overwrite them
        bf16* sWo = reinterpret_cast<bf16*>(smem);
#pragma unroll
        for (int sct = 0; sct < NTPW; ++sct) {
            const int ct = wave + NW * sct;
            if (ct < NUT || ct >= NCT) continue;
            const int col = (ct - NUT) * 16 + (lane & 15);
#pragma unroll
            for (int R2 = 0; R2 < 4; ++R2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sWo[(R2 * 16 + 4 * (lane >> 4) + e) * Cfg::LDW + col] = (bf16)acc[sct][R2][e];
            }
        }
        __syncthreads();
        for (int u = tid; u < C * DK / 8; u += NT) {  // Wk in fragment order
            const int Rt = u >> 8, ks = (u >> 6) & 3, lf = u & 63;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(
                sWo + (Rt * 16 + (lf & 15)) * Cfg::LDW + ks * 32 + 8 * (lf >> 4)), reinterpret_cast<u32x4*>(gW) + u);
        }
    }
}

// ================================================================ host side
static inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout layout_units(size_t nch, size_t header, int dk, int dv, bool in_bf16, int C) {
    WsLayout w{};
    const size_t es = in_bf16 ? 2 : 4;
    size_t off = 0;
    w.cu = off; off = al256(off + header);
    w.qt = off; off = al256(off + nch * C * dk * es);
    w.wk = off; off = al256(off + nch * C * dk * es);
    w.kb = off; off = al256(off + nch * C * dk * es);
    w.p = off;  off = al256(off + nch * C * C * es);
    w.u = off;  off = al256(off + nch * C * dv * (hot_config(in_bf16, dk, C) ? 2 : 4));
    w.gam = off; off = al256(off + nch * dk * 4);
    w.seg_e = w.seg_m = w.seg_s = off;
    w.total = off;
    return w;
}

// Segments for the hot chain.  The plain chain runs one workgroup per (sequence,
// head, 32 value columns); when those number fewer than the 256 CUs and the
// sequence is long, its chunks are cut into segments.  Segment 0 starts from the
// call's initial state, so its outputs run in the first launch beside the maps of
// segments 1 .. nseg - 2; the outputs of segments 1 .. nseg - 1 follow the scan.
// Each launch takes (nseg - 1) workgroups per pair, about SEG_TARGET_WG in all.
// A chunk of outputs costs about 10/7 of a chunk of maps there, so segment 0 is
// 7/10 as long as the others and the first launch's two kinds of work end together.
SegPlan seg_plan(int B, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints) {
    const int NC = (T + C - 1) / C;
    SegPlan p{NC, 1, NC};
    if (!hot_config(in_bf16, dk, C) || checkpoints) return p;
    const long bh = (long)B * H;
    if (bh == 0 || bh * (dv / 32) >= 256) return p;
    long n1 = SEG_TARGET_WG / bh;                            // segments after the first
    if (n1 > NC / SEG_MIN_CHUNKS - 1) n1 = NC / SEG_MIN_CHUNKS - 1;
    if (n1 < SEG_MIN_LATER) return p;
    const long L = (10L * NC + 10 * n1 + 6) / (10 * n1 + 7);  // ceil(NC / (n1 + 0.7))
    long L0 = 7 * L / 10 > 0 ? 7 * L / 10 : 1;
    const long last = NC - L0 - (n1 - 1) * L;                // the last segment's chunks
    if (last > L) L0 += last - L;
    const long nseg = 1 + (NC - L0 + L - 1) / L;
    if (nseg < 1 + SEG_MIN_LATER) return p;
    return SegPlan{(int)L, (int)nseg, (int)L0};
}

SegPlan seg_plan_of(const ChunkArgs& a) {
    if (a.cu_seqlens) return SegPlan{0, 1, 0};
    return seg_plan(a.B, a.T, a.H, a.dk, a.dv, a.in_bf16, a.C, a.checkpoints);
}

WsLayout ws_layout(int B, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints) {
    const size_t NC = (size_t)((T + C - 1) / C);
    WsLayout w = layout_units((size_t)B * H * NC, 0, dk, dv, in_bf16, C);
    const SegPlan sp = seg_plan(B, T, H, dk, dv, in_bf16, C, checkpoints);
    if (sp.nseg > 1) {
        const size_t items = (size_t)B * H * sp.nseg;
        w.seg_e = w.total;
        w.seg_m = al256(w.seg_e + items * dk * dv * 4);
        w.seg_s = al256(w.seg_m + items * dk * dk * 4);
        w.total = al256(w.seg_s + items * dk * dv * 4);
    }
    return w;
}

WsLayout ws_layout_packed(int N, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints) {
    const size_t chunks = (size_t)((T + C - 1) / C) + (size_t)N;
    (void)checkpoints;                                       // packed batches never run in segments
    return layout_units(chunks * H, 2 * ((size_t)N + 1) * 4, dk, dv, in_bf16, C);   // cu_chunks, cu_tok
}

WsLayout ws_layout_of(const ChunkArgs& a) {
    return a.cu_seqlens ? ws_layout_packed(a.N, a.T, a.H, a.dk, a.dv, a.in_bf16, a.C, a.checkpoints)
                        : ws_layout(a.B, a.T, a.H, a.dk, a.dv, a.in_bf16, a.C, a.checkpoints);
}

UnitMap unit_map(const ChunkArgs& a) {
    UnitMap m;
    m.T_len = a.T; m.H = a.H; m.C = a.C;
    m.NC = (a.T + a.C - 1) / a.C;
    m.BH = (long)a.B * a.H;
    m.cu_seqlens = a.cu_seqlens;
    m.cu_chunks = a.cu_seqlens ? reinterpret_cast<const int*>((const char*)a.ws + ws_layout_of(a).cu) : nullptr;
    m.cu_tok = m.cu_chunks ? m.cu_chunks + (a.N + 1) : nullptr;
    m.nseq = a.N;
    return m;
}

long unit_count(const ChunkArgs& a) {
    if (a.cu_seqlens) return ((long)(a.T + a.C - 1) / a.C + a.N) * a.H;
    return (long)a.B * a.H * ((a.T + a.C - 1) / a.C);
}

long seq_head_count(const ChunkArgs& a) { return (long)(a.cu_seqlens ? a.N : a.B) * a.H; }

// Offsets of a packed batch.  cu_tok[i] = min(T, max(0, cu_seqlens[0..i])) for
// i = 0..N: a running maximum, so sequence s = [cu_tok[s], cu_tok[s+1]) never
// overlaps another and the lengths sum to at most T.  cu_chunks[0] = 0 and
// cu_chunks[s+1] = cu_chunks[s] + ceil(length of s / C).  One workgroup of 1024
// threads walks the N+1 offsets in blocks of 1024, carrying the running maximum
// and the chunk sum from block to block.
__global__ __launch_bounds__(1024) void packed_chunks_kernel(const int* __restrict__ cu_seqlens, int nseq,
                                                             int T_len, int C, int* __restrict__ cu_chunks,
                                                             int* __restrict__ cu_tok) {
    __shared__ int sm[1024];
    __shared__ int sc[1024];
    __shared__ int carry_max, carry_sum;
    const int tid = threadIdx.x;
    if (tid == 0) { carry_max = 0; carry_sum = 0; }
    __syncthreads();
    for (int base = 0; base <= nseq; base += 1024) {
        const int i = base + tid;
        const bool in = i <= nseq;
        const int prev_last = carry_max;                      // clamped offset of index base - 1 (0 at start)
        sm[tid] = in ? (int)clamp_tok(cu_seqlens[i], 0, T_len) : 0;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {            // inclusive running maximum
            const int x = tid >= off ? sm[tid - off] : 0;
            __syncthreads();
            sm[tid] = sm[tid] > x ? sm[tid] : x;
            __syncthreads();
        }
        const int m = sm[tid] > prev_last ? sm[tid] : prev_last;
        const int mp = tid > 0 ? (sm[tid - 1] > prev_last ? sm[tid - 1] : prev_last) : prev_last;
        // chunks of sequence i - 1 (index 0 ends no sequence)
        sc[tid] = (in && i >= 1) ? (m - mp + C - 1) / C : 0;
        if (in) cu_tok[i] = m;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {            // inclusive sum
            const int x = tid >= off ? sc[tid - off] : 0;
            __syncthreads();
            sc[tid] += x;
            __syncthreads();
        }
        if (in) cu_chunks[i] = carry_sum + sc[tid];
        __syncthreads();
        if (tid == 0) {
            carry_sum += sc[1023];
            carry_max = sm[1023] > prev_last ? sm[1023] : prev_last;
        }
        __syncthreads();
    }
}

template <typename T, int DK, int DV, int C>
static hipError_t launch_intra(const ChunkArgs& a) {
    typedef IntraCfg<T, DK, DV, C> Cfg;
    if constexpr (!Cfg::FITS) {
        return hipErrorInvalidValue;
    } else {
        const long nch = unit_count(a);
        if (nch == 0) return hipSuccess;
        const WsLayout w = ws_layout_of(a);
        char* ws = (char*)a.ws;
        hipLaunchKernelGGL((chunk_intra_kernel<T, DK, DV, C>), dim3((unsigned)nch), dim3(256), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta,
                           (T*)(ws + w.qt), (T*)(ws + w.wk), (T*)(ws + w.kb), (T*)(ws + w.p),
                           (float*)(ws + w.u), (float*)(ws + w.gam), unit_map(a), a.gate | a.pre, a.ck_t, a.ck_a);
        return hipGetLastError();
    }
}

template <typename T, int DK, int DV, int C>
static constexpr bool combo_fits() {
    return IntraCfg<T, DK, DV, C>::FITS && chain_fits<T, float, DK, DV, C, 16>();
}

bool chunk_supported(int dk, int dv, int C, bool in_bf16) {
#define KDA_FIT(T, DK, DV, CC) if (dk == DK && dv == DV && C == CC) return combo_fits<T, DK, DV, CC>();
#define KDA_FIT_C(T, DK, DV) KDA_FIT(T, DK, DV, 16) KDA_FIT(T, DK, DV, 32) KDA_FIT(T, DK, DV, 64) KDA_FIT(T, DK, DV, 128)
    if (in_bf16) {
        KDA_FIT_C(bf16, 64, 64) KDA_FIT_C(bf16, 64, 128) KDA_FIT_C(bf16, 128, 64) KDA_FIT_C(bf16, 128, 128)
    } else {
        KDA_FIT_C(float, 64, 64) KDA_FIT_C(float, 64, 128) KDA_FIT_C(float, 128, 64) KDA_FIT_C(float, 128, 128)
    }
#undef KDA_FIT_C
#undef KDA_FIT
    return false;
}

template <int DV, bool GEN>
static hipError_t launch_intra64(const ChunkArgs& a) {
    constexpr int DK = 128;
    const long nch = unit_count(a);
    if (nch == 0) return hipSuccess;
    if (GEN && (!a.ck_t || !a.ck_a)) return hipErrorInvalidValue;
    const WsLayout w = ws_layout_of(a);
    char* ws = (char*)a.ws;
    // the in-kernel q, k normalisation as a template constant: the plain call
    // carries no multiplies by 1 and no row sums
    auto kernel = (a.gate | a.pre) & MODE_QK_L2NORM ? chunk_intra64_kernel<DV, GEN, true>
                                                     : chunk_intra64_kernel<DV, GEN, false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)nch), dim3(512), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta,
                       (bf16*)(ws + w.qt), (bf16*)(ws + w.wk), (bf16*)(ws + w.kb), (bf16*)(ws + w.p),
                       (void*)(ws + w.u), (float*)(ws + w.gam), unit_map(a), a.gate | a.pre, a.ck_t, a.ck_a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t intra_c(const ChunkArgs& a) {
    if constexpr (sizeof(T) == 2 && DK == 128) {
        if (hot_layout(a)) return launch_intra64<DV, false>(a);
        // the backward pass's forward stage in this configuration: the same kernel,
        // also storing the checkpoints T and A
        if (hot_config(a.in_bf16, DK, a.C) && a.checkpoints) return launch_intra64<DV, true>(a);
    }
    switch (a.C) {
        case 16: return launch_intra<T, DK, DV, 16>(a);
        case 32: return launch_intra<T, DK, DV, 32>(a);
        case 64: return launch_intra<T, DK, DV, 64>(a);
        default: return launch_intra<T, DK, DV, 128>(a);
    }
}
template <typename T>
static hipError_t intra_dims(const ChunkArgs& a) {
    if (a.dk == 64) return a.dv == 64 ? intra_c<T, 64, 64>(a) : intra_c<T, 64, 128>(a);
    return a.dv == 64 ? intra_c<T, 128, 64>(a) : intra_c<T, 128, 128>(a);
}
hipError_t run_chunk_intra(const ChunkArgs& a) {
    if (a.cu_seqlens && a.N > 0) {
        int* cu_chunks = reinterpret_cast<int*>((char*)a.ws + ws_layout_of(a).cu);
        hipLaunchKernelGGL(packed_chunks_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, a.N, a.T,
                           a.C, cu_chunks, cu_chunks + (a.N + 1));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return a.in_bf16 ? intra_dims<bf16>(a) : intra_dims<float>(a);
}

hipError_t run_chunk_chain(const ChunkArgs& a) {
    if (hot_config(a.in_bf16, a.dk, a.C)) return run_chunk_chain64(a);   // with checkpoints in the backward pass
    return a.in_bf16 ? run_chunk_chain_bf16(a) : run_chunk_chain_f32(a);
}

}  // namespace kda
