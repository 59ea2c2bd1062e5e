// kda_chunk_chain.h -- stage 2 of the chunkwise forward: the sequential state
// recurrence across chunks and the outputs.  Included once per input dtype.
#pragma once

#include "kda_chunk.h"

namespace kda {

template <typename T, typename TOut, int DK, int DV, int C, int DVS>
__global__ __launch_bounds__(256) void chunk_chain_kernel(
    const T* __restrict__ ws_qt, const T* __restrict__ ws_wk, const T* __restrict__ ws_kb,
    const T* __restrict__ ws_p, const float* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, float* __restrict__ sT, UnitMap um,
    float* __restrict__ ck_state, float* __restrict__ ck_w) {
    // ck_state / ck_w (NULL in the forward pass): per unit, the fp32 state at the
    // chunk's start [dk][dv] and the chunk's W = U - Wk S [C][dv], kept for the
    // backward pass.  o may be NULL (outputs not stored).
    typedef ChainCfg<T, TOut, DK, DV, C, DVS> Cfg;
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, CK = Cfg::CK, NJ = Cfg::NJ, E16 = Cfg::E16;
    constexpr int NTW = Cfg::NTW, NTS = Cfg::NTS, KSTEP = Mma<T>::KSTEP;
    constexpr int NSL = DV / DVS;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* sQt = reinterpret_cast<T*>(smem);
    T* sWk = reinterpret_cast<T*>(smem + Cfg::OFF_WK);
    T* sKbT = reinterpret_cast<T*>(smem + Cfg::OFF_KBT);
    T* sP = reinterpret_cast<T*>(smem + Cfg::OFF_P);
    float* sU = reinterpret_cast<float*>(smem + Cfg::OFF_U);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::OFF_GAM);
    T* sST = reinterpret_cast<T*>(smem + Cfg::OFF_ST);
    T* sWT = reinterpret_cast<T*>(smem + Cfg::OFF_WT);
    TOut* sO = reinterpret_cast<TOut*>(smem + Cfg::OFF_O);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Slices of one head share an XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so the per-chunk operands they all read come from one L2.
    long bh;
    int sl;
    {
        const long nwg = (long)gridDim.x, id = blockIdx.x;
        if (!um.cu_seqlens && nwg % (8 * NSL) == 0) {
            const long xcd = id % 8, local = id / 8;
            sl = (int)(local % NSL);
            bh = (local / NSL) * 8 + xcd;
        } else {
            bh = id / NSL;
            sl = (int)(id % NSL);
        }
    }
    const int j0 = sl * DVS;
    // sequence (batch row, or packed sequence) and head; its chunks and tokens
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int NC = sr.nchunks;
    auto unit_of = [&](int n) -> long { return unit_id(um, sq, h, n, sr.chunk0); };

    // ---- register prefetch of one chunk's operands (16-byte units), one
    // statically sized register array per operand
    constexpr int PQ = (Cfg::U_QT + 255) / 256, PK = (Cfg::U_KB + 255) / 256, PP = (Cfg::U_P + 255) / 256,
                  PU = (Cfg::U_U + 255) / 256;
    constexpr int D = Cfg::DEPTH;
    u32x4 preQ[D][PQ], preW[D][PQ], preK[D][PK], preP[D][PP], preU[D][PU], preG[D];
#define KDA_CHAIN_PREFETCH(SL, CH)                                                                     \
    {                                                                                              \
        const long ch_ = (CH);                                                                     \
        const u32x4* gq_ = reinterpret_cast<const u32x4*>(ws_qt + ch_ * (long)C * DK);             \
        const u32x4* gw_ = reinterpret_cast<const u32x4*>(ws_wk + ch_ * (long)C * DK);             \
        const u32x4* gk_ = reinterpret_cast<const u32x4*>(ws_kb + ch_ * (long)DK * C);             \
        const u32x4* gp_ = reinterpret_cast<const u32x4*>(ws_p + ch_ * (long)C * C);               \
        const float* gu_ = ws_u + ch_ * (long)C * DV + j0;                                         \
        _Pragma("unroll") for (int i = 0; i < PQ; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_QT) { preQ[SL][i] = gq_[u]; preW[SL][i] = gw_[u]; }                             \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PK; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_KB) preK[SL][i] = gk_[u];                                                   \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PP; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_P) preP[SL][i] = gp_[u];                                                    \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PU; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_U)                                                                      \
                preU[SL][i] = *reinterpret_cast<const u32x4*>(gu_ + (long)(u / (DVS / 4)) * DV + 4 * (u % (DVS / 4))); \
        }                                                                                          \
        if (tid < Cfg::U_G) preG[SL] = reinterpret_cast<const u32x4*>(ws_gam + ch_ * (long)DK)[tid];  \
    }
#define KDA_CHAIN_COMMIT(SL)                                                                         \
    {                                                                                              \
        _Pragma("unroll") for (int i = 0; i < PQ; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_QT) {                                                                   \
                const int e = u * E16;                                                             \
                *reinterpret_cast<u32x4*>(sQt + (e / DK) * LDK + e % DK) = preQ[SL][i];                \
                *reinterpret_cast<u32x4*>(sWk + (e / DK) * LDK + e % DK) = preW[SL][i];                \
            }                                                                                      \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PK; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_KB) {                                                                   \
                const int e = u * E16;                                                             \
                *reinterpret_cast<u32x4*>(sKbT + (e / C) * LDC + e % C) = preK[SL][i];             \
            }                                                                                      \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PP; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_P) {                                                                    \
                const int e = u * E16;                                                             \
                *reinterpret_cast<u32x4*>(sP + (e / C) * LDC + e % C) = preP[SL][i];                   \
            }                                                                                      \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < PU; ++i) {                                           \
            const int u = tid + 256 * i;                                                           \
            if (u < Cfg::U_U) reinterpret_cast<u32x4*>(sU)[u] = preU[SL][i];                           \
        }                                                                                          \
        if (tid < Cfg::U_G) reinterpret_cast<u32x4*>(sGam)[tid] = preG[SL];                            \
    }

    // zero the contraction padding once (columns C..CK never receive data)
    if constexpr (CK > C) {
        for (int u = tid; u < (DK + C + DVS) * (CK - C); u += 256) {
            const int row = u / (CK - C), i = C + u % (CK - C);
            if (row < DK) sKbT[row * LDC + i] = from_f32<T>(0.f);
            else if (row < DK + C) sP[(row - DK) * LDC + i] = from_f32<T>(0.f);
            else sWT[(row - DK - C) * LDC + i] = from_f32<T>(0.f);
        }
    }

#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < NC) KDA_CHAIN_PREFETCH(d, unit_of(d));

    typedef typename Mma<T>::frag frag;
    const int fr = lane & 15, fk = (lane >> 4) * Mma<T>::KPL;     // fragment row, k offset
    floatx4 accS[Cfg::SPW][NJ];
    static_for<Cfg::SPW>([&](auto SI) {
        constexpr int si = SI;
        const int ct = wave + 4 * si;
        static_for<NJ>([&](auto JI) {
            constexpr int jt = JI;
            accS[si][jt] = zero4();
            if (s0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = ct * 16 + 4 * (lane >> 4) + e, j = jt * 16 + (lane & 15);
                    accS[si][jt][e] = s0[(bh * DK + c) * (long)DV + j0 + j];
                }
            }
        });
    });
    // S^T as the B operand of the products with S: sST[j][c], 4 consecutive c per lane
    auto write_state_operand = [&]() {
        static_for<Cfg::SPW>([&](auto SI) {
            constexpr int si = SI;
            const int ct = wave + 4 * si;
            static_for<NJ>([&](auto JI) {
                constexpr int jt = JI;
                const int j = jt * 16 + (lane & 15), c = ct * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) sST[j * LDK + c + e] = from_f32<T>(accS[si][jt][e]);
            });
        });
    };
    write_state_operand();

    for (int n0 = 0; n0 < NC; n0 += D) {
      static_for<D>([&](auto DI) {
        constexpr int d = DI;
        const int n = n0 + d;
        if (n >= NC) return;
        if (ck_state) {                                             // the state this chunk starts from
            float* cks = ck_state + unit_of(n) * (long)DK * DV;
            static_for<Cfg::SPW>([&](auto SI) {
                constexpr int si = SI;
                const int ct = wave + 4 * si;
                static_for<NJ>([&](auto JI) {
                    constexpr int jt = JI;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        cks[(ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + (lane & 15)] = accS[si][jt][e];
                });
            });
        }
        KDA_CHAIN_COMMIT(d);                                        // chunk n operands -> LDS
        if (n + D < NC) KDA_CHAIN_PREFETCH(d, unit_of(n + D));   // in flight for D chunks
        __syncthreads();

        // ---- W = U - Wk S (to LDS, transposed) and the state part of O;
        //      the Wk and Qt fragments are shared by all value-column tiles
        floatx4 accO[Cfg::RPW][NJ];
        static_for<Cfg::RPW>([&](auto RI) {
            constexpr int ri = RI;
            const int R = wave + 4 * ri;
            if (R < C / 16) {
                floatx4 wk[NJ];
                static_for<NJ>([&](auto JI) { wk[JI] = zero4(); accO[ri][JI] = zero4(); });
                for (int k0 = 0; k0 < DK; k0 += KSTEP) {
                    const frag fw = *reinterpret_cast<const frag*>(sWk + (R * 16 + fr) * LDK + k0 + fk);
                    const frag fq = *reinterpret_cast<const frag*>(sQt + (R * 16 + fr) * LDK + k0 + fk);
                    static_for<NJ>([&](auto JI) {
                        constexpr int J = JI;
                        const frag fb = *reinterpret_cast<const frag*>(sST + (J * 16 + fr) * LDK + k0 + fk);
                        wk[J] = Mma<T>::mma(fw, fb, wk[J]);
                        accO[ri][J] = Mma<T>::mma(fq, fb, accO[ri][J]);
                    });
                }
                static_for<NJ>([&](auto JI) {
                    constexpr int J = JI;
                    const int j = J * 16 + (lane & 15), r = R * 16 + 4 * (lane >> 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sWT[j * LDC + r + e] = from_f32<T>(sU[(r + e) * DVS + j] - wk[J][e]);
                    if (ck_w) {
                        float* ckw = ck_w + unit_of(n) * (long)C * DV;
#pragma unroll
                        for (int e = 0; e < 4; ++e) ckw[(r + e) * (long)DV + j0 + j] = sU[(r + e) * DVS + j] - wk[J][e];
                    }
                });
            }
        });
        __syncthreads();

        // ---- O += P W ; S = gam * S + Kb^T W
        static_for<Cfg::RPW>([&](auto RI) {
            constexpr int ri = RI;
            const int R = wave + 4 * ri;
            if (R < C / 16) {
                const int K = ((16 * (R + 1) + KSTEP - 1) / KSTEP) * KSTEP;
                for (int k0 = 0; k0 < K; k0 += KSTEP) {
                    const frag fp = *reinterpret_cast<const frag*>(sP + (R * 16 + fr) * LDC + k0 + fk);
                    static_for<NJ>([&](auto JI) {
                        constexpr int J = JI;
                        const frag fb = *reinterpret_cast<const frag*>(sWT + (J * 16 + fr) * LDC + k0 + fk);
                        accO[ri][J] = Mma<T>::mma(fp, fb, accO[ri][J]);
                    });
                }
                static_for<NJ>([&](auto JI) {
                    constexpr int J = JI;
                    const int j = J * 16 + (lane & 15);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = R * 16 + 4 * (lane >> 4) + e;
                        if constexpr (Cfg::STAGE_O) {
                            sO[r * DVS + j] = from_f32<TOut>(accO[ri][J][e]);
                        } else {
                            const int tt = n * C + r;
                            if (o && sr.tok_begin + tt < sr.tok_end)
                                o[((sr.tok_begin + tt) * H + h) * DV + j0 + j] = from_f32<TOut>(accO[ri][J][e]);
                        }
                    }
                });
            }
        });
        static_for<Cfg::SPW>([&](auto SI) {
            constexpr int si = SI;
            const int ct = wave + 4 * si;
            float gm[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) gm[e] = sGam[ct * 16 + 4 * (lane >> 4) + e];
            static_for<NJ>([&](auto JI) {
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[si][JI][e] *= gm[e];
            });
            for (int k0 = 0; k0 < CK; k0 += KSTEP) {
                const frag fa = *reinterpret_cast<const frag*>(sKbT + (ct * 16 + fr) * LDC + k0 + fk);
                static_for<NJ>([&](auto JI) {
                    constexpr int J = JI;
                    const frag fb = *reinterpret_cast<const frag*>(sWT + (J * 16 + fr) * LDC + k0 + fk);
                    accS[si][J] = Mma<T>::mma(fa, fb, accS[si][J]);
                });
            }
        });
        __syncthreads();
        if constexpr (Cfg::STAGE_O) {
            constexpr int EO = 16 / sizeof(TOut);
            constexpr int NUO = C * DVS / EO;
            for (int u = tid; u < NUO; u += 256) {
                const int r = (u * EO) / DVS, jj = (u * EO) % DVS;
                const int tt = n * C + r;
                if (o && sr.tok_begin + tt < sr.tok_end)
                    *reinterpret_cast<uint4*>(o + ((sr.tok_begin + tt) * H + h) * DV + j0 + jj) =
                        *reinterpret_cast<const uint4*>(sO + r * DVS + jj);
            }
        }
        write_state_operand();
      });
    }

    if (sT) {
        static_for<Cfg::SPW>([&](auto SI) {
            constexpr int si = SI;
            const int ct = wave + 4 * si;
            static_for<NJ>([&](auto JI) {
                constexpr int jt = JI;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = ct * 16 + 4 * (lane >> 4) + e, j = jt * 16 + (lane & 15);
                    sT[(bh * DK + c) * (long)DV + j0 + j] = accS[si][jt][e];
                }
            });
        });
    }
}

#undef KDA_CHAIN_PREFETCH
#undef KDA_CHAIN_COMMIT

// ================================================================ launch
template <typename T, typename TOut, int DK, int DV, int C, int DVS>
static hipError_t launch_chain_dvs(const ChunkArgs& a) {
    typedef ChainCfg<T, TOut, DK, DV, C, DVS> Cfg;
    if constexpr (!Cfg::FITS || DVS > DV) {
        return hipErrorInvalidValue;
    } else {
        const long nwg = seq_head_count(a) * (DV / DVS);
        if (nwg == 0) return hipSuccess;
        const WsLayout w = ws_layout_of(a);
        char* ws = (char*)a.ws;
        hipLaunchKernelGGL((chunk_chain_kernel<T, TOut, DK, DV, C, DVS>), dim3((unsigned)nwg), dim3(256), 0,
                           a.stream, (const T*)(ws + w.qt), (const T*)(ws + w.wk), (const T*)(ws + w.kb),
                           (const T*)(ws + w.p), (const float*)(ws + w.u), (const float*)(ws + w.gam),
                           a.s0, (TOut*)a.o, a.sT, unit_map(a), a.ck_state, a.ck_w);
        return hipGetLastError();
    }
}

// Value-column slice width: enough workgroups to cover the chip (>= 256 when
// possible), as wide as possible otherwise, and within the LDS budget.
template <typename T, typename TOut, int DK, int DV, int C>
static int pick_dvs(long bh) {
    int dvs = 16;
    const int cands[3] = {64, 32, 16};
    const bool fits[3] = {chain_fits<T, TOut, DK, DV, C, 64>(), chain_fits<T, TOut, DK, DV, C, 32>(),
                          chain_fits<T, TOut, DK, DV, C, 16>()};
    for (int i = 0; i < 3; ++i) {
        if (!fits[i]) continue;
        dvs = cands[i];
        if (bh * (DV / cands[i]) >= 256) break;
    }
    return dvs;
}

template <typename T, typename TOut, int DK, int DV, int C>
static hipError_t launch_chain(const ChunkArgs& a) {
    const int dvs = pick_dvs<T, TOut, DK, DV, C>(seq_head_count(a));
    if (dvs == 64) return launch_chain_dvs<T, TOut, DK, DV, C, 64>(a);
    if (dvs == 32) return launch_chain_dvs<T, TOut, DK, DV, C, 32>(a);
    return launch_chain_dvs<T, TOut, DK, DV, C, 16>(a);
}

template <typename T, typename TOut, int DK, int DV>
static hipError_t chain_c(const ChunkArgs& a) {
    switch (a.C) {
        case 16: return launch_chain<T, TOut, DK, DV, 16>(a);
        case 32: return launch_chain<T, TOut, DK, DV, 32>(a);
        case 64: return launch_chain<T, TOut, DK, DV, 64>(a);
        default: return launch_chain<T, TOut, DK, DV, 128>(a);
    }
}
template <typename T, typename TOut>
static hipError_t chain_dims(const ChunkArgs& a) {
    if (a.dk == 64) return a.dv == 64 ? chain_c<T, TOut, 64, 64>(a) : chain_c<T, TOut, 64, 128>(a);
    return a.dv == 64 ? chain_c<T, TOut, 128, 64>(a) : chain_c<T, TOut, 128, 128>(a);
}
}  // namespace kda
