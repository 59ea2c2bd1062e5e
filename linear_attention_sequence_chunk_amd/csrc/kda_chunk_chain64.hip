// kda_chunk_chain64.hip -- stage 2 of the chunkwise forward for the hot
// configuration (bf16 inputs, C = 64, dk = 128): the sequential state recurrence
// across chunks and the outputs, reading the workspace that
// chunk_intra64_kernel writes in MFMA fragment order.
//
// Per chunk (the chunkwise form of kda_chunk.h):
//   W = U - Wk S,   O = Qt S + P W,   S <- Diag(gam) S + Kb^T W
// One workgroup of 8 waves per (b, h, slice of DVS value columns).  Every
// per-chunk operand is an MFMA A operand or the initial value of an
// accumulator, and the workspace stores each wave's share as whole 16-byte
// lanes, so the operands go from memory straight into registers (DEPTH chunks in
// flight) and never through LDS.  Only S^T and W^T, the B operands that every
// wave needs, are exchanged through LDS.
//   waves 0-3 ("W waves"): row tile R = wave of W = U - Wk S
//   waves 4-7 ("O waves"): row tile R = wave - 4 of O = Qt S + P W
//   all waves           : state rows 16*wave .. +15:  S <- gam S + Kb^T W
// Two barriers per chunk: S^T ready -> (W, Qt S) -> W^T ready -> (P W, S update).
#include "kda_chunk.h"

namespace kda {

// Workspace of this configuration, per chunk unit (chunk-major, as for every layout):
//   Qt, Wk [4 row tiles][4 k-steps][64 lanes][8 bf16]  lane l: row 16R + l%16, channels 32u + 8(l/16) + 0..7
//   Kb^T   [8 channel tiles][2 k-steps][64][8 bf16]     lane l: channel 16c + l%16, tokens 32u + 8(l/16) + 0..7
//   P      [4 row tiles][2 k-steps][64][8 bf16]         (row tiles 0, 1 at k-step 1 lie above the diagonal:
//                                                        never written, never read)
//   U      [4 row tiles][DV/16 column tiles][64][4] bf16  lane l, element e: row 16R + 4(l/16) + e, column 16J + l%16
//   gam    [DK] fp32
template <typename TOut, int DV, int DVS>
struct Chain64Cfg {
    static constexpr int C = 64, DK = 128, NT = 512, NJ = DVS / 16, NSL = DV / DVS;
    static constexpr int LDK = DK + 8, LDC = C + 8;   // padded bf16 rows of S^T, W^T
    static constexpr int DEPTH = 4;                    // chunks in flight
    static constexpr size_t OFF_ST = 0;
    static constexpr size_t OFF_WT = OFF_ST + size_t(DVS) * LDK * 2;
    static constexpr size_t OFF_O = OFF_WT + size_t(DVS) * LDC * 2;               // per O wave: [16][DVS]
    static constexpr size_t TOTAL = OFF_O + size_t(4) * 16 * DVS * sizeof(TOut);
    static_assert(NJ >= 1 && NJ <= 2 && DV % DVS == 0, "slice width 16 or 32");
    static_assert((16 * DVS * sizeof(TOut)) % 16 == 0, "output staging rows");
};

template <typename TOut, int DV, int DVS>
__global__ __launch_bounds__(512) void chunk_chain64_kernel(
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const bf16* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, float* __restrict__ sT, UnitMap um) {
    typedef Chain64Cfg<TOut, DV, DVS> Cfg;
    constexpr int C = Cfg::C, DK = Cfg::DK, NJ = Cfg::NJ, NSL = Cfg::NSL, LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr int D = Cfg::DEPTH;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    bf16* sST = reinterpret_cast<bf16*>(smem + Cfg::OFF_ST);
    bf16* sWT = reinterpret_cast<bf16*>(smem + Cfg::OFF_WT);

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

    const bool wW = wave < 4;                    // uniform per wave
    const int R = wave & 3, ct = wave;
    const int fr = lane & 15, fk = 8 * (lane >> 4);
    TOut* sO = reinterpret_cast<TOut*>(smem + Cfg::OFF_O) + R * 16 * DVS;

    // ---- operand registers, D chunks in flight
    // Every wave issues the same load instructions in every chunk (past the last
    // chunk the last one is loaded again), so that the number of loads in flight is
    // the same on every path and each chunk waits only for its own operands, D - 1
    // chunks of loads staying in flight.  The loads a role does not need (U for the
    // O waves, P for the W waves) repeat an address the wave has just requested, so
    // they cost no L1 miss.
    u32x4 fA[D][4];      // Wk (W waves) or Qt (O waves), row tile R, 4 k-steps
    u32x2 fU[D][NJ];     // U tiles of this slice (W waves; a repeat of fA on O waves)
    u32x4 fX[D][2];      // P k-steps (O waves, k-step 1 of row tiles 0, 1 not used; a repeat of fK on W waves)
    u32x4 fK[D][2];      // Kb^T channel tile ct, 2 k-steps
    u32x4 fG[D];         // gam of this lane's 4 state rows
    // first half: what phase 1 consumes; second half: what phase 2 consumes
#define KDA_C64_PREFETCH_1(SL, CH)                                                                  \
    {                                                                                               \
        const long ch_ = (CH);                                                                      \
        const u32x4* a_ = reinterpret_cast<const u32x4*>((wW ? ws_wk : ws_qt) + ch_ * (long)(C * DK)) \
                          + R * 4 * 64 + lane;                                                      \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) fA[SL][u] = a_[u * 64];                       \
        const u32x2* u_ = wW ? reinterpret_cast<const u32x2*>(ws_u + ch_ * (long)(C * DV))          \
                                   + (R * (DV / 16) + sl * NJ) * 64 + lane                          \
                             : reinterpret_cast<const u32x2*>(a_);                                  \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j) fU[SL][j] = u_[wW ? j * 64 : 0];             \
    }
#define KDA_C64_PREFETCH_2(SL, CH)                                                                  \
    {                                                                                               \
        const long ch_ = (CH);                                                                      \
        const u32x4* k_ = reinterpret_cast<const u32x4*>(ws_kb + ch_ * (long)(DK * C)) + ct * 2 * 64 + lane; \
        {                                                                                           \
            const u32x4* p_ = wW ? k_ : reinterpret_cast<const u32x4*>(ws_p + ch_ * (long)(C * C)) + R * 2 * 64 + lane; \
            fX[SL][0] = p_[0];                                                                      \
            fX[SL][1] = p_[wave >= 6 ? 64 : 0];     /* O waves of row tiles 2, 3 only */          \
        }                                                                                           \
        fK[SL][0] = k_[0];                                                                          \
        fK[SL][1] = k_[64];                                                                         \
        fG[SL] = *reinterpret_cast<const u32x4*>(ws_gam + ch_ * (long)DK + ct * 16 + 4 * (lane >> 4)); \
    }

    if (NC > 0) {                                                   // an empty sequence loads nothing
#pragma unroll
        for (int d = 0; d < D; ++d) {
            KDA_C64_PREFETCH_1(d, unit_of(d < NC ? d : NC - 1));
            KDA_C64_PREFETCH_2(d, unit_of(d < NC ? d : NC - 1));
        }
    }

    // ---- state rows 16*ct + 4(l/16) + e, columns j0 + 16 jt + l%16, fp32 in accumulators
    floatx4 accS[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        accS[jt] = zero4();
        if (s0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                accS[jt][e] = s0[(bh * DK + ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + fr];
        }
    }
    // S^T as the B operand of Qt S and Wk S: sST[j][c], 4 consecutive c per lane
    auto write_state_operand = [&]() {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (bf16)accS[jt][e];
            *reinterpret_cast<bf16x4*>(sST + (jt * 16 + fr) * LDK + ct * 16 + 4 * (lane >> 4)) = v4;
        }
    };
    write_state_operand();

    // one chunk n whose operands sit in register slot d
    auto step = [&](auto DI, int n) {
        constexpr int d = DI;
        __syncthreads();                                            // S^T of chunk n's start state

        // ---- phase 1: W waves W = U - Wk S (to LDS as W^T); O waves O = Qt S
        floatx4 acc[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] = zero4();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bf16x8 fa = __builtin_bit_cast(bf16x8, fA[d][u]);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sST + (jt * 16 + fr) * LDK + u * 32 + fk);
                acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[jt], 0, 0, 0);
            }
        }
        if (wW) {
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                const bf16x4 uu = __builtin_bit_cast(bf16x4, fU[d][jt]);
                bf16x4 w4;
#pragma unroll
                for (int e = 0; e < 4; ++e) w4[e] = (bf16)((float)uu[e] - acc[jt][e]);
                *reinterpret_cast<bf16x4*>(sWT + (jt * 16 + fr) * LDC + R * 16 + 4 * (lane >> 4)) = w4;
            }
        }
        KDA_C64_PREFETCH_1(d, unit_of(n + D < NC ? n + D : NC - 1));
        __syncthreads();                                            // W^T complete

        // ---- phase 2: O waves O += P W (stored); all waves S = gam S + Kb^T W
        if (!wW) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u == 1 && R < 2) break;                         // P is lower triangular
                const bf16x8 fp = __builtin_bit_cast(bf16x8, fX[d][u]);
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) {
                    const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sWT + (jt * 16 + fr) * LDC + u * 32 + fk);
                    acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp, fb, acc[jt], 0, 0, 0);
                }
            }
            // this wave's 16 x DVS output tile, through its own LDS rows, as 16-byte row pieces
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) sO[(4 * (lane >> 4) + e) * DVS + jt * 16 + fr] = from_f32<TOut>(acc[jt][e]);
            constexpr int EO = 16 / sizeof(TOut), PPR = DVS / EO, NUO = 16 * PPR;   // pieces per row, per tile
#pragma unroll
            for (int u = lane; u < NUO; u += 64) {
                const int r = u / PPR, jj = (u % PPR) * EO;
                const int tt = n * C + R * 16 + r;
                if (sr.tok_begin + tt < sr.tok_end)
                    *reinterpret_cast<u32x4*>(o + ((sr.tok_begin + tt) * H + h) * DV + j0 + jj) =
                        *reinterpret_cast<const u32x4*>(sO + r * DVS + jj);
            }
        }
        {
            const floatx4 gm = __builtin_bit_cast(floatx4, fG[d]);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[jt][e] *= gm[e];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 fa = __builtin_bit_cast(bf16x8, fK[d][u]);
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) {
                    const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sWT + (jt * 16 + fr) * LDC + u * 32 + fk);
                    accS[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, accS[jt], 0, 0, 0);
                }
            }
        }
        write_state_operand();                                      // read only after the next barrier
        KDA_C64_PREFETCH_2(d, unit_of(n + D < NC ? n + D : NC - 1));
    };
    // whole rounds of D chunks with no condition inside (the loads in flight are
    // then the same on every path), then the last NC % D chunks
    int n0 = 0;
    for (; n0 + D <= NC; n0 += D) static_for<D>([&](auto DI) { step(DI, n0 + DI); });
    static_for<D>([&](auto DI) {
        if (n0 + DI < NC) step(DI, n0 + DI);
    });

    if (sT) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sT[(bh * DK + ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + fr] = accS[jt][e];
    }
}

#undef KDA_C64_PREFETCH_1
#undef KDA_C64_PREFETCH_2

template <typename TOut, int DV, int DVS>
static hipError_t launch_chain64_dvs(const ChunkArgs& a) {
    constexpr int C = 64, DK = 128;
    const long nwg = seq_head_count(a) * (DV / DVS);
    if (nwg == 0) return hipSuccess;
    const WsLayout w = ws_layout_of(a);
    char* ws = (char*)a.ws;
    hipLaunchKernelGGL((chunk_chain64_kernel<TOut, DV, DVS>), dim3((unsigned)nwg), dim3(512), 0, a.stream,
                       (const bf16*)(ws + w.qt), (const bf16*)(ws + w.wk), (const bf16*)(ws + w.kb),
                       (const bf16*)(ws + w.p), (const bf16*)(ws + w.u), (const float*)(ws + w.gam),
                       a.s0, (TOut*)a.o, a.sT, unit_map(a));
    return hipGetLastError();
}

// Slice width: 32 value columns when that gives at least 256 workgroups, else 16.
template <typename TOut, int DV>
static hipError_t launch_chain64(const ChunkArgs& a) {
    const long bh = seq_head_count(a);
    if (bh * (DV / 32) >= 256) return launch_chain64_dvs<TOut, DV, 32>(a);
    return launch_chain64_dvs<TOut, DV, 16>(a);
}

hipError_t run_chunk_chain64(const ChunkArgs& a) {
    if (a.dv == 64) return a.out_bf16 ? launch_chain64<bf16, 64>(a) : launch_chain64<float, 64>(a);
    return a.out_bf16 ? launch_chain64<bf16, 128>(a) : launch_chain64<float, 128>(a);
}

}  // namespace kda
