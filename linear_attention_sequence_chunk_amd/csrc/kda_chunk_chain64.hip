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
//
// Long sequences with few (sequence, head) pairs are cut into segments of L
// chunks that run side by side (segment-affine form).  A segment maps its start
// state to its end state affinely, S -> M S + E, with M = prod over its chunks of
// (Diag(gam) - Kb^T Wk) and E its end state from a zero start.  Three launches:
//   maps  (CHAIN_MAPS): each segment but the last runs the chain, without
//         outputs, on the augmented state [S | I]: value columns from a zero
//         start (segment 0 from the call's initial state) give E, the dk extra
//         columns from the identity with U taken as 0 give M;
//   scan  (chain_seg_scan_kernel): start states Sst_0 = S0, Sst_1 = E_0,
//         Sst_{s+1} = M_s Sst_s + E_s, in fp32;
//   outputs (CHAIN_SEG): every segment runs the chain with outputs from its
//         start state; the last writes the final state.
// This is the chunk recurrence regrouped (the state after a chunk is an affine
// function of the state before it), so the result equals the sequential chain
// up to rounding; the extra cost is the maps launch.
#include "kda_chunk.h"

namespace kda {

// Workspace of this configuration, per chunk unit (chunk-major, as for every layout):
//   Qt, Wk [4 row tiles][4 k-steps][64 lanes][8 bf16]  lane l: row 16R + l%16, channels 32u + 8(l/16) + 0..7
//   Kb^T   [8 channel tiles][2 k-steps][64][8 bf16]     lane l: channel 16c + l%16, tokens 32u + 8(l/16) + 0..7
//   P      [4 row tiles][2 k-steps][64][8 bf16]         (row tiles 0, 1 at k-step 1 lie above the diagonal:
//                                                        never written, never read)
//   U      [4 row tiles][DV/16 column tiles][64][4] bf16  lane l, element e: row 16R + 4(l/16) + e, column 16J + l%16
//   gam    [DK] fp32
enum ChainMode { CHAIN_PLAIN = 0, CHAIN_MAPS = 1, CHAIN_SEG = 2 };

template <typename TOut, int DV, int DVS>
struct Chain64Cfg {
    static constexpr int C = 64, DK = 128, NT = 512, NJ = DVS / 16, NSL = DV / DVS;
    // padded bf16 rows of S^T and W^T: 24 and 16 elements, measured against 8 and 8
    // (bank conflicts: the 1M workload's chain 8.4 -> 7.9 ms; 32-element pads are worst)
    static constexpr int LDK = DK + 24, LDC = C + 16;
    // chunks in flight: four for slices of 16 or 32 columns; fewer for wider
    // slices, whose accumulators take the registers
    static constexpr int DEPTH = NJ <= 2 ? 4 : (NJ <= 4 ? 3 : 2);
    static constexpr size_t OFF_ST = 0;
    static constexpr size_t OFF_WT = OFF_ST + size_t(DVS) * LDK * 2;
    static constexpr size_t OFF_O = OFF_WT + size_t(DVS) * LDC * 2;               // per O wave: [16][DVS]
    static constexpr size_t TOTAL = OFF_O + size_t(4) * 16 * DVS * sizeof(TOut);
    // slices of 16 .. 128 value columns; the maps launch may also take all DV + DK
    // augmented columns in one workgroup (DVS = 256 with DV = DK = 128)
    static_assert(((NJ == 1 || NJ == 2 || NJ == 4 || NJ == 8) && DV % DVS == 0) || (DV == 128 && DVS == 256),
                  "slice width 16 .. 128, or the whole augmented state");
    static_assert((16 * DVS * sizeof(TOut)) % 16 == 0, "output staging rows");
};

// Segments of a long sequence (CHAIN_MAPS, CHAIN_SEG); per (sequence, head) pair
// bh and segment s, the arrays hold [bh][s][DK][...] fp32.
struct Seg64 {
    int L;                  // chunks per segment
    int nseg;               // segments per (sequence, head)
    float* E;               // end state from a zero start (segment 0: from S0), [.][.][DK][DV]
    float* M;               // linear part of the segment's map, [.][.][DK][DK]
    float* Sst;             // start state of each segment, [.][.][DK][DV]
};

// The maps launch keeps one chunk in flight; with slices of at most 128 columns
// two of its workgroups share a CU.  The other modes keep DEPTH chunks in flight.
template <typename TOut, int DV, int DVS, int MODE>
__global__ __launch_bounds__(512, MODE == CHAIN_MAPS && DVS <= 128 ? 2 : 1) void chunk_chain64_kernel(
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const bf16* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, float* __restrict__ sT, UnitMap um, Seg64 sg) {
    typedef Chain64Cfg<TOut, DV, DVS> Cfg;
    constexpr int C = Cfg::C, DK = Cfg::DK, NJ = Cfg::NJ, NSL = Cfg::NSL, LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr bool MAPS = MODE == CHAIN_MAPS, OUT = MODE != CHAIN_MAPS;
    constexpr int D = MAPS && NJ >= 4 ? 1 : Cfg::DEPTH;
    // slices per work item: the maps launch also runs the DK identity columns
    constexpr int NSLW = MAPS ? (DV + DK) / DVS : NSL;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    bf16* sST = reinterpret_cast<bf16*>(smem + Cfg::OFF_ST);
    bf16* sWT = reinterpret_cast<bf16*>(smem + Cfg::OFF_WT);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Slices of one work item (a (sequence, head) pair, or one of its segments)
    // share an XCD (workgroups are dealt to the 8 XCDs round-robin), so the
    // per-chunk operands they all read come from one L2.
    long item;
    int sl;
    {
        const long nwg = (long)gridDim.x, id = blockIdx.x;
        if (!um.cu_seqlens && nwg % (8 * NSLW) == 0) {
            const long xcd = id % 8, local = id / 8;
            sl = (int)(local % NSLW);
            item = (local / NSLW) * 8 + xcd;
        } else {
            item = id / NSLW;
            sl = (int)(id % NSLW);
        }
    }
    // work item -> (sequence, head) pair and segment
    const int nsegw = MODE == CHAIN_PLAIN ? 1 : (MAPS ? sg.nseg - 1 : sg.nseg);
    const long bh = item / nsegw;
    const int seg = (int)(item % nsegw);
    // first column of the slice; in the maps launch, of the augmented state
    // [value columns 0 .. DV-1 | identity columns DV .. DV+DK-1]
    const int j0 = sl * DVS;
    if (MAPS && j0 >= DV && seg == 0) return;            // segment 0 starts from a known state: no M
    // sequence (batch row, or packed sequence) and head; its chunks and tokens
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int c0 = MODE == CHAIN_PLAIN ? 0 : seg * sg.L;                      // first chunk of the segment
    const int NC = MODE == CHAIN_PLAIN ? sr.nchunks
                                       : (sr.nchunks - c0 < sg.L ? sr.nchunks - c0 : sg.L);
    auto unit_of = [&](int n) -> long { return unit_id(um, sq, h, c0 + n, sr.chunk0); };

    const bool wW = wave < 4;                    // uniform per wave
    const int R = wave & 3, ct = wave;
    // W = U - Wk S: the W waves, all column tiles; in the maps launch, where the O
    // waves have no outputs to form, every wave, half the column tiles each
    constexpr int NJW = MAPS && NJ >= 2 ? NJ / 2 : NJ;
    const bool isW = MAPS || wW;
    const int jw0 = MAPS && NJ >= 2 ? (wave >> 2) * NJW : 0;
    // this wave's W columns are identity columns (maps launch): U is 0 there
    const bool identW = MAPS && j0 + 16 * jw0 >= DV;
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
    u32x2 fU[D][NJW];    // U tiles of this wave's W columns (a repeat of fA where U is not needed)
    u32x4 fX[D][2];      // P k-steps (O waves, k-step 1 of row tiles 0, 1 not used; a repeat of fK on W waves)
    u32x4 fK[D][2];      // Kb^T channel tile ct, 2 k-steps
    u32x4 fG[D];         // gam of this lane's 4 state rows
    // first half: what phase 1 consumes; second half: what phase 2 consumes
    // In the maps launch the O waves compute nothing: their operand loads repeat
    // the W waves' (Wk of the same row tile, Kb^T), and identity slices, whose U
    // is 0, repeat the Wk address for their U loads.
#define KDA_C64_PREFETCH_1(SL, CH)                                                                  \
    {                                                                                               \
        const long ch_ = (CH);                                                                      \
        const u32x4* a_ = reinterpret_cast<const u32x4*>((wW || MAPS ? ws_wk : ws_qt) + ch_ * (long)(C * DK)) \
                          + R * 4 * 64 + lane;                                                      \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) fA[SL][u] = a_[u * 64];                       \
        const bool uu_ = isW && !identW;                                                            \
        const u32x2* u_ = uu_ ? reinterpret_cast<const u32x2*>(ws_u + ch_ * (long)(C * DV))         \
                                    + (R * (DV / 16) + (j0 / 16) + jw0) * 64 + lane                 \
                              : reinterpret_cast<const u32x2*>(a_);                                 \
        _Pragma("unroll") for (int j = 0; j < NJW; ++j) fU[SL][j] = u_[uu_ ? j * 64 : 0];           \
    }
#define KDA_C64_PREFETCH_2(SL, CH)                                                                  \
    {                                                                                               \
        const long ch_ = (CH);                                                                      \
        const u32x4* k_ = reinterpret_cast<const u32x4*>(ws_kb + ch_ * (long)(DK * C)) + ct * 2 * 64 + lane; \
        {                                                                                           \
            const u32x4* p_ = wW || MAPS ? k_ : reinterpret_cast<const u32x4*>(ws_p + ch_ * (long)(C * C)) + R * 2 * 64 + lane; \
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
    // start: the call's initial state (plain; segment 0 of the maps launch), the
    // segment's start state (outputs launch), zero (other segments' E), the
    // identity (M)
    const float* init = MODE == CHAIN_SEG ? sg.Sst + (bh * sg.nseg + seg) * (long)(DK * DV)
                                          : (MODE == CHAIN_PLAIN || seg == 0 ? (s0 ? s0 + bh * (long)(DK * DV) : nullptr)
                                                                             : nullptr);
    floatx4 accS[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        accS[jt] = zero4();
        if (MAPS && j0 + jt * 16 >= DV) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                accS[jt][e] = (ct * 16 + 4 * (lane >> 4) + e == j0 + jt * 16 - DV + fr) ? 1.f : 0.f;
        } else if (init) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                accS[jt][e] = init[(ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + fr];
        }
    }
    // S^T as the B operand of Qt S and Wk S: sST[j][c], 4 consecutive c per lane
    auto write_state_operand = [&]() __attribute__((always_inline)) {
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
    auto step = [&](auto DI, int n) __attribute__((always_inline)) {
        constexpr int d = DI;
        __syncthreads();                                            // S^T of chunk n's start state

        // ---- phase 1: W waves W = U - Wk S (to LDS as W^T); O waves O = Qt S
        floatx4 acc[NJW];
#pragma unroll
        for (int jt = 0; jt < NJW; ++jt) acc[jt] = zero4();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bf16x8 fa = __builtin_bit_cast(bf16x8, fA[d][u]);
#pragma unroll
            for (int jt = 0; jt < NJW; ++jt) {
                const bf16x8 fb =
                    *reinterpret_cast<const bf16x8*>(sST + ((jw0 + jt) * 16 + fr) * LDK + u * 32 + fk);
                acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[jt], 0, 0, 0);
            }
        }
        if (isW) {
#pragma unroll
            for (int jt = 0; jt < NJW; ++jt) {
                const bf16x4 uu = __builtin_bit_cast(bf16x4, fU[d][jt]);
                bf16x4 w4;
#pragma unroll
                for (int e = 0; e < 4; ++e) w4[e] = (bf16)((identW ? 0.f : (float)uu[e]) - acc[jt][e]);
                *reinterpret_cast<bf16x4*>(sWT + ((jw0 + jt) * 16 + fr) * LDC + R * 16 + 4 * (lane >> 4)) = w4;
            }
        }
        KDA_C64_PREFETCH_1(d, unit_of(n + D < NC ? n + D : NC - 1));
        __syncthreads();                                            // W^T complete

        // ---- phase 2: O waves O += P W (stored); all waves S = gam S + Kb^T W
        if (OUT && !wW) {
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
                const int tt = (c0 + n) * C + R * 16 + r;
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

    // end state: the call's final state (plain; the last segment of the outputs
    // launch), or the segment's E or M (maps launch)
    if constexpr (MAPS) {
        float* E = sg.E + (bh * sg.nseg + seg) * (long)(DK * DV);
        float* M = sg.M + (bh * sg.nseg + seg) * (long)(DK * DK);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int col = j0 + jt * 16;
            if (col >= DV && seg == 0) continue;           // M of segment 0 is never used
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = ct * 16 + 4 * (lane >> 4) + e;
                if (col >= DV) M[row * (long)DK + col - DV + fr] = accS[jt][e];
                else E[row * (long)DV + col + fr] = accS[jt][e];
            }
        }
    } else if (MODE == CHAIN_PLAIN || seg == sg.nseg - 1) {
        if (sT) {
            float* fin = sT + bh * (long)(DK * DV);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    fin[(ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + fr] = accS[jt][e];
        }
    }
}

// Start states of the segments from their maps: Sst_0 = S0 (zeros when NULL),
// Sst_1 = E_0 (segment 0 ran from S0 itself), Sst_{s+1} = M_s Sst_s + E_s.
// One workgroup per ((sequence, head), 4 value columns); thread t holds row t/2,
// columns 2(t%2) and 2(t%2)+1.  M_s is staged transposed in LDS (padded rows, so
// a wave's 32 rows read 32 banks), the next map is loaded into registers while
// the current one is used, and the sum over the DK channels runs in a fixed
// order in fp32.
template <int DK, int DV>
__global__ __launch_bounds__(256) void chain_seg_scan_kernel(const float* __restrict__ s0, Seg64 sg) {
    constexpr int NCOL = 4, PER = DK * DK / 4 / 256;       // float4 of a map per thread
    static_assert(DK == 128 && DV % NCOL == 0, "128 rows, 2 threads per row");
    __shared__ float sMT[DK][DK + 1];
    __shared__ float sS[DK][NCOL];
    const int cb = (int)(blockIdx.x % (DV / NCOL));
    const long bh = blockIdx.x / (DV / NCOL);
    const int tid = threadIdx.x, r = tid >> 1, jp = 2 * (tid & 1), col = cb * NCOL + jp;
    const long base = bh * sg.nseg;
    if (tid < DK) {
#pragma unroll
        for (int j = 0; j < NCOL; ++j) {
            const float x = s0 ? s0[(bh * DK + tid) * (long)DV + cb * NCOL + j] : 0.f;
            sS[tid][j] = x;
            sg.Sst[(base * DK + tid) * (long)DV + cb * NCOL + j] = x;
        }
    }
    floatx4 mreg[PER];
    auto load_map = [&](int s) {
        const floatx4* M = reinterpret_cast<const floatx4*>(sg.M + (base + s) * (long)(DK * DK));
#pragma unroll
        for (int i = 0; i < PER; ++i) mreg[i] = M[tid + 256 * i];
    };
    if (sg.nseg > 2) load_map(1);                          // M_1 is first used for Sst_2
    for (int s = 1; s < sg.nseg; ++s) {
        const float* E = sg.E + (base + s - 1) * (long)(DK * DV);
        const float e0 = E[r * DV + col], e1 = E[r * DV + col + 1];
        if (s > 1) {                                       // M_{s-1}, in registers, to LDS
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int u = tid + 256 * i, row = u >> 5, c0 = (u & 31) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) sMT[c0 + e][row] = mreg[i][e];
            }
            if (s + 1 < sg.nseg) load_map(s);              // the next step's map
        }
        __syncthreads();
        float a0 = 0.f, a1 = 0.f;
        if (s > 1) {
            for (int c = 0; c < DK; ++c) {
                const float m = sMT[c][r];
                a0 = fmaf(m, sS[c][jp], a0);
                a1 = fmaf(m, sS[c][jp + 1], a1);
            }
        }
        a0 += e0;
        a1 += e1;
        __syncthreads();
        sS[r][jp] = a0;
        sS[r][jp + 1] = a1;
        float* dst = sg.Sst + ((base + s) * DK + r) * (long)DV + col;
        dst[0] = a0;
        dst[1] = a1;
    }
}

#undef KDA_C64_PREFETCH_1
#undef KDA_C64_PREFETCH_2

template <typename TOut, int DV, int DVS, int MODE>
static hipError_t launch_chain64_mode(const ChunkArgs& a, long items, const Seg64& sg) {
    constexpr int C = 64, DK = 128;
    constexpr int NSLW = MODE == CHAIN_MAPS ? (DV + DK) / DVS : DV / DVS;
    const long nwg = items * NSLW;
    if (nwg == 0) return hipSuccess;
    const WsLayout w = ws_layout_of(a);
    char* ws = (char*)a.ws;
    hipLaunchKernelGGL((chunk_chain64_kernel<TOut, DV, DVS, MODE>), dim3((unsigned)nwg), dim3(512), 0, a.stream,
                       (const bf16*)(ws + w.qt), (const bf16*)(ws + w.wk), (const bf16*)(ws + w.kb),
                       (const bf16*)(ws + w.p), (const bf16*)(ws + w.u), (const float*)(ws + w.gam),
                       a.s0, MODE == CHAIN_MAPS ? nullptr : (TOut*)a.o, a.sT, unit_map(a), sg);
    return hipGetLastError();
}

// Slice width: 32 value columns when that gives at least 256 workgroups, else 16.
template <typename TOut, int DV>
static hipError_t launch_chain64(const ChunkArgs& a) {
    const long bh = seq_head_count(a);
    const SegPlan plan = seg_plan_of(a);
    if (plan.nseg > 1) {
        // segments: maps of all but the last, their scan, then every segment's outputs
        constexpr int DVS = SEG_DVS < DV ? SEG_DVS : DV;
        const WsLayout w = ws_layout_of(a);
        char* ws = (char*)a.ws;
        Seg64 sg{plan.L, plan.nseg, (float*)(ws + w.seg_e), (float*)(ws + w.seg_m), (float*)(ws + w.seg_s)};
        // (the maps write no outputs: one instantiation serves both output types);
        // with DV = DK every segment's whole augmented state is one workgroup, so
        // its Wk and Kb^T are fetched once
        constexpr int DVS_MAPS = DV == 128 ? 256 : DVS;
        hipError_t e = launch_chain64_mode<bf16, DV, DVS_MAPS, CHAIN_MAPS>(a, bh * (plan.nseg - 1), sg);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((chain_seg_scan_kernel<128, DV>), dim3((unsigned)(bh * (DV / 4))), dim3(256), 0,
                           a.stream, a.s0, sg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_chain64_mode<TOut, DV, DVS, CHAIN_SEG>(a, bh * plan.nseg, sg);
    }
    const Seg64 none{0, 1, nullptr, nullptr, nullptr};
    if (bh * (DV / 32) >= 256) return launch_chain64_mode<TOut, DV, 32, CHAIN_PLAIN>(a, bh, none);
    return launch_chain64_mode<TOut, DV, 16, CHAIN_PLAIN>(a, bh, none);
}

hipError_t run_chunk_chain64(const ChunkArgs& a) {
    if (a.dv == 64) return a.out_bf16 ? launch_chain64<bf16, 64>(a) : launch_chain64<float, 64>(a);
    return a.out_bf16 ? launch_chain64<bf16, 128>(a) : launch_chain64<float, 128>(a);
}

}  // namespace kda
