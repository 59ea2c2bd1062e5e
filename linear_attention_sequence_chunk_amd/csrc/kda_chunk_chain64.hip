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
// Long sequences with few (sequence, head) pairs are cut into segments (segment 0
// of L0 chunks, the others of L) that run side by side (segment-affine form).  A
// segment maps its start state to its end state affinely, S -> M S + E, with
// M = prod over its chunks of (Diag(gam) - Kb^T Wk) and E its end state from a
// zero start.  Three launches:
//   first (chain_maps64_kernel): segment 0 runs the chain with outputs from the
//         call's initial state and keeps its end state as E_0; beside it, each
//         segment 1 .. nseg - 2 runs the chain without outputs on the augmented
//         state [S | I]: value columns from a zero start give E, the dk extra
//         columns from the identity with U taken as 0 give M;
//   scan  (chain_seg_scan_kernel): start states Sst_0 = S0, Sst_1 = E_0,
//         Sst_{s+1} = M_s Sst_s + E_s, in fp32;
//   outputs (CHAIN_SEG): segments 1 .. nseg - 1 run the chain with outputs from
//         their start states; the last writes the final state.
// This is the chunk recurrence regrouped (the state after a chunk is an affine
// function of the state before it), so the result equals the sequential chain
// up to rounding; the extra cost is the maps.
#include "kda_chunk.h"

namespace kda {

// Workspace of this configuration, per chunk unit (chunk-major, as for every layout):
//   Qt, Wk [4 row tiles][4 k-steps][64 lanes][8 bf16]  lane l: row 16R + l%16, channels 32u + 8(l/16) + 0..7
//   Kb^T   [8 channel tiles][2 k-steps][64][8 bf16]     lane l: channel 16c + l%16, tokens 32u + 8(l/16) + 0..7
//   P      [4 row tiles][2 k-steps][64][8 bf16]         (row tiles 0, 1 at k-step 1 lie above the diagonal:
//                                                        never written, never read)
//   U      [4 row tiles][DV/16 column tiles][64][4] bf16  lane l, element e: row 16R + 4(l/16) + e, column 16J + l%16
//   gam    [DK] fp32
// CHAIN_CKPT: the plain chain without outputs, keeping the fp32 start state and W
// of every chunk for the backward pass
enum ChainMode { CHAIN_PLAIN = 0, CHAIN_SEG = 1, CHAIN_CKPT = 2 };

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
    // CHAIN_CKPT: each wave's 16 state rows, then the W waves' 16 rows of W, fp32,
    // staged so that the checkpoints go out as 16-byte row pieces
    static constexpr int LCK = DVS + 4;
    static constexpr size_t OFF_CK = TOTAL;
    static constexpr size_t TOTAL_CK = OFF_CK + size_t(12) * 16 * LCK * 4;
    static_assert((NJ == 1 || NJ == 2 || NJ == 4 || NJ == 8) && DV % DVS == 0, "slice width 16 .. 128");
    static_assert((16 * DVS * sizeof(TOut)) % 16 == 0, "output staging rows");
};

// Segments of a long sequence (maps and CHAIN_SEG launches); per (sequence, head) pair
// bh and segment s, the arrays hold [bh][s][DK][...] fp32.
struct Seg64 {
    int L0;                 // chunks of segment 0
    int L;                  // chunks of every later segment (the last may have fewer)
    int nseg;               // segments per (sequence, head)
    float* E;               // end state from a zero start (segment 0: from S0), [.][.][DK][DV]
    float* M;               // linear part of the segment's map, [.][.][DK][DK]
    float* Sst;             // start state of each segment, [.][.][DK][DV]
};
__device__ inline int seg_first(const Seg64& sg, int s) { return s == 0 ? 0 : sg.L0 + (s - 1) * sg.L; }
__device__ inline int seg_chunks(const Seg64& sg, int s, int nchunks) {
    const int c0 = seg_first(sg, s), len = s == 0 ? sg.L0 : sg.L;
    return nchunks - c0 < len ? nchunks - c0 : len;
}

// The chain of one work item and slice of DVS value columns: a (sequence, head)
// pair (CHAIN_PLAIN), or segment seg_lo + item % seg_cnt of pair item / seg_cnt
// (CHAIN_SEG).  smem holds Cfg::TOTAL bytes.
template <typename TOut, int DV, int DVS, int MODE>
__device__ __forceinline__ void chain64_run(
    char* smem, long item, int sl, int seg_lo, int seg_cnt,
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const bf16* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, float* __restrict__ sT, const UnitMap& um,
    const Seg64& sg, float* __restrict__ ck_state, float* __restrict__ ck_w) {
    typedef Chain64Cfg<TOut, DV, DVS> Cfg;
    constexpr int C = Cfg::C, DK = Cfg::DK, NJ = Cfg::NJ, LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr int D = Cfg::DEPTH;

    bf16* sST = reinterpret_cast<bf16*>(smem + Cfg::OFF_ST);
    bf16* sWT = reinterpret_cast<bf16*>(smem + Cfg::OFF_WT);
    float* sCk = reinterpret_cast<float*>(smem + Cfg::OFF_CK);    // CHAIN_CKPT only
    constexpr int LCK = Cfg::LCK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 16 staged fp32 rows of DVS columns to global rows of DV floats, 16 bytes a lane
    auto ckpt_rows = [&](const float* rows, float* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < DVS / 16; ++p) {
            const int u = lane + 64 * p, r = u / (DVS / 4), c4 = u % (DVS / 4);
            *reinterpret_cast<floatx4*>(dst + r * (long)DV + 4 * c4) =
                *reinterpret_cast<const floatx4*>(rows + r * LCK + 4 * c4);
        }
    };
    // work item -> (sequence, head) pair and segment
    const long bh = item / seg_cnt;
    const int seg = seg_lo + (int)(item % seg_cnt);
    const int j0 = sl * DVS;                      // first value column of the slice
    // sequence (batch row, or packed sequence) and head; its chunks and tokens
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int c0 = MODE != CHAIN_SEG ? 0 : seg_first(sg, seg);              // first chunk of the segment
    const int NC = MODE != CHAIN_SEG ? sr.nchunks : seg_chunks(sg, seg, sr.nchunks);
    auto unit_of = [&](int n) -> long { return unit_id(um, sq, h, c0 + n, sr.chunk0); };

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
    u32x2 fU[D][NJ];     // U tiles of the slice (W waves; a repeat of fA on O waves)
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
                                   + (R * (DV / 16) + (j0 / 16)) * 64 + lane                        \
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
    // start: the call's initial state (plain; segment 0), or the segment's start state
    const float* init = MODE == CHAIN_SEG && seg > 0 ? sg.Sst + (bh * sg.nseg + seg) * (long)(DK * DV)
                                                     : (s0 ? s0 + bh * (long)(DK * DV) : nullptr);
    floatx4 accS[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        accS[jt] = zero4();
        if (init) {
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
                if constexpr (MODE == CHAIN_CKPT) {                // W of chunk n, fp32, to this wave's rows
                    float* wt = sCk + (8 + R) * 16 * LCK;
#pragma unroll
                    for (int e = 0; e < 4; ++e) wt[(4 * (lane >> 4) + e) * LCK + jt * 16 + fr] = (float)uu[e] - acc[jt][e];
                }
            }
            if constexpr (MODE == CHAIN_CKPT) ckpt_rows(sCk + (8 + R) * 16 * LCK, ck_w + unit_of(n) * (long)(C * DV) +
                                                        (R * 16) * (long)DV + j0);
        }
        if constexpr (MODE == CHAIN_CKPT) {                        // the state chunk n starts from
            float* st = sCk + wave * 16 * LCK;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[(4 * (lane >> 4) + e) * LCK + jt * 16 + fr] = accS[jt][e];
            ckpt_rows(st, ck_state + unit_of(n) * (long)(DK * DV) + (ct * 16) * (long)DV + j0);
        }
        KDA_C64_PREFETCH_1(d, unit_of(n + D < NC ? n + D : NC - 1));
        __syncthreads();                                            // W^T complete

        // ---- phase 2: O waves O += P W; all waves S = gam S + Kb^T W and the next
        // S^T (what the next chunk waits for) before the O waves store their outputs
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
        if (MODE != CHAIN_CKPT && !wW) {
            // this wave's 16 x DVS output tile, through its own LDS rows, as 16-byte row
            // pieces with streaming stores (no later kernel here reads o)
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
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(sO + r * DVS + jj),
                        reinterpret_cast<u32x4*>(o + ((sr.tok_begin + tt) * H + h) * DV + j0 + jj));
            }
        }
        KDA_C64_PREFETCH_2(d, unit_of(n + D < NC ? n + D : NC - 1));
    };
    // whole rounds of D chunks with no condition inside (the loads in flight are
    // then the same on every path), then the last NC % D chunks
    int n0 = 0;
    for (; n0 + D <= NC; n0 += D) static_for<D>([&](auto DI) { step(DI, n0 + DI); });
    static_for<D>([&](auto DI) {
        if (n0 + DI < NC) step(DI, n0 + DI);
    });

    // end state: the call's final state (plain; the last segment), or segment 0's
    // end state E_0, which the scan takes as segment 1's start state
    float* fin = nullptr;
    if (MODE != CHAIN_SEG || seg == sg.nseg - 1) fin = sT ? sT + bh * (long)(DK * DV) : nullptr;
    else if (seg == 0) fin = sg.E + (bh * sg.nseg) * (long)(DK * DV);
    if (fin) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                fin[(ct * 16 + 4 * (lane >> 4) + e) * (long)DV + j0 + jt * 16 + fr] = accS[jt][e];
    }
}

template <typename TOut, int DV, int DVS, int MODE>
__global__ __launch_bounds__(512, 1) void chunk_chain64_kernel(
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const bf16* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, float* __restrict__ sT, UnitMap um, Seg64 sg,
    int seg_lo, int seg_cnt, float* __restrict__ ck_state, float* __restrict__ ck_w) {
    typedef Chain64Cfg<TOut, DV, DVS> Cfg;
    constexpr int NSL = Cfg::NSL;
    __shared__ __attribute__((aligned(16))) char smem[MODE == CHAIN_CKPT ? Cfg::TOTAL_CK : Cfg::TOTAL];
    // Slices of one work item (a (sequence, head) pair, or one of its segments)
    // share an XCD (workgroups are dealt to the 8 XCDs round-robin), so the
    // per-chunk operands they all read come from one L2.
    long item;
    int sl;
    {
        const long nwg = (long)gridDim.x, id = blockIdx.x;
        if (!um.cu_seqlens && nwg % (8 * NSL) == 0) {
            const long xcd = id % 8, local = id / 8;
            sl = (int)(local % NSL);
            item = (local / NSL) * 8 + xcd;
        } else {
            item = id / NSL;
            sl = (int)(id % NSL);
        }
    }
    chain64_run<TOut, DV, DVS, MODE>(smem, item, sl, seg_lo, seg_cnt, ws_qt, ws_wk, ws_kb, ws_p, ws_u, ws_gam,
                                     s0, o, sT, um, sg, ck_state, ck_w);
}

// The maps launch with the whole augmented state [S | I] (DV + DK columns) in one
// workgroup of 8 waves.  Each wave owns 32 columns (waves 0 .. DV/32 - 1 value
// columns, the next four the identity columns) and carries them through the
// whole chunk step on its own:
//   V = U - Wk S     (64 x 32; U taken as 0 on identity columns)
//   S <- gam S + Kb^T V   (DK x 32, fp32 in accumulators)
// so neither S nor V is exchanged between waves.  The B operand of each product
// is built in registers from the accumulators of the previous one: a 16 x 16 fp32
// accumulator gives lane l the rows 4(l/16) .. +3 of its column, so the B operand
// of a 32-deep k-step is taken from two vertically adjacent tiles, lane l holding
// rows {4(l/16) .. +3} and {16 + 4(l/16) .. +3}.  The A operands (Wk, Kb^T) are
// read with the same order of k: two 8-byte pieces of their fragment-order rows.
// Wk, Kb^T, U and gam are staged in LDS once per workgroup, double-buffered by
// chunk parity, from registers loaded two chunks ahead.  One barrier per chunk.
template <int DV>
struct Maps64Cfg {
    static constexpr int C = 64, DK = 128;
    static constexpr int NVW = DV / 32, NAW = NVW + DK / 32;     // value waves; waves holding columns
    static constexpr int NWK = C * DK * 2 / 16 / 512, NUV = C * DV * 2 / 16 / 512;   // 16-byte loads a lane
    static constexpr size_t OFF_WK = 0;                                  // Wk, fragment order
    static constexpr size_t OFF_KB = OFF_WK + size_t(C) * DK * 2;       // Kb^T, fragment order
    static constexpr size_t OFF_U = OFF_KB + size_t(DK) * C * 2;        // U, fragment order
    static constexpr size_t OFF_G = OFF_U + size_t(C) * DV * 2;         // gam [DK] fp32
    static constexpr size_t BUF = OFF_G + size_t(DK) * 4;
    static constexpr size_t TOTAL = 2 * BUF;
    static_assert(NAW <= 8 && NWK >= 1 && NUV >= 1, "wave and load mapping");
    static_assert(TOTAL <= 160 * 1024, "LDS");
};

// The first launch of the segmented chain: workgroups 0 .. nout - 1 run segment 0
// of each (sequence, head) pair with its outputs (its start state is the call's
// S0, and its end state is E_0); the others the maps of segments 1 .. nseg - 2.
template <typename TOut, int DV>
__global__ __launch_bounds__(512, 1) void chain_maps64_kernel(
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const bf16* __restrict__ ws_u, const float* __restrict__ ws_gam,
    const float* __restrict__ s0, TOut* __restrict__ o, UnitMap um, Seg64 sg, long nout) {
    typedef Maps64Cfg<DV> Cfg;
    typedef Chain64Cfg<TOut, DV, DV> OCfg;
    constexpr int C = Cfg::C, DK = Cfg::DK, NVW = Cfg::NVW, NAW = Cfg::NAW, NWK = Cfg::NWK, NUV = Cfg::NUV;
    constexpr size_t BUF = Cfg::BUF;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL > OCfg::TOTAL ? Cfg::TOTAL : OCfg::TOTAL];
    if (blockIdx.x < nout) {
        chain64_run<TOut, DV, DV, CHAIN_SEG>(smem, blockIdx.x, 0, 0, 1, ws_qt, ws_wk, ws_kb, ws_p, ws_u, ws_gam,
                                             s0, o, nullptr, um, sg, nullptr, nullptr);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 15, fg = lane >> 4;
    const long item = blockIdx.x - nout;
    const int nsegw = sg.nseg - 2;                   // segment 0 and the last segment need no map
    const long bh = item / nsegw;
    const int seg = 1 + (int)(item % nsegw);
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int c0 = seg_first(sg, seg);
    const int NC = seg_chunks(sg, seg, sr.nchunks);
    auto unit_of = [&](int n) -> long { return unit_id(um, sq, h, c0 + (n < NC ? n : NC - 1), sr.chunk0); };

    // ---- staging: chunk m in register slot m % 2, then in LDS buffer m % 2
    u32x4 fW[2][NWK], fK[2][NWK], fV[2][NUV], fG[2];
    auto load = [&](auto SI, long ch) __attribute__((always_inline)) {
        constexpr int sl = SI;
        const u32x4* a = reinterpret_cast<const u32x4*>(ws_wk + ch * (long)(C * DK)) + tid;
        const u32x4* k = reinterpret_cast<const u32x4*>(ws_kb + ch * (long)(DK * C)) + tid;
        const u32x4* u = reinterpret_cast<const u32x4*>(ws_u + ch * (long)(C * DV)) + tid;
#pragma unroll
        for (int i = 0; i < NWK; ++i) { fW[sl][i] = a[512 * i]; fK[sl][i] = k[512 * i]; }
#pragma unroll
        for (int i = 0; i < NUV; ++i) fV[sl][i] = u[512 * i];
        fG[sl] = reinterpret_cast<const u32x4*>(ws_gam + ch * (long)DK)[tid & (DK / 4 - 1)];
    };
    auto stage = [&](auto SI) __attribute__((always_inline)) {
        constexpr int sl = SI;
        char* b = smem + sl * BUF;
#pragma unroll
        for (int i = 0; i < NWK; ++i) {
            reinterpret_cast<u32x4*>(b + Cfg::OFF_WK)[tid + 512 * i] = fW[sl][i];
            reinterpret_cast<u32x4*>(b + Cfg::OFF_KB)[tid + 512 * i] = fK[sl][i];
        }
#pragma unroll
        for (int i = 0; i < NUV; ++i) reinterpret_cast<u32x4*>(b + Cfg::OFF_U)[tid + 512 * i] = fV[sl][i];
        if (tid < DK / 4) reinterpret_cast<u32x4*>(b + Cfg::OFF_G)[tid] = fG[sl];
    };
    if (NC > 0) {
        load(std::integral_constant<int, 0>{}, unit_of(0));
        load(std::integral_constant<int, 1>{}, unit_of(1));
        stage(std::integral_constant<int, 0>{});
        load(std::integral_constant<int, 0>{}, unit_of(2));
    }

    // ---- this wave's 32 columns of [S | I]: tiles (r, jt), rows 16r + 4(l/16) + e,
    // column 32 w + 16 jt + l%16 of the value part (w < NVW) or of the identity part
    const bool val = wave < NVW, act = wave < NAW;               // uniform per wave
    const int cbase = 32 * (val ? wave : wave - NVW);
    floatx4 accS[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                accS[r][jt][e] = !val && 16 * r + 4 * fg + e == cbase + 16 * jt + fr ? 1.f : 0.f;
    // byte offset of lane l's first 8-byte A piece in a 1 KB fragment (the second is 512 bytes on)
    const int aoff = (fr + 16 * (fg >> 1)) * 16 + 8 * (fg & 1);
    auto afrag = [&](const char* f) __attribute__((always_inline)) -> bf16x8 {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(f + aoff), hi = *reinterpret_cast<const u32x2*>(f + aoff + 512);
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };

    // chunk n, whose operands are in LDS buffer d = n % 2
    auto step = [&](auto DI, int n) __attribute__((always_inline)) {
        constexpr int d = DI, d1 = 1 - DI;
        __syncthreads();                                   // buffer d complete; buffer d1 no longer read
        stage(std::integral_constant<int, d1>{});          // chunk n + 1
        load(std::integral_constant<int, d1>{}, unit_of(n + 3));
        if (!act) return;
        const char* b = smem + d * BUF;
        // V = U - Wk S: accumulators start from U (value columns) and add Wk (-S)
        floatx4 accV[4][2];
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                accV[R][jt] = zero4();
                if (val) {
                    const bf16x4 uu = *reinterpret_cast<const bf16x4*>(
                        b + Cfg::OFF_U + ((R * (DV / 16) + 2 * wave + jt) * 64 + lane) * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) accV[R][jt][e] = (float)uu[e];
                }
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 bs[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bs[jt][e] = (bf16)(-accS[2 * s][jt][e]);
                    bs[jt][4 + e] = (bf16)(-accS[2 * s + 1][jt][e]);
                }
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const bf16x8 fa = afrag(b + Cfg::OFF_WK + (R * 4 + s) * 1024);
                accV[R][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bs[0], accV[R][0], 0, 0, 0);
                accV[R][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bs[1], accV[R][1], 0, 0, 0);
            }
        }
        // S <- gam S + Kb^T V
        bf16x8 bv[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bv[s][jt][e] = (bf16)accV[2 * s][jt][e];
                    bv[s][jt][4 + e] = (bf16)accV[2 * s + 1][jt][e];
                }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const floatx4 gm = *reinterpret_cast<const floatx4*>(b + Cfg::OFF_G + (16 * r + 4 * fg) * 4);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[r][jt][e] *= gm[e];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 fa = afrag(b + Cfg::OFF_KB + (r * 2 + s) * 1024);
                accS[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bv[s][0], accS[r][0], 0, 0, 0);
                accS[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bv[s][1], accS[r][1], 0, 0, 0);
            }
    };
    // pairs of chunks (slot and buffer parities as constants), then an odd last one
    int n0 = 0;
    for (; n0 + 2 <= NC; n0 += 2) {
        step(std::integral_constant<int, 0>{}, n0);
        step(std::integral_constant<int, 1>{}, n0 + 1);
    }
    if (n0 < NC) step(std::integral_constant<int, 0>{}, n0);

    // E (value columns) and M (identity columns)
    if (!act) return;
    float* dst = val ? sg.E + (bh * sg.nseg + seg) * (long)(DK * DV)
                     : sg.M + (bh * sg.nseg + seg) * (long)(DK * DK);
    const int ld = val ? DV : DK;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(16 * r + 4 * fg + e) * (long)ld + cbase + 16 * jt + fr] = accS[r][jt][e];
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
static hipError_t launch_chain64_mode(const ChunkArgs& a, long items, const Seg64& sg, int seg_lo, int seg_cnt) {
    const long nwg = items * (DV / DVS);
    if (nwg == 0) return hipSuccess;
    const WsLayout w = ws_layout_of(a);
    char* ws = (char*)a.ws;
    hipLaunchKernelGGL((chunk_chain64_kernel<TOut, DV, DVS, MODE>), dim3((unsigned)nwg), dim3(512), 0, a.stream,
                       (const bf16*)(ws + w.qt), (const bf16*)(ws + w.wk), (const bf16*)(ws + w.kb),
                       (const bf16*)(ws + w.p), (const bf16*)(ws + w.u), (const float*)(ws + w.gam),
                       a.s0, (TOut*)a.o, a.sT, unit_map(a), sg, seg_lo, seg_cnt, a.ck_state, a.ck_w);
    return hipGetLastError();
}

// Slice width: 32 value columns when that gives at least 256 workgroups, else 16.
template <typename TOut, int DV>
static hipError_t launch_chain64(const ChunkArgs& a) {
    const long bh = seq_head_count(a);
    const SegPlan plan = seg_plan_of(a);
    if (plan.nseg > 2) {
        // segments: segment 0's outputs beside the maps of segments 1 .. nseg - 2,
        // the scan of the maps, then the outputs of segments 1 .. nseg - 1
        static_assert(SEG_DVS >= DV, "one workgroup per segment holds every value column");
        const WsLayout w = ws_layout_of(a);
        char* ws = (char*)a.ws;
        Seg64 sg{plan.L0, plan.L, plan.nseg, (float*)(ws + w.seg_e), (float*)(ws + w.seg_m), (float*)(ws + w.seg_s)};
        // every segment's whole augmented state is one workgroup, so its Wk and
        // Kb^T are fetched once
        const long nwg = bh + bh * (plan.nseg - 2);
        hipLaunchKernelGGL((chain_maps64_kernel<TOut, DV>), dim3((unsigned)nwg), dim3(512), 0, a.stream,
                           (const bf16*)(ws + w.qt), (const bf16*)(ws + w.wk), (const bf16*)(ws + w.kb),
                           (const bf16*)(ws + w.p), (const bf16*)(ws + w.u), (const float*)(ws + w.gam), a.s0,
                           (TOut*)a.o, unit_map(a), sg, bh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((chain_seg_scan_kernel<128, DV>), dim3((unsigned)(bh * (DV / 4))), dim3(256), 0,
                           a.stream, a.s0, sg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_chain64_mode<TOut, DV, DV, CHAIN_SEG>(a, bh * (plan.nseg - 1), sg, 1, plan.nseg - 1);
    }
    const Seg64 none{0, 0, 1, nullptr, nullptr, nullptr};
    if (a.checkpoints) {                                       // the backward pass's forward chain
        if (!a.ck_state || !a.ck_w) return hipErrorInvalidValue;
        if (bh * (DV / 32) >= 256) return launch_chain64_mode<TOut, DV, 32, CHAIN_CKPT>(a, bh, none, 0, 1);
        return launch_chain64_mode<TOut, DV, 16, CHAIN_CKPT>(a, bh, none, 0, 1);
    }
    if (bh * (DV / 32) >= 256) return launch_chain64_mode<TOut, DV, 32, CHAIN_PLAIN>(a, bh, none, 0, 1);
    return launch_chain64_mode<TOut, DV, 16, CHAIN_PLAIN>(a, bh, none, 0, 1);
}

hipError_t run_chunk_chain64(const ChunkArgs& a) {
    if (a.dv == 64) return a.out_bf16 ? launch_chain64<bf16, 64>(a) : launch_chain64<float, 64>(a);
    return a.out_bf16 ? launch_chain64<bf16, 128>(a) : launch_chain64<float, 128>(a);
}

}  // namespace kda
