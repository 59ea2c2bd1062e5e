// kda_chunk.h -- chunkwise-parallel KDA forward on gfx950: two stages.
//
// Shared by kda_chunk_intra.hip (stage 1 and the host dispatch) and
// kda_chunk_chain_*.hip (stage 2, one file per input dtype so that they build in
// parallel).
//
// The chunkwise form (chunk paragraph of "一个KimiK3装下22580个GPT-2…";
// sections 十六 and 十七 of "我终于看懂了 KDA…"): the sequence is cut into chunks
// of C tokens; inside a chunk the work is parallel (masked attention scores and
// the chunk's rank-1 updates folded into matrix products, the WY / DPLR view),
// across chunks the state is carried sequentially.  For a chunk with local
// positions r, i, start state S and per-channel log-gate prefix sums G:
//
//   A_ri = sum_c k_rc k_ic e^{G_rc - G_ic} (i < r)     P_ri = sum_c q_rc k_ic e^{G_rc - G_ic} (i <= r)
//   T    = (I + Diag(beta) A)^-1
//   U    = T Diag(beta) V          Wk = T Diag(beta) (e^G * K)
//   W    = U - Wk S                (row r is the token's correction u_r)
//   O    = (e^G * Q) S + P W
//   S   <- Diag(e^{G_last}) S + (e^{G_last - G} * K)^T W
//
// Stage 1 (chunk_intra_kernel, one workgroup per (b, h, chunk), all chunks in
// parallel) computes everything that does not depend on S into a workspace:
// Qt = e^G*Q, Wk, Kb = e^{G_last-G}*K, P, U and gam = e^{G_last}.
// Stage 2 (chunk_chain_kernel, one workgroup per (b, h, value-column slice))
// walks the chunks in order with the fp32 state in MFMA accumulators.
//
// Exponent safety.  e^{G_r - G_i} is never formed as e^{G_r} * e^{-G_i} across a
// whole chunk (the chunk sum of log-gates can pass -88, where e^{-G} overflows
// fp32).  The chunk is split into 16-token sub-blocks; a pair of sub-blocks
// (R, I), I < R, is handled at the level of the binary split where they separate,
// with the split point m as reference: the row factor e^{G_r - G_{m-1}} and the
// column factor e^{G_{m-1} - G_i} are both <= 1.  Diagonal sub-blocks use the
// block start as reference; this is exact as long as the block's own log-gate sum
// stays above -SAFE_SPAN, otherwise that block is computed term by term.
// Prefix sums are kept block-local (16 tokens) so that exponent differences do
// not lose digits to a large running sum.
#pragma once

#include <utility>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// ------------------------------------------------------------ compile-time helpers
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
// Lower-triangular sub-block pairs (R, I), I <= R, enumerated p = R(R+1)/2 + I.
constexpr int pair_R(int p) { int R = 0; while ((R + 1) * (R + 2) / 2 <= p) ++R; return R; }
constexpr int pair_I(int p) { return p - pair_R(p) * (pair_R(p) + 1) / 2; }
// Segment length (tokens) of the binary split that separates R and I; 0 = diagonal.
constexpr int pair_level(int p) { return pair_R(p) == pair_I(p) ? 0 : 32 << ilog2(pair_R(p) ^ pair_I(p)); }
constexpr size_t align16(size_t x) { return (x + 15) & ~size_t(15); }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr size_t smax(size_t a, size_t b) { return a > b ? a : b; }

constexpr size_t LDS_LIMIT = 160 * 1024;

// Two accumulators sharing the B operand: acc1 += A1 B, acc2 += A2 B.
template <typename T>
__device__ inline void mma_tile2(floatx4& acc1, floatx4& acc2, const T* __restrict__ a1,
                                 const T* __restrict__ a2, int lda, const T* __restrict__ bt,
                                 int ldb, int K, int lane) {
    typedef typename Mma<T>::frag frag;
    const int r = lane & 15, kg = lane >> 4;
    const int oa = r * lda + kg * Mma<T>::KPL, ob = r * ldb + kg * Mma<T>::KPL;
    for (int k0 = 0; k0 < K; k0 += Mma<T>::KSTEP) {
        frag fb = *reinterpret_cast<const frag*>(bt + ob + k0);
        frag f1 = *reinterpret_cast<const frag*>(a1 + oa + k0);
        frag f2 = *reinterpret_cast<const frag*>(a2 + oa + k0);
        acc1 = Mma<T>::mma(f1, fb, acc1);
        acc2 = Mma<T>::mma(f2, fb, acc2);
    }
}

// fp32 MFMA with both operands stored row-major: A[row][k], B[k][col].
__device__ inline floatx4 mma_f32_rowB(floatx4 acc, const float* a, int lda, const float* b,
                                       int ldb, int K, int lane) {
    const int r = lane & 15, kg = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * lda + k0 + kg], b[(k0 + kg) * ldb + r], acc, 0, 0, 0);
    return acc;
}

template <typename T> struct Pair2;
template <> struct Pair2<bf16> {
    __device__ static inline void load(const bf16* p, float& x, float& y) {
        bf16x2 v = *reinterpret_cast<const bf16x2*>(p); x = (float)v[0]; y = (float)v[1];
    }
    __device__ static inline void store(bf16* p, float x, float y) {
        bf16x2 v; v[0] = (bf16)x; v[1] = (bf16)y; *reinterpret_cast<bf16x2*>(p) = v;
    }
};
template <> struct Pair2<float> {
    __device__ static inline void load(const float* p, float& x, float& y) {
        float2 v = *reinterpret_cast<const float2*>(p); x = v.x; y = v.y;
    }
    __device__ static inline void store(float* p, float x, float y) {
        *reinterpret_cast<float2*>(p) = make_float2(x, y);
    }
};

// ================================================================ stage 1: intra
template <typename T, int DK, int DV, int C>
struct IntraCfg {
    static constexpr int NB = C / 16;                       // 16-token sub-blocks
    static constexpr int NP = NB * (NB + 1) / 2;            // lower-triangular block pairs
    static constexpr int NSLOT = (NP + 3) / 4;              // per-wave accumulator slots
    static constexpr int NLV = ilog2(NB);                   // cross levels
    static constexpr int HR = cmax(16, C / 2);              // rows per operand buffer
    static constexpr int NPASS = C / HR;                    // passes of the diagonal level
    static constexpr int PADT = sizeof(T) == 2 ? 8 : 4;     // 16-byte row padding
    static constexpr int LDK = DK + PADT;
    static constexpr int CK = cmax(C, Mma<T>::KSTEP);       // contraction length over positions
    static constexpr int LDT = CK + PADT;
    static constexpr int LDA = C + 8;
    static constexpr size_t SZ_L = size_t(C) * DK * 4;
    static constexpr size_t SZ_OP = size_t(HR) * LDK * sizeof(T);
    static constexpr size_t PHASE_S = SZ_L + 3 * SZ_OP;
    static constexpr size_t SZ_TB = align16(size_t(C) * LDT * sizeof(T));
    static constexpr size_t SZ_A = size_t(C) * LDA * 4;
    static constexpr size_t SZ_VK = size_t(DV + DK) * LDT * sizeof(T);
    static constexpr size_t PHASE_W = SZ_TB + smax(SZ_A, SZ_VK);
    static constexpr size_t OFF_TOT = align16(smax(PHASE_S, PHASE_W));
    static constexpr size_t OFF_OFF = OFF_TOT + size_t(NB) * DK * 4;
    static constexpr size_t OFF_BETA = OFF_OFF + size_t(NB) * DK * 4;
    static constexpr size_t OFF_FLAG = OFF_BETA + size_t(C) * 4;
    static constexpr size_t OFF_QN = align16(OFF_FLAG + size_t(NB) * 4);   // 1/||q||, 1/||k|| [2][C]
    static constexpr size_t TOTAL = align16(OFF_QN + size_t(2) * C * 4);
    static constexpr bool FITS = TOTAL <= LDS_LIMIT;
};

// ================================================================ stage 2: chain
template <typename T, typename TOut, int DK, int DV, int C, int DVS>
struct ChainCfg {
    static constexpr int PADT = sizeof(T) == 2 ? 8 : 4;
    static constexpr int LDK = DK + PADT;
    static constexpr int CK = cmax(C, Mma<T>::KSTEP);
    static constexpr int LDC = CK + PADT;
    static constexpr int NJ = DVS / 16;
    static constexpr int NTW = (C / 16) * NJ;               // W / O tiles
    static constexpr int NTS = (DK / 16) * NJ;              // state tiles
    // each wave owns whole row tiles: RPW rows of W / O, SPW rows of the state
    static constexpr int RPW = (C / 16 + 3) / 4, SPW = DK / 64;
    // prefetch units of 16 bytes: Qt, Wk, Kb^T, P (input dtype), U slice, gam (fp32)
    static constexpr int E16 = 16 / sizeof(T);
    static constexpr int U_QT = C * DK / E16, U_WK = U_QT, U_KB = DK * C / E16, U_P = C * C / E16;
    static constexpr int U_U = C * DVS / 4, U_G = DK / 4;
    static constexpr int B1 = U_QT, B2 = B1 + U_WK, B3 = B2 + U_KB, B4 = B3 + U_P, B5 = B4 + U_U;
    static constexpr int NU = B5 + U_G;
    static constexpr int NUPT = (NU + 255) / 256;
    // chunks in flight: as many 16-byte-unit register sets as ~160 VGPRs allow
    static constexpr int DEPTH = (160 / (4 * NUPT)) < 1 ? 1 : ((160 / (4 * NUPT)) > 3 ? 3 : 160 / (4 * NUPT));
    static constexpr size_t SZ_QT = size_t(C) * LDK * sizeof(T);
    static constexpr size_t SZ_KBT = align16(size_t(DK) * LDC * sizeof(T));
    static constexpr size_t SZ_P = align16(size_t(C) * LDC * sizeof(T));
    static constexpr size_t SZ_U = size_t(C) * DVS * 4;
    static constexpr size_t SZ_GAM = size_t(DK) * 4;
    static constexpr size_t SZ_ST = size_t(DVS) * LDK * sizeof(T);
    static constexpr size_t SZ_WT = align16(size_t(DVS) * LDC * sizeof(T));
    static constexpr size_t SZ_O = align16(size_t(C) * DVS * sizeof(TOut));
    static constexpr size_t OFF_WK = SZ_QT;
    static constexpr size_t OFF_KBT = OFF_WK + SZ_QT;
    static constexpr size_t OFF_P = OFF_KBT + SZ_KBT;
    static constexpr size_t OFF_U = OFF_P + SZ_P;
    static constexpr size_t OFF_GAM = OFF_U + SZ_U;
    static constexpr size_t OFF_ST = OFF_GAM + SZ_GAM;
    static constexpr size_t OFF_WT = OFF_ST + SZ_ST;
    static constexpr size_t OFF_O = OFF_WT + SZ_WT;
    // outputs are staged in LDS for 16-byte row stores when there is room
    static constexpr bool STAGE_O = OFF_O + SZ_O <= LDS_LIMIT && (DVS * sizeof(TOut)) % 16 == 0;
    static constexpr size_t TOTAL = STAGE_O ? OFF_O + SZ_O : OFF_O;
    static constexpr bool FITS = TOTAL <= LDS_LIMIT && NUPT <= 40 && U_G <= 256;
};

template <typename T, typename TOut, int DK, int DV, int C, int DVS>
constexpr bool chain_fits() { return DVS <= DV && ChainCfg<T, TOut, DK, DV, C, DVS>::FITS; }

// ------------------------------------------------------------ chunk units
// Fixed-length batches [B,T,H,d]: chunk n of sequence b and head h is unit
// n * (B*H) + b*H + h (chunk-major).  Packed variable-length batches [T,H,d]
// with token offsets cu_seqlens[N+1]: chunk j, counted over all sequences in
// order, of head h is unit j*H + h.  A device pass (packed_chunks_kernel) first
// turns the offsets into cu_tok[s] = min(T, max(0, cu_seqlens[0..s])), a
// running maximum clamped to [0, T], and cu_chunks[s], the first chunk of
// sequence s; every kernel reads only those.  Sequence s is tokens
// [cu_tok[s], cu_tok[s+1]): the ranges are disjoint and lie inside [0, T]
// whatever cu_seqlens holds, so the chunks of all sequences number at most
// ceil(T/C) + N, the units the workspace and the grids are sized for.
struct UnitMap {
    int T_len;                 // tokens per sequence (fixed) or in all (packed)
    int H, C, NC;              // NC: chunks per sequence (fixed)
    long BH;                   // B*H (fixed)
    const int* cu_seqlens;     // NULL for fixed-length batches (only tested against NULL)
    const int* cu_chunks;      // [N+1] first chunk of each sequence, then the total
    const int* cu_tok;         // [N+1] clamped, non-decreasing token offsets
    int nseq;
};
struct SeqRange { long tok_begin, tok_end, chunk0; int nchunks; };
struct UnitPos { long tok0; int count, h; };

__device__ inline long clamp_tok(long x, long lo, long hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Tokens and chunks of sequence s (b for fixed-length batches).
__device__ inline SeqRange seq_range(const UnitMap& m, int s) {
    SeqRange r;
    if (!m.cu_seqlens) {
        r.tok_begin = (long)s * m.T_len; r.tok_end = r.tok_begin + m.T_len;
        r.chunk0 = 0; r.nchunks = m.NC;
    } else {
        r.tok_begin = m.cu_tok[s];
        r.tok_end = m.cu_tok[s + 1];
        r.chunk0 = m.cu_chunks[s];
        r.nchunks = m.cu_chunks[s + 1] - m.cu_chunks[s];
    }
    return r;
}
// Unit id of chunk n of (sequence s, head h); chunk0 from seq_range.
__device__ inline long unit_id(const UnitMap& m, int s, int h, int n, long chunk0) {
    return m.cu_seqlens ? (chunk0 + n) * m.H + h : (long)n * m.BH + (long)s * m.H + h;
}
// First token and token count of a unit; false for a unit past the last chunk
// of a packed batch (the grid is sized for the most chunks there can be).
// Units number fewer than 2^31 (the host refuses larger calls), so the divisions
// here are 32-bit unsigned: a few dozen instructions at each workgroup's start
// instead of the several hundred of a 64-bit division.
__device__ inline bool unit_pos(const UnitMap& m, long unit, UnitPos& p) {
    const unsigned u = (unsigned)unit, H = (unsigned)m.H;
    if (!m.cu_seqlens) {
        const unsigned BH = (unsigned)m.BH;
        const unsigned n32 = u / BH, bh = u - n32 * BH, b = bh / H;
        const int n = (int)n32;
        p.h = (int)(bh - b * H);
        p.tok0 = (long)b * m.T_len + (long)n * m.C;
        p.count = m.T_len - n * m.C < m.C ? m.T_len - n * m.C : m.C;
        return true;
    }
    const unsigned j32 = u / H;
    const long j = j32;
    p.h = (int)(u - j32 * H);
    if (j >= m.cu_chunks[m.nseq]) return false;
    int lo = 0, hi = m.nseq;                     // cu_chunks[lo] <= j < cu_chunks[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (m.cu_chunks[mid] <= j) lo = mid; else hi = mid;
    }
    const SeqRange r = seq_range(m, lo);
    p.tok0 = r.tok_begin + (j - r.chunk0) * m.C;
    const long left = r.tok_end - p.tok0;
    p.count = left < m.C ? (int)left : m.C;
    return true;
}

// Host side: the map for a call (cu_chunks inside the workspace for packed batches).
UnitMap unit_map(const ChunkArgs& a);
long unit_count(const ChunkArgs& a);          // workgroups of the intra stage
long seq_head_count(const ChunkArgs& a);      // (sequence, head) pairs of the chain stage

// Stage 2 for each input dtype (kda_chunk_chain_bf16.hip, kda_chunk_chain_f32.hip).
hipError_t run_chunk_chain_bf16(const ChunkArgs& a);
hipError_t run_chunk_chain_f32(const ChunkArgs& a);

// The hot configuration has its own pair of kernels, chunk_intra64_kernel and
// chunk_chain64_kernel, and its own workspace format; both stages decide with this.
inline bool hot_layout(const ChunkArgs& a) { return hot_config(a.in_bf16, a.dk, a.C) && !a.checkpoints; }
hipError_t run_chunk_chain64(const ChunkArgs& a);   // kda_chunk_chain64.hip

}  // namespace kda
