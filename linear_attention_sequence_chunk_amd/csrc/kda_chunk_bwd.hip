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
// stages, which run again for this (fp32 checkpoints).  Gradients accumulate
// in fp32; products of fp32 operands over the long dimensions run on bf16 MFMA
// with each operand split into bf16 hi + lo parts (about 16 significant bits).
#include "kda_chunk.h"

namespace kda {

// ================================================================ fp32 MFMA helpers
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][slot] and B[slot][l%16], and
// accumulator element e of lane l is D[4(l/16)+e][l%16].  A 16-deep contraction
// is four instructions in which lane l covers k = 4(l/16) + m (m = 0..3): the same
// slot assignment on both operands, so four consecutive k come from one 16-byte
// load where k is the contiguous index.
__device__ __forceinline__ floatx4 mfma4(floatx4 acc, float a, float b) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(floatx4 acc, floatx4 a, floatx4 b) {
    acc = mfma4(acc, a[0], b[0]);
    acc = mfma4(acc, a[1], b[1]);
    acc = mfma4(acc, a[2], b[2]);
    return mfma4(acc, a[3], b[3]);
}
__device__ __forceinline__ floatx4 lds4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
// Four consecutive rows of one column of an LDS matrix with row stride ld.
__device__ __forceinline__ floatx4 col4(const float* p, int ld) {
    return floatx4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}
// Sum over the 16 lanes holding one accumulator row (one DPP row): rotations by 8
// and 4 within the row, then the swaps inside each quad.  Every lane of the row
// ends with the sum (in a lane-dependent order).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_f<0x128>(x);       // row_ror:8
    x += dpp_f<0x124>(x);       // row_ror:4
    x += dpp_f<0x4E>(x);        // quad_perm [2, 3, 0, 1]
    return x + dpp_f<0xB1>(x);  // quad_perm [1, 0, 3, 2]
}
// Sum over the four lanes holding one accumulator column.
__device__ __forceinline__ float col_sum4(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}
// 16 bytes of T as fp32 (8 values for bf16, 4 for fp32).
template <typename T> struct Unpack16;
template <> struct Unpack16<bf16> {
    static constexpr int N = 8;
    __device__ static __forceinline__ void run(u32x4 x, float* o) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(x[i] << 16);
            o[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
        }
    }
};
template <> struct Unpack16<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ void run(u32x4 x, float* o) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(x[i]);
    }
};

// ================================================================ reverse chain
// One workgroup of 256 threads (4 waves) per (sequence, head, slice of 32 value
// columns), walking the chunks from last to first.  The slice of dS (DK x 32)
// stays in MFMA accumulators, wave w owning the 16-channel blocks w, w + 4, ...
// The earlier chunk's operands are loaded into registers while a chunk computes.
template <typename T, int DK, int DV, int C>
struct BwdChainCfg {
    static constexpr int DVS = 32, NSL = DV / DVS, NB = C / 16, NKB = DK / 16, KPW = NKB / 4;
    static constexpr int LKB = C + 4, LP = C + 4, LWK = DK + 4, LJ = DVS + 4;
    static constexpr int F_KB = 0;                                          // sKb [DK][C]: Kb^T
    static constexpr int F_P = F_KB + DK * LKB;                             // sP  [C][C]
    static constexpr int F_WK = F_P + C * LP;                               // sWk [C][DK]
    static constexpr int F_QT = F_WK + C * LWK;                             // sQt [C][DK]
    static constexpr int F_DO = F_QT + C * LWK;                             // sdO [C][DVS]
    static constexpr int F_S = F_DO + C * LJ;                               // sS  [DK][DVS]: dS'
    static constexpr int F_DW = F_S + DK * LJ;                              // sdW [C][DVS]
    static constexpr int F_G = F_DW + C * LJ;                               // sGam [DK]
    static constexpr int FLOATS = F_G + DK;
    static constexpr int EPU = 16 / (int)sizeof(T);                         // elements per 16 bytes
    static constexpr int U_KB = DK * C / EPU, U_P = C * C / EPU, U_DO = C * DVS / 4;
    static constexpr int PKB = (U_KB + 255) / 256, PP = (U_P + 255) / 256, PDO = (U_DO + 255) / 256;
    static constexpr bool FITS = size_t(FLOATS) * 4 <= LDS_LIMIT && NKB % 4 == 0;
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256, 1) void chunk_bwd_chain_kernel(
    const T* __restrict__ ws_qt, const T* __restrict__ ws_wk, const T* __restrict__ ws_kb,
    const T* __restrict__ ws_p, const float* __restrict__ ws_gam, const float* __restrict__ dO,
    const float* __restrict__ dST, float* __restrict__ dS0, float* __restrict__ ck_dS,
    float* __restrict__ ck_dW, UnitMap um) {
    typedef BwdChainCfg<T, DK, DV, C> Cfg;
    constexpr int DVS = Cfg::DVS, NSL = Cfg::NSL, NB = Cfg::NB, KPW = Cfg::KPW, EPU = Cfg::EPU;
    constexpr int LKB = Cfg::LKB, LP = Cfg::LP, LWK = Cfg::LWK, LJ = Cfg::LJ;
    constexpr int PKB = Cfg::PKB, PP = Cfg::PP, PDO = Cfg::PDO;
    __shared__ __attribute__((aligned(16))) float smem[Cfg::FLOATS];
    float* sKb = smem + Cfg::F_KB;
    float* sP = smem + Cfg::F_P;
    float* sWk = smem + Cfg::F_WK;
    float* sQt = smem + Cfg::F_QT;
    float* sdO = smem + Cfg::F_DO;
    float* sS = smem + Cfg::F_S;
    float* sdW = smem + Cfg::F_DW;
    float* sGam = smem + Cfg::F_G;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, kg = lane >> 4;
    // the slices of one head share an XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so the chunk operands they all read come from one L2
    long bh;
    int sl;
    {
        const long nwg = (long)gridDim.x, id = blockIdx.x;
        if (nwg % 8 == 0) {
            const long o = (id % 8) * (nwg / 8) + id / 8;
            bh = o / NSL;
            sl = (int)(o % NSL);
        } else {
            bh = id / NSL;
            sl = (int)(id % NSL);
        }
    }
    const int j0 = sl * DVS;
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int NC = sr.nchunks;

    floatx4 ds[KPW][2];
#pragma unroll
    for (int p = 0; p < KPW; ++p)
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * (wave + 4 * p) + 4 * kg + e;
                ds[p][J][e] = dST ? dST[(bh * DK + c) * (long)DV + j0 + 16 * J + lr] : 0.f;
            }

    u32x4 rKb[PKB], rWk[PKB], rQt[PKB], rP[PP];
    floatx4 rdO[PDO];
    float rG = 0.f;
#define KDA_BWD_FETCH(N)                                                                          \
    {                                                                                             \
        const long un = unit_id(um, sq, h, (N), sr.chunk0);                                      \
        const u32x4* gkb = reinterpret_cast<const u32x4*>(ws_kb + un * (long)DK * C);             \
        const u32x4* gwk = reinterpret_cast<const u32x4*>(ws_wk + un * (long)C * DK);             \
        const u32x4* gqt = reinterpret_cast<const u32x4*>(ws_qt + un * (long)C * DK);             \
        const u32x4* gp = reinterpret_cast<const u32x4*>(ws_p + un * (long)C * C);                \
        _Pragma("unroll") for (int x = 0; x < PKB; ++x) {                                         \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_KB % 256 == 0 || u < Cfg::U_KB) {                                          \
                rKb[x] = gkb[u];                                                                  \
                rWk[x] = gwk[u];                                                                  \
                rQt[x] = gqt[u];                                                                  \
            }                                                                                     \
        }                                                                                         \
        _Pragma("unroll") for (int x = 0; x < PP; ++x) {                                          \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_P % 256 == 0 || u < Cfg::U_P) rP[x] = gp[u];                               \
        }                                                                                         \
        const long t0 = sr.tok_begin + (long)(N) * C;                                             \
        _Pragma("unroll") for (int x = 0; x < PDO; ++x) {                                         \
            const int u = tid + 256 * x, r = u / (DVS / 4), q4 = u % (DVS / 4);                   \
            if (Cfg::U_DO % 256 == 0 || u < Cfg::U_DO)                                            \
                rdO[x] = t0 + r < sr.tok_end                                                      \
                             ? *reinterpret_cast<const floatx4*>(dO + ((t0 + r) * H + h) * DV + j0 + 4 * q4) \
                             : zero4();                                                           \
        }                                                                                         \
        if (tid < DK) rG = ws_gam[un * DK + tid];                                                 \
    }
#define KDA_BWD_STORE()                                                                           \
    {                                                                                             \
        _Pragma("unroll") for (int x = 0; x < PKB; ++x) {                                         \
            const int u = tid + 256 * x, e0 = u * EPU;                                            \
            if (Cfg::U_KB % 256 == 0 || u < Cfg::U_KB) {                                          \
                float f[EPU];                                                                     \
                Unpack16<T>::run(rKb[x], f);                                                      \
                _Pragma("unroll") for (int i = 0; i < EPU; i += 4)                                \
                    *reinterpret_cast<floatx4*>(sKb + (e0 / C) * LKB + e0 % C + i) =              \
                        floatx4{f[i], f[i + 1], f[i + 2], f[i + 3]};                              \
                Unpack16<T>::run(rWk[x], f);                                                      \
                _Pragma("unroll") for (int i = 0; i < EPU; i += 4)                                \
                    *reinterpret_cast<floatx4*>(sWk + (e0 / DK) * LWK + e0 % DK + i) =            \
                        floatx4{-f[i], -f[i + 1], -f[i + 2], -f[i + 3]};                          \
                Unpack16<T>::run(rQt[x], f);                                                      \
                _Pragma("unroll") for (int i = 0; i < EPU; i += 4)                                \
                    *reinterpret_cast<floatx4*>(sQt + (e0 / DK) * LWK + e0 % DK + i) =            \
                        floatx4{f[i], f[i + 1], f[i + 2], f[i + 3]};                              \
            }                                                                                     \
        }                                                                                         \
        _Pragma("unroll") for (int x = 0; x < PP; ++x) {                                          \
            const int u = tid + 256 * x, e0 = u * EPU;                                            \
            if (Cfg::U_P % 256 == 0 || u < Cfg::U_P) {                                            \
                float f[EPU];                                                                     \
                Unpack16<T>::run(rP[x], f);                                                       \
                _Pragma("unroll") for (int i = 0; i < EPU; i += 4)                                \
                    *reinterpret_cast<floatx4*>(sP + (e0 / C) * LP + e0 % C + i) =                \
                        floatx4{f[i], f[i + 1], f[i + 2], f[i + 3]};                              \
            }                                                                                     \
        }                                                                                         \
        _Pragma("unroll") for (int x = 0; x < PDO; ++x) {                                         \
            const int u = tid + 256 * x, r = u / (DVS / 4), q4 = u % (DVS / 4);                   \
            if (Cfg::U_DO % 256 == 0 || u < Cfg::U_DO)                                            \
                *reinterpret_cast<floatx4*>(sdO + r * LJ + 4 * q4) = rdO[x];                      \
        }                                                                                         \
        if (tid < DK) sGam[tid] = rG;                                                             \
    }

    if (NC > 0) KDA_BWD_FETCH(NC - 1);
    for (int n = NC - 1; n >= 0; --n) {
        const long unit = unit_id(um, sq, h, n, sr.chunk0);
        __syncthreads();                                    // the later chunk's readers are done
        KDA_BWD_STORE();
        // dS', the cotangent of this chunk's end state: to LDS and to its checkpoint
        float* cds = ck_dS + unit * (long)DK * DV;
#pragma unroll
        for (int p = 0; p < KPW; ++p)
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * (wave + 4 * p) + 4 * kg + e, j = 16 * J + lr;
                    sS[c * LJ + j] = ds[p][J][e];
                    cds[c * (long)DV + j0 + j] = ds[p][J][e];
                }
        if (n > 0) KDA_BWD_FETCH(n - 1);
        __syncthreads();

        // dW = Kb dS' + P^T dO: output tiles (R, J), wave w taking w, w + 4, ...
        float* cdw = ck_dW + unit * (long)C * DV;
        for (int t = wave; t < 2 * NB; t += 4) {
            const int R = t >> 1, J = t & 1;
            floatx4 acc = zero4();
#pragma unroll 4
            for (int c0 = 0; c0 < DK; c0 += 16)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int c = c0 + 4 * kg + m;
                    acc = mfma4(acc, sKb[c * LKB + 16 * R + lr], sS[c * LJ + 16 * J + lr]);
                }
            for (int i0 = 16 * R; i0 < C; i0 += 16)             // P[i][r] = 0 for i < r
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = i0 + 4 * kg + m;
                    acc = mfma4(acc, sP[i * LP + 16 * R + lr], sdO[i * LJ + 16 * J + lr]);
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e, j = 16 * J + lr;
                sdW[r * LJ + j] = acc[e];
                cdw[r * (long)DV + j0 + j] = acc[e];
            }
        }
        __syncthreads();

        // dS = Diag(gam) dS' - Wk^T dW + Qt^T dO  (sWk holds -Wk)
#pragma unroll
        for (int p = 0; p < KPW; ++p) {
            const int cb = 16 * (wave + 4 * p);
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                floatx4 acc = ds[p][J];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= sGam[cb + 4 * kg + e];
#pragma unroll 2
                for (int r0 = 0; r0 < C; r0 += 16)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int r = r0 + 4 * kg + m;
                        acc = mfma4(acc, sQt[r * LWK + cb + lr], sdO[r * LJ + 16 * J + lr]);
                        acc = mfma4(acc, sWk[r * LWK + cb + lr], sdW[r * LJ + 16 * J + lr]);
                    }
                ds[p][J] = acc;
            }
        }
    }
#undef KDA_BWD_FETCH
#undef KDA_BWD_STORE
    if (dS0) {
#pragma unroll
        for (int p = 0; p < KPW; ++p)
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * (wave + 4 * p) + 4 * kg + e;
                    dS0[(bh * DK + c) * (long)DV + j0 + 16 * J + lr] = ds[p][J][e];
                }
    }
}

// ================================================================ reverse chain, bf16 inputs
// The same recurrence for bf16 inputs, on bf16 MFMA (16x16x32).  The chunk operands
// Kb^T, P, Wk and Qt are bf16 in the workspace, so exact as MFMA operands; the fp32
// ones (dS', dO, dW) are split into bf16 hi + lo parts (hi = bf16(x), lo =
// bf16(x - hi), about 16 significant bits) and each product takes two MFMAs.
// Every product here contracts over the index that is not the contiguous one of
// the forward's layout, so those operands are read with the LDS transpose read
// (ds_read_b64_tr_b16) and every array is staged as it lies in memory.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// One operand fragment of v_mfma_f32_16x16x32_bf16 (8 consecutive k of row or
// column mn0 + l%16 in lane l, k = k0 + 8(l/16) + 0..7) from X[k][mn] stored
// row-major with mn contiguous.  Within each group of 16 lanes the transpose read
// hands lane d, element e the element d%4 of lane 4e + d/4, so lane s points at
// X[k0 + 8g + s/4][mn0 + 4(s%4)] (and four rows further for elements 4..7).
__device__ __forceinline__ bf16x8 frag_tr(const bf16* X, int ld, int k0, int mn0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const bf16* p0 = X + (k0 + 8 * g + (s >> 2)) * ld + mn0 + 4 * (s & 3);
    const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)const_cast<bf16*>(p0));
    const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)const_cast<bf16*>(p0 + 4 * ld));
    const short8v c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, c);
}
// The same fragment from Z[mn][k] stored row-major with k contiguous: one 16-byte read.
__device__ __forceinline__ bf16x8 frag_n(const bf16* Z, int ld, int k0, int mn0, int lane) {
    return *reinterpret_cast<const bf16x8*>(Z + (mn0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
__device__ __forceinline__ floatx4 mfma32(floatx4 acc, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split4(floatx4 x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (bf16)x[e];
        lo[e] = (bf16)(x[e] - (float)hi[e]);
    }
}

template <int DK, int DV, int C>
struct BwdChainHCfg {
    static constexpr int DVS = 32, NSL = DV / DVS, NB = C / 16, KPW = DK / 64;
    // row lengths in bf16: the four rows one transpose read touches fall into
    // separate bank windows; the 16-byte reads stay aligned
    static constexpr int LKB = C + 8;                 // Kb^T [DK][C]
    static constexpr int LP = C + 8;                  // P    [C][C]
    static constexpr int LW = DK + 16;                // Wk (negated), Qt  [C][DK]
    static constexpr int LO = DVS + 16;               // dO hi, lo         [C][DVS]
    static constexpr int LS = DK + 8;                 // dS'^T hi, lo      [DVS][DK]
    static constexpr int LD = C + 8;                  // dW^T hi, lo       [DVS][C]
    static constexpr size_t O_KB = 0;
    static constexpr size_t O_P = O_KB + size_t(DK) * LKB * 2;
    static constexpr size_t O_WK = O_P + size_t(C) * LP * 2;
    static constexpr size_t O_QT = O_WK + size_t(C) * LW * 2;
    static constexpr size_t O_OH = O_QT + size_t(C) * LW * 2;
    static constexpr size_t O_OL = O_OH + size_t(C) * LO * 2;
    static constexpr size_t O_SH = O_OL + size_t(C) * LO * 2;
    static constexpr size_t O_SL = O_SH + size_t(DVS) * LS * 2;
    static constexpr size_t O_WH = O_SL + size_t(DVS) * LS * 2;
    static constexpr size_t O_WL = O_WH + size_t(DVS) * LD * 2;
    static constexpr size_t O_G = O_WL + size_t(DVS) * LD * 2;
    static constexpr size_t BYTES = O_G + size_t(DK) * 4;
    static constexpr int U_KB = DK * C / 8, U_P = C * C / 8, U_DO = C * DVS / 4;   // 16-byte units
    static constexpr int PKB = (U_KB + 255) / 256, PP = (U_P + 255) / 256, PDO = (U_DO + 255) / 256;
    static constexpr bool FITS = (C == 32 || C == 64) && BYTES <= LDS_LIMIT && DK % 64 == 0 && DV % DVS == 0;
};

template <int DK, int DV, int C>
__global__ __launch_bounds__(256, 1) void chunk_bwd_chain_h_kernel(
    const bf16* __restrict__ ws_qt, const bf16* __restrict__ ws_wk, const bf16* __restrict__ ws_kb,
    const bf16* __restrict__ ws_p, const float* __restrict__ ws_gam, const float* __restrict__ dO,
    const float* __restrict__ dST, float* __restrict__ dS0, float* __restrict__ ck_dS,
    float* __restrict__ ck_dW, UnitMap um) {
    typedef BwdChainHCfg<DK, DV, C> Cfg;
    constexpr int DVS = Cfg::DVS, NSL = Cfg::NSL, NB = Cfg::NB, KPW = Cfg::KPW;
    constexpr int LKB = Cfg::LKB, LP = Cfg::LP, LW = Cfg::LW, LO = Cfg::LO, LS = Cfg::LS, LD = Cfg::LD;
    constexpr int PKB = Cfg::PKB, PP = Cfg::PP, PDO = Cfg::PDO;
    // dk = 128, C = 64 (bf16): the forward stages wrote Kb^T, Wk, Qt and P in MFMA
    // fragment order (16-byte pieces of 8 consecutive elements of a row; the two
    // blocks of P above the diagonal not written, and never read here)
    constexpr bool FRAG = DK == 128 && C == 64;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
    bf16* sKb = reinterpret_cast<bf16*>(smem + Cfg::O_KB);
    bf16* sP = reinterpret_cast<bf16*>(smem + Cfg::O_P);
    bf16* sWk = reinterpret_cast<bf16*>(smem + Cfg::O_WK);
    bf16* sQt = reinterpret_cast<bf16*>(smem + Cfg::O_QT);
    bf16* sOh = reinterpret_cast<bf16*>(smem + Cfg::O_OH);
    bf16* sOl = reinterpret_cast<bf16*>(smem + Cfg::O_OL);
    bf16* sSh = reinterpret_cast<bf16*>(smem + Cfg::O_SH);
    bf16* sSl = reinterpret_cast<bf16*>(smem + Cfg::O_SL);
    bf16* sWh = reinterpret_cast<bf16*>(smem + Cfg::O_WH);
    bf16* sWl = reinterpret_cast<bf16*>(smem + Cfg::O_WL);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::O_G);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, kg = lane >> 4;
    // the slices of one head share an XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so the chunk operands they all read come from one L2
    long bh;
    int sl;
    {
        const long nwg = (long)gridDim.x, id = blockIdx.x;
        if (nwg % 8 == 0) {
            const long o = (id % 8) * (nwg / 8) + id / 8;
            bh = o / NSL;
            sl = (int)(o % NSL);
        } else {
            bh = id / NSL;
            sl = (int)(id % NSL);
        }
    }
    const int j0 = sl * DVS;
    const int H = um.H, sq = (int)(bh / H), h = (int)(bh % H);
    const SeqRange sr = seq_range(um, sq);
    const int NC = sr.nchunks;

    // dS slice in accumulators: rows 16(wave + 4p) + 4(l/16) + e, columns 16J + l%16
    floatx4 ds[KPW][2];
#pragma unroll
    for (int p = 0; p < KPW; ++p)
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * (wave + 4 * p) + 4 * kg + e;
                ds[p][J][e] = dST ? dST[(bh * DK + c) * (long)DV + j0 + 16 * J + lr] : 0.f;
            }

    // the next chunk's operands, in registers while a chunk computes
    u32x4 rKb[PKB], rWk[PKB], rQt[PKB], rP[PP];
    floatx4 rdO[PDO];
    float rG = 0.f;
#define KDA_BWDH_FETCH(N)                                                                         \
    {                                                                                             \
        const long un = unit_id(um, sq, h, (N), sr.chunk0);                                      \
        const u32x4* gkb = reinterpret_cast<const u32x4*>(ws_kb + un * (long)DK * C);             \
        const u32x4* gwk = reinterpret_cast<const u32x4*>(ws_wk + un * (long)C * DK);             \
        const u32x4* gqt = reinterpret_cast<const u32x4*>(ws_qt + un * (long)C * DK);             \
        const u32x4* gp = reinterpret_cast<const u32x4*>(ws_p + un * (long)C * C);                \
        _Pragma("unroll") for (int x = 0; x < PKB; ++x) {                                         \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_KB % 256 == 0 || u < Cfg::U_KB) {                                          \
                rKb[x] = gkb[u];                                                                  \
                rWk[x] = gwk[u];                                                                  \
                rQt[x] = gqt[u];                                                                  \
            }                                                                                     \
        }                                                                                         \
        _Pragma("unroll") for (int x = 0; x < PP; ++x) {                                          \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_P % 256 == 0 || u < Cfg::U_P) rP[x] = gp[u];                               \
        }                                                                                         \
        const long t0 = sr.tok_begin + (long)(N) * C;                                             \
        _Pragma("unroll") for (int x = 0; x < PDO; ++x) {                                         \
            const int u = tid + 256 * x, r = u / (DVS / 4), q4 = u % (DVS / 4);                   \
            const long tr = t0 + r < sr.tok_end ? t0 + r : t0;                                    \
            if (Cfg::U_DO % 256 == 0 || u < Cfg::U_DO)                                            \
                rdO[x] = *reinterpret_cast<const floatx4*>(dO + (tr * H + h) * DV + j0 + 4 * q4); \
        }                                                                                         \
        if (tid < DK) rG = ws_gam[un * DK + tid];                                                 \
    }
    // to LDS as they lie in memory (Wk negated; dO split, rows past the end zero)
#define KDA_BWDH_STORE(N)                                                                         \
    {                                                                                             \
        _Pragma("unroll") for (int x = 0; x < PKB; ++x) {                                         \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_KB % 256 == 0 || u < Cfg::U_KB) {                                          \
                const int e0 = 8 * u, lf = u & 63;                                                \
                const int okb = FRAG ? (16 * (u >> 7) + (lf & 15)) * LKB + 32 * ((u >> 6) & 1) + 8 * (lf >> 4) \
                                     : (e0 / C) * LKB + e0 % C;                                   \
                const int ow = FRAG ? (16 * (u >> 8) + (lf & 15)) * LW + 32 * ((u >> 6) & 3) + 8 * (lf >> 4) \
                                    : (e0 / DK) * LW + e0 % DK;                                   \
                *reinterpret_cast<u32x4*>(sKb + okb) = rKb[x];                                    \
                const u32x4 nw = {rWk[x][0] ^ 0x80008000u, rWk[x][1] ^ 0x80008000u,               \
                                  rWk[x][2] ^ 0x80008000u, rWk[x][3] ^ 0x80008000u};              \
                *reinterpret_cast<u32x4*>(sWk + ow) = nw;                                         \
                *reinterpret_cast<u32x4*>(sQt + ow) = rQt[x];                                     \
            }                                                                                     \
        }                                                                                         \
        _Pragma("unroll") for (int x = 0; x < PP; ++x) {                                          \
            const int u = tid + 256 * x;                                                          \
            if (Cfg::U_P % 256 == 0 || u < Cfg::U_P) {                                            \
                const int e0 = 8 * u, lf = u & 63;                                                \
                const int op = FRAG ? (16 * (u >> 7) + (lf & 15)) * LP + 32 * ((u >> 6) & 1) + 8 * (lf >> 4) \
                                    : (e0 / C) * LP + e0 % C;                                     \
                *reinterpret_cast<u32x4*>(sP + op) = rP[x];                                       \
            }                                                                                     \
        }                                                                                         \
        const long t0 = sr.tok_begin + (long)(N) * C;                                             \
        _Pragma("unroll") for (int x = 0; x < PDO; ++x) {                                         \
            const int u = tid + 256 * x, r = u / (DVS / 4), q4 = u % (DVS / 4);                   \
            if (Cfg::U_DO % 256 == 0 || u < Cfg::U_DO) {                                          \
                const floatx4 o4 = t0 + r < sr.tok_end ? rdO[x] : zero4();                        \
                bf16x4 hi, lo;                                                                    \
                split4(o4, hi, lo);                                                               \
                *reinterpret_cast<bf16x4*>(sOh + r * LO + 4 * q4) = hi;                           \
                *reinterpret_cast<bf16x4*>(sOl + r * LO + 4 * q4) = lo;                           \
            }                                                                                     \
        }                                                                                         \
        if (tid < DK) sGam[tid] = rG;                                                             \
    }

    if (NC > 0) KDA_BWDH_FETCH(NC - 1);
    for (int n = NC - 1; n >= 0; --n) {
        const long unit = unit_id(um, sq, h, n, sr.chunk0);
        __syncthreads();                                    // the later chunk's readers are done
        KDA_BWDH_STORE(n);
        // dS', the cotangent of this chunk's end state: split to LDS (transposed
        // rows, four channels a lane) and to its checkpoint
        float* cds = ck_dS + unit * (long)DK * DV;
#pragma unroll
        for (int p = 0; p < KPW; ++p)
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                const int c0 = 16 * (wave + 4 * p) + 4 * kg, j = 16 * J + lr;
                bf16x4 hi, lo;
                split4(ds[p][J], hi, lo);
                *reinterpret_cast<bf16x4*>(sSh + j * LS + c0) = hi;
                *reinterpret_cast<bf16x4*>(sSl + j * LS + c0) = lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) cds[(c0 + e) * (long)DV + j0 + j] = ds[p][J][e];
            }
        if (n > 0) KDA_BWDH_FETCH(n - 1);
        __syncthreads();

        // dW = Kb dS' + P^T dO: output tiles (R, J), wave w taking w, w + 4, ...
        float* cdw = ck_dW + unit * (long)C * DV;
#pragma unroll
        for (int t = wave; t < 2 * NB; t += 4) {
            const int R = t >> 1, J = t & 1;
            floatx4 acc = zero4();
#pragma unroll
            for (int c0 = 0; c0 < DK; c0 += 32) {
                const bf16x8 a = frag_tr(sKb, LKB, c0, 16 * R, lane);          // Kb[r][c] = Kb^T[c][r]
                acc = mfma32(acc, a, frag_n(sSh, LS, c0, 16 * J, lane));
                acc = mfma32(acc, a, frag_n(sSl, LS, c0, 16 * J, lane));
            }
#pragma unroll
            for (int i0 = 0; i0 < C; i0 += 32) {
                if (i0 + 32 <= 16 * R) continue;                                // P[i][r] = 0 for i < r
                const bf16x8 a = frag_tr(sP, LP, i0, 16 * R, lane);            // P^T[r][i] = P[i][r]
                acc = mfma32(acc, a, frag_tr(sOh, LO, i0, 16 * J, lane));
                acc = mfma32(acc, a, frag_tr(sOl, LO, i0, 16 * J, lane));
            }
            bf16x4 hi, lo;
            split4(acc, hi, lo);
            *reinterpret_cast<bf16x4*>(sWh + (16 * J + lr) * LD + 16 * R + 4 * kg) = hi;
            *reinterpret_cast<bf16x4*>(sWl + (16 * J + lr) * LD + 16 * R + 4 * kg) = lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) cdw[(16 * R + 4 * kg + e) * (long)DV + j0 + 16 * J + lr] = acc[e];
        }
        __syncthreads();

        // dS = Diag(gam) dS' - Wk^T dW + Qt^T dO  (sWk holds -Wk)
#pragma unroll
        for (int p = 0; p < KPW; ++p) {
            const int cb = 16 * (wave + 4 * p);
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                floatx4 acc = ds[p][J];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= sGam[cb + 4 * kg + e];
#pragma unroll
                for (int r0 = 0; r0 < C; r0 += 32) {
                    const bf16x8 aq = frag_tr(sQt, LW, r0, cb, lane);            // Qt^T[c][r]
                    acc = mfma32(acc, aq, frag_tr(sOh, LO, r0, 16 * J, lane));
                    acc = mfma32(acc, aq, frag_tr(sOl, LO, r0, 16 * J, lane));
                    const bf16x8 aw = frag_tr(sWk, LW, r0, cb, lane);            // -Wk^T[c][r]
                    acc = mfma32(acc, aw, frag_n(sWh, LD, r0, 16 * J, lane));
                    acc = mfma32(acc, aw, frag_n(sWl, LD, r0, 16 * J, lane));
                }
                ds[p][J] = acc;
            }
        }
    }
#undef KDA_BWDH_FETCH
#undef KDA_BWDH_STORE
    if (dS0) {
#pragma unroll
        for (int p = 0; p < KPW; ++p)
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * (wave + 4 * p) + 4 * kg + e;
                    dS0[(bh * DK + c) * (long)DV + j0 + 16 * J + lr] = ds[p][J][e];
                }
    }
}

// ================================================================ per-chunk gradients
// One workgroup per chunk unit with one wave per 16-channel block (8 waves for
// dk = 128, two to a SIMD).  Wave w owns channels 16w .. 16w + 15 from start to
// end: its elements are rows 16R + 4(l/16) + e, channel 16w + l%16 (the MFMA
// accumulator layout), and dQt, dKb, T^T dWk, the raw k and q, the prefix sums G
// of the log-gate and the decayed operands of the last phase stay in its
// registers, so the last phase (decays, pairwise decays, the prefix-sum adjoint)
// runs without workgroup barriers or LDS of its own.  The C x C products are split
// by column block (wave w < C/16: block w) and go through LDS.
//   phase 1  the products over the value channels (dQt, dWk, dKb, dgam, dP,
//            dW V^T) on bf16 MFMA with fp32 operands split into bf16 hi + lo:
//            the rows of dO, W and dW are staged in LDS once per workgroup, each
//            wave's S and dS' blocks come straight into registers
//   then     dV = Diag(beta) T^T dW;  G and Kt = e^G K;  dT, T^T dWk;  dM, dA;
//            the per-wave last phase;  dbeta from per-wave partial sums
template <int DK, int DV, int C>
struct BwdIntraCfg {
    static constexpr int NB = C / 16, NKB = DK / 16, NVB = DV / 16;
    static constexpr int NW = NKB, NT = 64 * NW;                            // one wave per channel block
    static constexpr int LC = C + 4, LK = DK + 4;
    static constexpr int LS1 = 40;                                          // staged bf16 row of phase 1
    static constexpr int F_T = 0, F_DP = C * LC, F_DA = 2 * C * LC;
    static constexpr int F_X = 3 * C * LC;                                  // shared by phases 1, 3, 4
    static constexpr int X1 = 2 * 3 * 2 * C * LS1 / 2;                      // phase 1: [2][3][hi, lo][C][LS1] bf16
    static constexpr int X3 = 2 * C * LK;                                   // dWk, Kt
    static constexpr int X4 = C * LC;                                       // X = T^T dT
    static constexpr int XN = X1 > X3 ? (X1 > X4 ? X1 : X4) : (X3 > X4 ? X3 : X4);
    static constexpr int F_BETA = F_X + XN;
    static constexpr int F_DB1 = F_BETA + C;                                // [C]
    static constexpr int F_DB2 = F_DB1 + C;                                 // [NW][C]
    static constexpr int F_DB3 = F_DB2 + NW * C;                            // [NW][C]
    static constexpr int F_HD = F_DB3 + NW * C;                             // [NW][C] per-head dg partials
    static constexpr int FLOATS = F_HD + NW * C;
    static constexpr bool FITS = size_t(FLOATS) * 4 <= LDS_LIMIT && NB <= NW;
};

// Eight consecutive values of T as loaded, and their bf16 hi + lo parts (bf16
// inputs are exact: lo = 0, and the product with them takes one MFMA fewer).
template <typename T> struct Raw8;
template <> struct Raw8<float> {
    typedef floatx4 type[2];
    static constexpr bool EXACT = false;
};
template <> struct Raw8<bf16> {
    typedef bf16x8 type[1];
    static constexpr bool EXACT = true;
};
// x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) for 8 fp32 values
__device__ __forceinline__ void split8(const floatx4 (&x)[2], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float v = x[m >> 2][m & 3];
        hi[m] = (bf16)v;
        lo[m] = (bf16)(v - (float)hi[m]);
    }
}
// a . b with a = ah + al, b = bh + bl in fp32 accumulation, the al.bl term dropped
__device__ __forceinline__ floatx4 mfma_x3(floatx4 acc, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// Row block of lower tile t, the tiles (R, I <= R) taken in row order
constexpr int lower_row(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }

// One 32-deep k step of phase 1, the operands a wave reads alone: its channel
// block of S and dS', and row block I of W and V (8 values a lane)
template <typename T>
struct BwdFragB {
    floatx4 s[2], ds[2], wi[2];
    typename Raw8<T>::type v;
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(DK * 4, 1) void chunk_bwd_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ dO,
    const float* __restrict__ ck_state, const float* __restrict__ ck_dS, const float* __restrict__ ck_w,
    const float* __restrict__ ck_dW, const float* __restrict__ ck_t, const float* __restrict__ ck_a,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta, UnitMap um, int gate) {
    typedef BwdIntraCfg<DK, DV, C> Cfg;
    constexpr int NB = Cfg::NB, NVB = Cfg::NVB, NW = Cfg::NW, NT = Cfg::NT;
    constexpr int LC = Cfg::LC, LK = Cfg::LK;
    static_assert(NT == DK * 4, "launch bounds");
    __shared__ __attribute__((aligned(16))) float smem[Cfg::FLOATS];
    float* sT = smem + Cfg::F_T;            // T [C][C]
    float* sdP = smem + Cfg::F_DP;          // dP (lower)
    float* sdA = smem + Cfg::F_DA;          // dW V^T -> dT -> dA (lower)
    float* sXa = smem + Cfg::F_X;
    float* sBeta = smem + Cfg::F_BETA;
    float* sDb1 = smem + Cfg::F_DB1;
    float* sDb2 = smem + Cfg::F_DB2;
    float* sDb3 = smem + Cfg::F_DB3;
    float* sHd = smem + Cfg::F_HD;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, kg = lane >> 4;
    const long unit = blockIdx.x;
    UnitPos up;
    if (!unit_pos(um, unit, up)) return;
    const int H = um.H, h = up.h, cnt = up.count;
    const long tok0 = up.tok0;
    auto grow = [&](int t) -> long { return (tok0 + t) * H + h; };
    auto valid = [&](int t) -> bool { return t < cnt; };
    // a row past the sequence end reads row 0 (and the value is then dropped), so
    // that loads need no branch and can all be in flight together
    auto crow = [&](int t) -> long { return grow(t < cnt ? t : 0); };
    const bool tri = wave < NB;             // owns the C x C column block I = wave
    const int cw = 16 * wave + lr;          // this lane's channel

    const float* S = ck_state + unit * (long)DK * DV;      // start state [DK][DV]
    const float* dSn = ck_dS + unit * (long)DK * DV;       // cotangent of the end state
    const float* W = ck_w + unit * (long)C * DV;
    const float* dW = ck_dW + unit * (long)C * DV;

    // ---- phase 0: T and beta to LDS, the dbeta partials cleared
    {
        constexpr int NTT = (C * C + NT - 1) / NT;
        float tv[NTT];
#pragma unroll
        for (int x = 0; x < NTT; ++x) {                             // 16x16 blocks above the diagonal: 0
            const int u = tid + NT * x, uu = u < C * C ? u : 0;
            tv[x] = ((uu % C) >> 4) > ((uu / C) >> 4) ? 0.f : ck_t[unit * (long)C * C + uu];
        }
        const float bt = tid < C ? beta[crow(tid)] : 0.f;
#pragma unroll
        for (int x = 0; x < NTT; ++x) {
            const int u = tid + NT * x;
            if (u < C * C) sT[(u / C) * LC + u % C] = tv[x];
        }
        if (tid < C) sBeta[tid] = valid(tid) ? bt : 0.f;
        for (int u = tid; u < NW * C; u += NT) sDb3[u] = 0.f;
    }
    __syncthreads();

    // ---- phase 1: dQt = dO S^T, dWk = -dW S^T, dKb = W dS'^T, dgam, dP = dO W^T,
    // dW V^T, contracted over the value channels 32 at a time
    float* sWk = sXa;                       // dWk [C][DK]  (phase 3 operand)
    float* sKt = sXa + C * LK;              // Kt = e^G K [C][DK]
    floatx4 aQ[NB], aKb[NB];                // kept to the end
    float dgam = 0.f;
    // this wave's raw gates and k, loaded while the last products run
    float gr[NB][4], kv[NB][4];
    {
        floatx4 aWk[NB], aP[NB], aV[NB];
#pragma unroll
        for (int R = 0; R < NB; ++R) aQ[R] = aKb[R] = aWk[R] = aP[R] = aV[R] = zero4();

        // k step js covers value channels 32 js .. 32 js + 31; in the MFMA operand
        // layout lane l holds channels 32 js + 8(l/16) .. +7 of its row (every
        // product contracts over the value channels, contiguous in every array).
        // The rows of dO, W and dW feed every wave: each step they are loaded once
        // per workgroup, split into bf16 hi + lo and staged in LDS (two buffers, one
        // barrier a step), loaded two steps ahead.  A wave's own operands (its
        // channel block of S and dS', row block I of W and V) go into registers one
        // step ahead.
        constexpr int NJS = DV / 32, LS1 = Cfg::LS1;
        // thread t takes the float4 pieces (row (t + NT h) / 8, channels 4 (t % 8) ..)
        // of each of dO, W and dW; with C x 8 < NT only the first C x 8 threads do
        constexpr int PPA = (C * 8 + NT - 1) / NT;
        bf16* sStage = reinterpret_cast<bf16*>(sXa);        // [2 buffers][3 arrays][hi, lo][C rows][LS1]
        auto stage_row = [&](int buf, int arr, int hl, int row) {
            return sStage + (((buf * 3 + arr) * 2 + hl) * C + row) * LS1;
        };
        const int ac4 = tid & 7;
        const float* pa[3][PPA];
        bool arow_in[PPA], arow_ok[PPA];
#pragma unroll
        for (int hh = 0; hh < PPA; ++hh) {
            const int row = (tid + NT * hh) >> 3;
            arow_in[hh] = row < C;
            const int rr = arow_in[hh] ? row : 0;
            arow_ok[hh] = valid(rr);
            pa[0][hh] = dO + crow(rr) * DV + 4 * ac4;
            pa[1][hh] = W + rr * DV + 4 * ac4;
            pa[2][hh] = dW + rr * DV + 4 * ac4;
        }
        floatx4 ra[2][3][PPA];
        BwdFragB<T> rb;
        auto load_a = [&](auto SL, int js) __attribute__((always_inline)) {
            constexpr int d = SL;
            const int col = 32 * (js < NJS ? js : NJS - 1);
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int hh = 0; hh < PPA; ++hh) ra[d][a][hh] = *reinterpret_cast<const floatx4*>(pa[a][hh] + col);
        };
        auto stage_a = [&](auto SL, int buf) __attribute__((always_inline)) {
            constexpr int d = SL;
#pragma unroll
            for (int hh = 0; hh < PPA; ++hh) {
                if (!arow_in[hh]) continue;
                const int row = (tid + NT * hh) >> 3;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const floatx4 x = a == 0 && !arow_ok[hh] ? zero4() : ra[d][a][hh];
                    bf16x4 hi, lo;
                    split4(x, hi, lo);
                    *reinterpret_cast<bf16x4*>(stage_row(buf, a, 0, row) + 4 * ac4) = hi;
                    *reinterpret_cast<bf16x4*>(stage_row(buf, a, 1, row) + 4 * ac4) = lo;
                }
            }
        };
        const int iw = 16 * (tri ? wave : 0) + lr;          // row of W, V in the operand of dP, dW V^T
        auto load_b = [&](int js) __attribute__((always_inline)) {
            const int jb = 32 * (js < NJS ? js : NJS - 1) + 8 * kg;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                rb.s[h2] = *reinterpret_cast<const floatx4*>(S + cw * DV + jb + 4 * h2);
                rb.ds[h2] = *reinterpret_cast<const floatx4*>(dSn + cw * DV + jb + 4 * h2);
                rb.wi[h2] = *reinterpret_cast<const floatx4*>(W + iw * DV + jb + 4 * h2);
            }
            if constexpr (Raw8<T>::EXACT) {
                rb.v[0] = *reinterpret_cast<const bf16x8*>(v + crow(iw) * DV + jb);
            } else {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) rb.v[h2] = *reinterpret_cast<const floatx4*>(v + crow(iw) * DV + jb + 4 * h2);
            }
        };
        const bool vrow_ok = valid(iw);
        // one k step: its shared operands in LDS buffer js % 2, its own in rb
        auto step = [&](auto SL, int js) __attribute__((always_inline)) {
            constexpr int d = SL, d1 = 1 - SL;
            __syncthreads();                                // buffer d staged; buffer d1 no longer read
            bf16x8 sh, sl, dsh, dsl, wih, wil, vh, vl;
            split8(rb.s, sh, sl);
            split8(rb.ds, dsh, dsl);
#pragma unroll
            for (int m = 0; m < 8; ++m) dgam += rb.s[m >> 2][m & 3] * rb.ds[m >> 2][m & 3];
            split8(rb.wi, wih, wil);
            if constexpr (Raw8<T>::EXACT) {
                vh = rb.v[0];
            } else {
                split8(rb.v, vh, vl);
            }
            if (!vrow_ok) {
#pragma unroll
                for (int m = 0; m < 8; ++m) { vh[m] = (bf16)0.f; vl[m] = (bf16)0.f; }
            }
            load_b(js + 1);
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                const int o = (16 * R + lr) * LS1 + 8 * kg;
                const bf16x8 oh = *reinterpret_cast<const bf16x8*>(stage_row(d, 0, 0, 0) + o);
                const bf16x8 ol = *reinterpret_cast<const bf16x8*>(stage_row(d, 0, 1, 0) + o);
                const bf16x8 wh = *reinterpret_cast<const bf16x8*>(stage_row(d, 1, 0, 0) + o);
                const bf16x8 wl = *reinterpret_cast<const bf16x8*>(stage_row(d, 1, 1, 0) + o);
                const bf16x8 dwh = *reinterpret_cast<const bf16x8*>(stage_row(d, 2, 0, 0) + o);
                const bf16x8 dwl = *reinterpret_cast<const bf16x8*>(stage_row(d, 2, 1, 0) + o);
                aQ[R] = mfma_x3(aQ[R], oh, ol, sh, sl);
                aWk[R] = mfma_x3(aWk[R], dwh, dwl, sh, sl);
                aKb[R] = mfma_x3(aKb[R], wh, wl, dsh, dsl);
                if (tri && R >= wave) {
                    aP[R] = mfma_x3(aP[R], oh, ol, wih, wil);
                    if constexpr (Raw8<T>::EXACT) {
                        aV[R] = mfma32(mfma32(aV[R], dwl, vh), dwh, vh);
                    } else {
                        aV[R] = mfma_x3(aV[R], dwh, dwl, vh, vl);
                    }
                }
            }
            stage_a(std::integral_constant<int, d1>{}, d1);   // step js + 1, read after the next barrier
            load_a(std::integral_constant<int, d1>{}, js + 3);
        };
        load_a(std::integral_constant<int, 0>{}, 0);
        load_b(0);
        load_a(std::integral_constant<int, 1>{}, 1);
        stage_a(std::integral_constant<int, 0>{}, 0);
        load_a(std::integral_constant<int, 0>{}, 2);
#pragma unroll 1
        for (int js = 0; js < NJS; js += 2) {
            step(std::integral_constant<int, 0>{}, js);
            step(std::integral_constant<int, 1>{}, js + 1);
        }
        // this wave's raw gates and k (for G and Kt after dV, and the last phase)
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                const long o = crow(r) * DK + cw;
                gr[R][e] = gate == GATE_CHANNEL ? g[o] : (gate == GATE_HEAD ? g[crow(r)] : 0.f);
                kv[R][e] = to_f32(k[o]);
            }
        __syncthreads();                                    // the staging area is phase 3's from here

#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int e = 0; e < 4; ++e) sWk[(16 * R + 4 * kg + e) * LK + cw] = -aWk[R][e];
        dgam = col_sum4(dgam);
        if (tri) {
            // column block I = wave of dP and dW V^T (lower part; zero above), and
            // the first dbeta term: (T^T dW V^T)_ii = sum_r T_ri (dW V^T)_ri
            const int i = 16 * wave + lr;
            float db = 0.f;
#pragma unroll
            for (int R = 0; R < NB; ++R)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * R + 4 * kg + e;
                    float pv = 0.f, vv = 0.f;
                    if (R >= wave && i <= r) { pv = aP[R][e]; vv = aV[R][e]; }
                    sdP[r * LC + i] = pv;
                    sdA[r * LC + i] = vv;
                    db += sT[r * LC + i] * vv;
                }
            db = col_sum4(db);
            if (kg == 0) sDb1[i] = db;
        }
    }
    // dV = Diag(beta) T^T dW: output tiles (R, J), wave w taking J = w, w + NW, ...
    for (int J = wave; J < NVB; J += NW) {
        float bcol[NB][4];
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int m = 0; m < 4; ++m) bcol[I][m] = dW[(16 * I + 4 * kg + m) * DV + 16 * J + lr];
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            floatx4 acc = zero4();
#pragma unroll
            for (int I = R; I < NB; ++I)                            // T[i][r] = 0 for i < r
#pragma unroll
                for (int m = 0; m < 4; ++m) acc = mfma4(acc, sT[(16 * I + 4 * kg + m) * LC + 16 * R + lr], bcol[I][m]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                if (valid(r)) __builtin_nontemporal_store(sBeta[r] * acc[e], dv + grow(r) * DV + 16 * J + lr);
            }
        }
    }

    // ---- phase 2: this wave's prefix sums G of the clamped log-gate (rows past
    // the sequence end add nothing), its block boundaries, Kt = e^G K
    //   gs[R] = G before block R, gm[R] = G at the end of block R (= gs[R + 1]), GC = G_C
    float G[NB][4], gs[NB + 1];
    unsigned floored = 0u;                  // the forward floors the log-gate at G_FLOOR: no gradient there
    {
        float run = 0.f;
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            float p4[4], acc = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                floored |= (gr[R][e] < G_FLOOR ? 1u : 0u) << (4 * R + e);
                acc += valid(r) ? clamp_g(gr[R][e]) : 0.f;
                p4[e] = acc;
            }
            // the four row groups of the block: lanes l%16 + 16 j hold group j
            const float t0 = __shfl(acc, lr), t1 = __shfl(acc, lr + 16), t2 = __shfl(acc, lr + 32),
                        t3 = __shfl(acc, lr + 48);
            const float before = (kg > 0 ? t0 : 0.f) + (kg > 1 ? t1 : 0.f) + (kg > 2 ? t2 : 0.f);
            gs[R] = run;
#pragma unroll
            for (int e = 0; e < 4; ++e) G[R][e] = run + before + p4[e];
            run += ((t0 + t1) + t2) + t3;
        }
        gs[NB] = run;
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                if (!valid(r)) kv[R][e] = 0.f;
                sKt[r * LK + cw] = kv[R][e] * __expf(G[R][e]);
            }
    }
    // q of this wave's elements, for the last phase
    float qv[NB][4];
#pragma unroll
    for (int R = 0; R < NB; ++R)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * R + 4 * kg + e;
            const float qx = to_f32(q[crow(r) * DK + cw]);
            qv[R][e] = valid(r) ? qx : 0.f;
        }
    __syncthreads();

    // ---- phase 3: dT = Diag-columns(beta) (dW V^T + dWk Kt^T) on the lower tiles
    // (R, I), tile t (in row order) on wave t % NW; T^T dWk on this wave's channel
    // block, with the second dbeta term, rows of (T^T dWk) Kt
    static_for<NB * (NB + 1) / 2>([&](auto TI) {
        constexpr int t = TI, R = lower_row(t), I = t - R * (R + 1) / 2;
        if (t % NW != wave) return;
        floatx4 acc = zero4();
#pragma unroll 4
        for (int c0 = 0; c0 < DK; c0 += 16)
            acc = mfma16(acc, lds4(sWk + (16 * R + lr) * LK + c0 + 4 * kg), lds4(sKt + (16 * I + lr) * LK + c0 + 4 * kg));
        const int i = 16 * I + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * R + 4 * kg + e;
            if (i <= r) sdA[r * LC + i] = sBeta[i] * (sdA[r * LC + i] + acc[e]);
        }
    });
    floatx4 aTd[NB];                        // T^T dWk, kept to the end
    {
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            floatx4 acc = zero4();
#pragma unroll
            for (int I = R; I < NB; ++I)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = 16 * I + 4 * kg + m;
                    acc = mfma4(acc, sT[i * LC + 16 * R + lr], sWk[i * LK + cw]);
                }
            aTd[R] = acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = row_sum16(acc[e] * sKt[(16 * R + 4 * kg + e) * LK + cw]);
                if (lr == 0) sDb2[wave * C + 16 * R + 4 * kg + e] = x;
            }
        }
    }
    __syncthreads();

    // ---- phase 4: X = T^T dT (lower tiles), then dM = -strict_lower(X T^T),
    // dbeta += rows of dM A (partials by column block), dA = Diag(beta) dM; tile t on
    // wave t % NW
    float* sXm = sXa;
    static_for<NB * (NB + 1) / 2>([&](auto TI) {
        constexpr int t = TI, R = lower_row(t), I = t - R * (R + 1) / 2;
        if (t % NW != wave) return;
        floatx4 acc = zero4();
#pragma unroll
        for (int M = R; M < NB; ++M)                                // T[m][r] = 0 for m < r
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int m = 16 * M + 4 * kg + mm;
                acc = mfma4(acc, sT[m * LC + 16 * R + lr], sdA[m * LC + 16 * I + lr]);
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) sXm[(16 * R + 4 * kg + e) * LC + 16 * I + lr] = acc[e];
    });
    __syncthreads();
    static_for<NB * (NB + 1) / 2>([&](auto TI) {
        constexpr int t = TI, R = lower_row(t), I = t - R * (R + 1) / 2;
        if (t % NW != wave) return;
        const int i = 16 * I + lr;
        float av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = ck_a[unit * (long)C * C + (16 * R + 4 * kg + e) * C + i];
        floatx4 acc = zero4();
#pragma unroll
        for (int M = 0; M <= I; ++M)                                // T[i][m] = 0 for m > i
            acc = mfma16(acc, lds4(sXm + (16 * R + lr) * LC + 16 * M + 4 * kg), lds4(sT + (16 * I + lr) * LC + 16 * M + 4 * kg));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * R + 4 * kg + e;
            const float dm = i < r ? -acc[e] : 0.f;
            const float x = row_sum16(dm * av[e]);
            if (lr == 0) sDb3[I * C + r] = x;
            sdA[r * LC + i] = sBeta[r] * dm;
        }
    });
    __syncthreads();

    // ---- phase 5, per wave over its channel block: the decays, the pairwise decays
    // of A and P, the prefix-sum adjoint.  Pairwise factors e^{G_r - G_i} (i <= r)
    // are split at 16-row block boundaries so that every factor formed is <= 1:
    //   Er_r = e^{G_r - gs(R(r))},  Ei_r = e^{gm(R(r)) - G_r},  B_RI = e^{gs(R) - gm(I)} (I < R).
    // Inside one block, e^{G_r - G_i} = Er_r / Er_i, exact while the block's log-gate
    // sum stays above -SAFE_SPAN; otherwise that block is done term by term.
    // The B operands of the products (K Ei, K Er, Q Er, K / Er of row block I) are
    // formed from this lane's own values: lane l holds rows 16I + 4(l/16) + m,
    // channel l%16.  e^G = e^{gs(R)} Er and e^{G_C - G} = e^{G_C - gm(R)} Ei.
    // The row blocks run last to first, so that the prefix-sum adjoint (dg_t =
    // dG_C + sum_{r >= t} dG_r, with dG_C from gam = e^{G_C} and Kb = e^{G_C - G} K)
    // is carried along: a suffix sum over the rows (rows past the sequence end
    // have dG = 0).
    {
        floatx4 er[NB], ei[NB];
        bool safe[NB];
        float gcp = 0.f;
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            safe[R] = gs[R + 1] - gs[R] >= -SAFE_SPAN;
            const float fb = __expf(gs[NB] - gs[R + 1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                er[R][e] = __expf(G[R][e] - gs[R]);
                ei[R][e] = __expf(gs[R + 1] - G[R][e]);
                gcp += fb * ei[R][e] * kv[R][e] * aKb[R][e];
            }
        }
        auto v4 = [&](const float (&x)[4]) { return floatx4{x[0], x[1], x[2], x[3]}; };
        float carry = dgam * __expf(gs[NB]) + col_sum4(gcp);
#pragma unroll
        for (int R = NB - 1; R >= 0; --R) {
            // each term's block factor rides on its B operand, so that the terms of
            // XA, XP, YA and YP each accumulate in one MFMA chain:
            //   XA = Er (sum_{I<R} dA_RI (B_RI Km_I) + dA_RR Ki),
            //   YA = Ei (sum_{I>R} dA^T_RI (B_IR Ks_I) + e^{-tot_R} dA^T_RR Ks_R),
            // with Ki = K / Er and e^{-tot_R} = (1/Er) / Ei on safe blocks (at most
            // e^SAFE_SPAN, finite in fp32), both zero on unsafe ones (done term by term)
            floatx4 xa = zero4(), xp = zero4(), ya = zero4(), yp = zero4();
#pragma unroll
            for (int I = 0; I < R; ++I) {                          // earlier column blocks
                const floatx4 km = v4(kv[I]) * ei[I] * __expf(gs[R] - gs[I + 1]);
                xa = mfma16(xa, lds4(sdA + (16 * R + lr) * LC + 16 * I + 4 * kg), km);
                xp = mfma16(xp, lds4(sdP + (16 * R + lr) * LC + 16 * I + 4 * kg), km);
            }
            floatx4 ier;                                            // 1 / Er (safe blocks only)
#pragma unroll
            for (int e = 0; e < 4; ++e) ier[e] = safe[R] ? __expf(gs[R] - G[R][e]) : 0.f;
            const floatx4 ki = v4(kv[R]) * ier;
            xa = mfma16(xa, lds4(sdA + (16 * R + lr) * LC + 16 * R + 4 * kg), ki);
            xp = mfma16(xp, lds4(sdP + (16 * R + lr) * LC + 16 * R + 4 * kg), ki);
#pragma unroll
            for (int I = R + 1; I < NB; ++I) {                     // later row blocks
                const float b = __expf(gs[I] - gs[R + 1]);
                ya = mfma16(ya, col4(sdA + (16 * I + 4 * kg) * LC + 16 * R + lr, LC), v4(kv[I]) * er[I] * b);
                yp = mfma16(yp, col4(sdP + (16 * I + 4 * kg) * LC + 16 * R + lr, LC), v4(qv[I]) * er[I] * b);
            }
            const float td = safe[R] ? __expf(gs[R] - gs[R + 1]) : 0.f;
            ya = mfma16(ya, col4(sdA + (16 * R + 4 * kg) * LC + 16 * R + lr, LC), v4(kv[R]) * er[R] * td);
            yp = mfma16(yp, col4(sdP + (16 * R + 4 * kg) * LC + 16 * R + lr, LC), v4(qv[R]) * er[R] * td);
            float XA[4], XP[4], YA[4], YP[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                XA[e] = er[R][e] * xa[e];
                XP[e] = er[R][e] * xp[e];
                YA[e] = ei[R][e] * ya[e];
                YP[e] = ei[R][e] * yp[e];
            }
            if (!safe[R]) {                                         // the diagonal block term by term
                // row i's G, k and q of this channel, from the lane holding row i (the
                // same channel: safe[R] is the same in both lanes)
#pragma unroll 1
                for (int i = 16 * R; i < 16 * R + 16; ++i) {
                    const int src = lr + 16 * ((i >> 2) & 3), ei2 = i & 3;
                    float gsel = 0.f, ksel = 0.f, qsel = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (m == ei2) { gsel = G[R][m]; ksel = kv[R][m]; qsel = qv[R][m]; }
                    const float Gi = __shfl(gsel, src), ki2 = __shfl(ksel, src), qi = __shfl(qsel, src);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * R + 4 * kg + e;
                        if (i <= r) {
                            const float wd = __expf(G[R][e] - Gi);
                            if (i < r) XA[e] += sdA[r * LC + i] * ki2 * wd;
                            XP[e] += sdP[r * LC + i] * ki2 * wd;
                        }
                        if (i >= r) {
                            const float wu = __expf(Gi - G[R][e]);
                            if (i > r) YA[e] += sdA[i * LC + r] * ki2 * wu;
                            YP[e] += sdP[i * LC + r] * qi * wu;
                        }
                    }
                }
            }
            float dGv[4];
            const float ea = __expf(gs[R]), fa = __expf(gs[NB] - gs[R + 1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                const float E = ea * er[R][e], F = fa * ei[R][e];
                const float kc = kv[R][e], qc = qv[R][e];
                const float dKt = sBeta[r] * aTd[R][e], dQt = aQ[R][e], dKb = aKb[R][e];
                const float dK = E * dKt + F * dKb + XA[e] + YA[e] + YP[e], dQ = E * dQt + XP[e];
                dGv[e] = E * kc * dKt + E * qc * dQt - F * kc * dKb + kc * XA[e] - kc * YA[e] + qc * XP[e] -
                         kc * YP[e];
                if (valid(r)) {                    // gradients: streaming stores (nothing here reads them)
                    __builtin_nontemporal_store(dQ, dq + grow(r) * DK + cw);
                    __builtin_nontemporal_store(dK, dk + grow(r) * DK + cw);
                }
            }
            // suffix sums of dG over this block's rows (4 in the lane, then the row
            // groups after it), on top of everything after the block
            float sfx[4];
            sfx[3] = dGv[3];
            sfx[2] = sfx[3] + dGv[2];
            sfx[1] = sfx[2] + dGv[1];
            sfx[0] = sfx[1] + dGv[0];
            const float t1 = __shfl(sfx[0], lane + 16), t2 = __shfl(sfx[0], lane + 32), t3 = __shfl(sfx[0], lane + 48);
            const float after = (kg < 3 ? t1 : 0.f) + (kg < 2 ? t2 : 0.f) + (kg < 1 ? t3 : 0.f);
            const float base = carry + after;
            carry += col_sum4(sfx[0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * kg + e;
                const float val = base + sfx[e];
                if (gate == GATE_CHANNEL) {
                    if (valid(r)) __builtin_nontemporal_store((floored >> (4 * R + e)) & 1u ? 0.f : val, dg + grow(r) * DK + cw);
                } else {
                    const float hs = row_sum16(val);
                    if (gate == GATE_HEAD && lr == 0) sHd[wave * C + r] = hs;
                }
            }
        }
    }
    __syncthreads();
    if (tid < C && valid(tid)) {
        float db = sDb1[tid];
        for (int w = 0; w < NW; ++w) db += sDb2[w * C + tid];
        for (int w = 0; w < NW; ++w) db += sDb3[w * C + tid];
        dbeta[grow(tid)] = db;
        if (gate == GATE_HEAD) {
            float s = 0.f;
            for (int w = 0; w < NW; ++w) s += sHd[w * C + tid];
            dg[grow(tid)] = g[grow(tid)] < G_FLOOR ? 0.f : s;
        }
    }
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
        typedef BwdChainHCfg<DK, DV, C> HC;
        if constexpr (sizeof(T) == 2 && HC::FITS) {
            hipLaunchKernelGGL((chunk_bwd_chain_h_kernel<DK, DV, C>), dim3((unsigned)(nsh * HC::NSL)), dim3(256), 0,
                               a.stream, (const bf16*)(ws + w.qt), (const bf16*)(ws + w.wk),
                               (const bf16*)(ws + w.kb), (const bf16*)(ws + w.p), (const float*)(ws + w.gam), b.dO,
                               b.dST, b.dS0, b.ck_dS, b.ck_dW, unit_map(a));
        } else {
            hipLaunchKernelGGL((chunk_bwd_chain_kernel<T, DK, DV, C>), dim3((unsigned)(nsh * CC::NSL)), dim3(256), 0,
                               a.stream, (const T*)(ws + w.qt), (const T*)(ws + w.wk), (const T*)(ws + w.kb),
                               (const T*)(ws + w.p), (const float*)(ws + w.gam), b.dO, b.dST, b.dS0, b.ck_dS,
                               b.ck_dW, unit_map(a));
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || units == 0) return e;
        hipLaunchKernelGGL((chunk_bwd_intra_kernel<T, DK, DV, C>), dim3((unsigned)units), dim3(IC::NT), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, b.dO, a.ck_state, b.ck_dS,
                           a.ck_w, b.ck_dW, a.ck_t, a.ck_a, b.dq, b.dk, b.dv, b.dg, b.dbeta,
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

// The checkpoints follow the forward workspace, one slot per unit of the grid.
static BwdLayout bwd_units(const WsLayout& fwd, size_t units, int dk, int dv, int C) {
    BwdLayout L{};
    L.fwd = fwd;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t off = al(L.fwd.total);
    L.t = off;     off = al(off + units * C * C * 4);
    L.a = off;     off = al(off + units * C * C * 4);
    L.state = off; off = al(off + units * dk * dv * 4);
    L.w = off;     off = al(off + units * C * dv * 4);
    L.dS = off;    off = al(off + units * dk * dv * 4);
    L.dW = off;    off = al(off + units * C * dv * 4);
    L.total = off;
    return L;
}

BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, bool in_bf16, int C) {
    const size_t units = (size_t)B * H * (size_t)((T + C - 1) / C);
    return bwd_units(ws_layout(B, T, H, dk, dv, in_bf16, C, true), units, dk, dv, C);
}

BwdLayout bwd_layout_packed(int N, int T, int H, int dk, int dv, bool in_bf16, int C) {
    const size_t units = ((size_t)((T + C - 1) / C) + (size_t)N) * H;     // as unit_count
    return bwd_units(ws_layout_packed(N, T, H, dk, dv, in_bf16, C, true), units, dk, dv, C);
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
