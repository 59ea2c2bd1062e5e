// kda_decode.hip -- single-token KDA step with the state updated in place.
//
// The step of section 十五 of "我终于看懂了 KDA…" (read the state, compute the
// output, update the state) with the order of its section 八 (decay, read, error,
// write).  With alpha = exp(g) the update expands to
//     r = S^T (alpha*k),  s = S^T (alpha*q),  u = beta (v - r),
//     o = s + (q.k) u,    S_new = Diag(alpha) S + k u^T,
// so each state element is read once and written once: the state stays in
// registers between the column reductions and the rewrite.
//
// One workgroup per (sequence, head): 1024 threads (16 waves) for a single token,
// where more waves in flight per CU measured faster than more rows per thread
// (6.2 against 5.6 TB/s), 512 for two tokens and 256 from three on (measured
// fastest there).  Every shape forms the column sums the same way (below), so
// that a call with T tokens equals T single steps bitwise.  Thread (ty, tx) owns the
// float4 of columns 4*tx..4*tx+3 in rows ty, ty+RG, ty+2RG, ...: every row read
// is a fully coalesced DV*4-byte line.  Column sums are combined in LDS in a
// fixed order (bitwise reproducible).
//
// Several tokens per call (T > 1, inputs [N,T,H,d]): the tokens are applied in
// order with the state kept in registers, so the state is read and written once
// per call instead of once per token; the result equals T single steps bitwise.
// Each token's inputs are loaded while the previous token is computed.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// One token's inputs as this thread uses them: channel tid % DK of q, k and the
// gate, value column tid % DV of v, beta, and for dk = 128 channel tid % 64 + 64
// of q and k.  Every thread issues the same loads
// whatever the gate layout and dtype (the gate as two 16-bit halves, the high one
// alone for bf16, from a valid stand-in address without gates), so a token's
// loads can be in flight while the previous token is computed.
template <typename TIn>
struct TokenIn {
    TIn q, k, v;
    TIn q2, k2;                  // channel tid % 64 + 64 (dk = 128): the rest of wave 0's q.k
    unsigned short glo, ghi;
    float beta;
};

template <typename TIn, int DK, int DV>
__device__ __forceinline__ TokenIn<TIn> load_token(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                   const TIn* __restrict__ v, const void* __restrict__ g,
                                                   const float* __restrict__ beta, int mode, long row, int tid) {
    const int c = tid % DK, cv = tid % DV;
    const int layout = gate_layout(mode);
    const bool gb = mode & MODE_GATE_BF16;
    const long gi = layout == 0 ? row * DK + c : row;
    const unsigned short* base = reinterpret_cast<const unsigned short*>(layout < 2 ? g : (const void*)beta);
    const long lo = layout < 2 ? (gb ? gi : 2 * gi) : 0;
    const long hi = layout < 2 ? (gb ? gi : 2 * gi + 1) : 0;
    TokenIn<TIn> x;
    x.q = q[row * DK + c];
    x.k = k[row * DK + c];
    if constexpr (DK > WAVE) {
        const int c2 = tid % WAVE + WAVE;
        x.q2 = q[row * DK + c2];
        x.k2 = k[row * DK + c2];
    }
    x.v = v[row * DV + cv];
    x.glo = base[lo];
    x.ghi = base[hi];
    x.beta = beta[row];
    return x;
}

// The log-gate from its loaded halves (0 without gates).
__device__ __forceinline__ float token_gate(unsigned short glo, unsigned short ghi, int mode) {
    const unsigned bits = ((unsigned)ghi << 16) | ((mode & MODE_GATE_BF16) ? 0u : (unsigned)glo);
    const float a = __uint_as_float(bits);
    const float x = (mode & MODE_GATE_SOFTPLUS) ? neg_softplus(a) : a;
    return gate_layout(mode) < 2 ? x : 0.f;
}

template <typename TIn, typename TOut, int DK, int DV, int NT, bool MULTI>
__global__ __launch_bounds__(NT, NT == 256 ? 3 : 1) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const void* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ state, TOut* __restrict__ o, int H, int T, int gate) {
    // No implicit multiply-add contraction: the fused operations are the explicit
    // fmaf calls, so that every launch shape performs the same arithmetic.
#pragma clang fp contract(off)
    constexpr int CG = DV / 4;       // threads across one row (float4 each)
    constexpr int RG = NT / CG;      // row groups
    constexpr int RPT = DK / RG;     // rows per thread
    // The column sums are formed as RED partial sums whatever NT is: partial y
    // covers rows y, y + RED, y + 2 RED, ... in that order, and the partials are
    // added in the order y = 0, 1, ...  A thread forms P of them, so every
    // launch shape gives the same result bitwise.
    constexpr int RED = 1024 / CG;
    constexpr int P = RED / RG;
    static_assert(DK % RG == 0 && RED % RG == 0 && DK % RED == 0, "row split");
    static_assert(NT >= DK && NT >= DV, "one thread per channel");

    // per-token vectors, double-buffered so that token t+1 can be staged while
    // token t's update still reads them
    __shared__ float s_ak[2][DK], s_aq[2][DK], s_k[2][DK], s_a[2][DK];
    __shared__ float s_red[2][RED][DV];
    __shared__ float s_u[DV];
    __shared__ float s_qk[2], s_iq[2], s_ik[2];

    const unsigned nhu = blockIdx.x;                     // one workgroup per (sequence, head)
    const long nh = nhu, n = nhu / (unsigned)H;
    const int h = (int)(nhu % (unsigned)H);
    const int tid = threadIdx.x;
    const int tx = tid % CG, ty = tid / CG;
    const int TT = MULTI ? T : 1;
    float* S = state + nh * (long)DK * DV;
    // With in-kernel L2 normalisation of q and k, the raw vectors go through the
    // state products and the scalars 1/||q||, 1/||k|| are applied to the results:
    // r = S^T(alpha*k)/||k||, s = S^T(alpha*q)/||q||, and the write k u^T uses
    // u/||k||.  Without it both scalars are 1 and change nothing.
    const bool qknorm = gate & MODE_QK_L2NORM;
    auto row_of = [&](int t) -> long { return (n * T + t) * H + h; };   // [N,T,H,d] inputs

    // The first token's inputs, then every state load: RPT independent 16-byte
    // loads in flight while the token's vectors are staged.
    TokenIn<TIn> cur = load_token<TIn, DK, DV>(q, k, v, g, beta, gate, row_of(0), tid);
    __builtin_amdgcn_sched_barrier(0);                   // issued before the state loads
    floatx4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (long)(ty + i * RG) * DV) + tx);
    __builtin_amdgcn_sched_barrier(0);

    // Stage a token's vectors in LDS buffer b.  Every thread stages its channel
    // (threads tid and tid + DK store equal values), so there is no branch for
    // the compiler to sink the loads into.
    auto stage = [&](const TokenIn<TIn>& x, int b) {
        const int c = tid % DK;
        const float a = __expf(token_gate(x.glo, x.ghi, gate));     // exp(-inf) = 0: alpha = 0 clears
        const float kc = to_f32(x.k), qc = to_f32(x.q);
        s_a[b][c] = a; s_k[b][c] = kc; s_ak[b][c] = a * kc; s_aq[b][c] = a * qc;
        if (tid < WAVE) {                                // q.k and the norms, fixed-order wave reduction
            float p = 0.f, nq = 0.f, nk = 0.f;
            p += qc * kc;
            nq += qc * qc;
            nk += kc * kc;
            if constexpr (DK > WAVE) {
                const float q2 = to_f32(x.q2), k2 = to_f32(x.k2);
                p += q2 * k2;
                nq += q2 * q2;
                nk += k2 * k2;
            }
#pragma unroll
            for (int off = WAVE / 2; off > 0; off >>= 1) {
                p += __shfl_xor(p, off);
                nq += __shfl_xor(nq, off);
                nk += __shfl_xor(nk, off);
            }
            if (tid == 0) {
                const float iq = qknorm ? inv_norm(nq) : 1.f, ik = qknorm ? inv_norm(nk) : 1.f;
                s_qk[b] = p * iq * ik;
                s_iq[b] = iq;
                s_ik[b] = ik;
            }
        }
    };
    stage(cur, 0);                                       // waits for the token's loads only

    int t = 0;
    do {                                                 // T >= 1: the host returns early for T = 0
        const int pb = t & 1;
        const long row = row_of(t);
        __syncthreads();
        // the next token's inputs (the last token's again at the end), in flight
        // while this token is computed
        TokenIn<TIn> nxt;
        if constexpr (MULTI) nxt = load_token<TIn, DK, DV>(q, k, v, g, beta, gate, row_of(t + 1 < T ? t + 1 : t), tid);

        float r[P][4], s[P][4];
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) { r[j][m] = 0.f; s[j][m] = 0.f; }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {              // row ty + i RG: partial ty + (i % P) RG
            const int c = ty + i * RG, j = i % P;
            const float ak = s_ak[pb][c], aq = s_aq[pb][c];
            r[j][0] = fmaf(ak, sv[i].x, r[j][0]); r[j][1] = fmaf(ak, sv[i].y, r[j][1]);
            r[j][2] = fmaf(ak, sv[i].z, r[j][2]); r[j][3] = fmaf(ak, sv[i].w, r[j][3]);
            s[j][0] = fmaf(aq, sv[i].x, s[j][0]); s[j][1] = fmaf(aq, sv[i].y, s[j][1]);
            s[j][2] = fmaf(aq, sv[i].z, s[j][2]); s[j][3] = fmaf(aq, sv[i].w, s[j][3]);
        }
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                s_red[0][ty + j * RG][4 * tx + m] = r[j][m];
                s_red[1][ty + j * RG][4 * tx + m] = s[j][m];
            }
        __syncthreads();

        if (tid < DV) {
            float rr = 0.f, ss = 0.f;
#pragma unroll
            for (int y = 0; y < RED; ++y) { rr += s_red[0][y][tid]; ss += s_red[1][y][tid]; }
            const float ik = s_ik[pb];
            const float u = cur.beta * (to_f32(cur.v) - rr * ik);
            s_u[tid] = u * ik;
            o[row * DV + tid] = from_f32<TOut>(ss * s_iq[pb] + s_qk[pb] * u);
        }
        __syncthreads();

        const float u0 = s_u[4 * tx], u1 = s_u[4 * tx + 1], u2 = s_u[4 * tx + 2], u3 = s_u[4 * tx + 3];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = ty + i * RG;
            const float a = s_a[pb][c], kc = s_k[pb][c];
            sv[i].x = fmaf(a, sv[i].x, kc * u0); sv[i].y = fmaf(a, sv[i].y, kc * u1);
            sv[i].z = fmaf(a, sv[i].z, kc * u2); sv[i].w = fmaf(a, sv[i].w, kc * u3);
        }
        if constexpr (MULTI) {                           // into the other buffer: no reader left there
            stage(nxt, pb ^ 1);
            cur = nxt;
        }
    } while (++t < TT);
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(sv[i], reinterpret_cast<floatx4*>(S + (long)(ty + i * RG) * DV) + tx);
}

// Workgroup size by tokens per call, as measured: 1024 threads for one token,
// 512 for two, 256 from three on (more workgroups per CU hide the per-token
// barriers once the state traffic is spread over several tokens).
template <typename TIn, typename TOut, int DK, int DV, int NT, bool MULTI>
static void launch_decode_nt(const DecodeArgs& a) {
    hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, NT, MULTI>), dim3((unsigned)((long)a.N * a.H)), dim3(NT),
                       0, a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (const void*)a.g, a.beta,
                       a.state, (TOut*)a.o, a.H, a.T, a.gate | a.pre);
}

template <typename TIn, typename TOut, int DK, int DV>
static hipError_t launch_decode(const DecodeArgs& a) {
    switch (decode_block_threads(a.T)) {
        case 1024: launch_decode_nt<TIn, TOut, DK, DV, 1024, false>(a); break;
        case 512: launch_decode_nt<TIn, TOut, DK, DV, 512, true>(a); break;
        default: launch_decode_nt<TIn, TOut, DK, DV, 256, true>(a); break;
    }
    return hipGetLastError();
}

template <typename TIn, typename TOut>
static hipError_t dispatch_dims(const DecodeArgs& a) {
    if (a.dk == 64 && a.dv == 64) return launch_decode<TIn, TOut, 64, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_decode<TIn, TOut, 64, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_decode<TIn, TOut, 128, 64>(a);
    return launch_decode<TIn, TOut, 128, 128>(a);
}

hipError_t run_decode_step(const DecodeArgs& a) {
    if (a.in_bf16) return a.out_bf16 ? dispatch_dims<bf16, bf16>(a) : dispatch_dims<bf16, float>(a);
    return a.out_bf16 ? dispatch_dims<float, bf16>(a) : dispatch_dims<float, float>(a);
}

}  // namespace kda
