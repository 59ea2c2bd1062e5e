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
// (6.2 against 5.6 TB/s), and 256 for several tokens (measured faster there).
// Both shapes form the column sums the same way (below), so that a call with T
// tokens equals T single steps bitwise.  Thread (ty, tx) owns the
// float4 of columns 4*tx..4*tx+3 in rows ty, ty+RG, ty+2RG, ...: every row read
// is a fully coalesced DV*4-byte line.  Column sums are combined in LDS in a
// fixed order (bitwise reproducible).
//
// Several tokens per call (T > 1, inputs [N,T,H,d]): the tokens are applied in
// order with the state kept in registers, so the state is read and written once
// per call instead of once per token; the result equals T single steps bitwise.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <typename TIn, typename TOut, int DK, int DV, int NT>
__global__ __launch_bounds__(NT) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
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

    // per-token vectors, double-buffered so that token t+1 can be staged while
    // token t's update still reads them
    __shared__ float s_ak[2][DK], s_aq[2][DK], s_k[2][DK], s_a[2][DK];
    __shared__ float s_red[2][RED][DV];
    __shared__ float s_u[DV];
    __shared__ float s_qk[2], s_iq[2], s_ik[2];

    const long nh = blockIdx.x;
    const long n = nh / H;
    const int h = (int)(nh % H);
    const int tid = threadIdx.x;
    const int tx = tid % CG, ty = tid / CG;
    float* S = state + nh * (long)DK * DV;
    // With in-kernel L2 normalisation of q and k, the raw vectors go through the
    // state products and the scalars 1/||q||, 1/||k|| are applied to the results:
    // r = S^T(alpha*k)/||k||, s = S^T(alpha*q)/||q||, and the write k u^T uses
    // u/||k||.  Without it both scalars are 1 and change nothing.
    const bool qknorm = gate & MODE_QK_L2NORM;

    // Issue every state load first: RPT independent 16-byte loads in flight.
    floatx4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (long)(ty + i * RG) * DV) + tx);

    for (int t = 0; t < T; ++t) {
        const int pb = t & 1;
        const long row = (n * T + t) * H + h;            // token t of (n, h); [N,T,H,d] inputs
        if (tid < DK) {
            const float a = __expf(gate_at(g, gate, row, DK, tid));   // exp(-inf) = 0: alpha = 0 clears
            const float kc = to_f32(k[row * DK + tid]);
            const float qc = to_f32(q[row * DK + tid]);
            s_a[pb][tid] = a; s_k[pb][tid] = kc; s_ak[pb][tid] = a * kc; s_aq[pb][tid] = a * qc;
        }
        if (tid < WAVE) {                                 // q.k and the norms, fixed-order wave reduction
            float p = 0.f, nq = 0.f, nk = 0.f;
#pragma unroll
            for (int c = tid; c < DK; c += WAVE) {
                const float qc = to_f32(q[row * DK + c]), kc = to_f32(k[row * DK + c]);
                p += qc * kc;
                nq += qc * qc;
                nk += kc * kc;
            }
#pragma unroll
            for (int off = WAVE / 2; off > 0; off >>= 1) {
                p += __shfl_xor(p, off);
                nq += __shfl_xor(nq, off);
                nk += __shfl_xor(nk, off);
            }
            if (tid == 0) {
                const float iq = qknorm ? inv_norm(nq) : 1.f, ik = qknorm ? inv_norm(nk) : 1.f;
                s_qk[pb] = p * iq * ik;
                s_iq[pb] = iq;
                s_ik[pb] = ik;
            }
        }
        __syncthreads();

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
            const float u = beta[row] * (to_f32(v[row * DV + tid]) - rr * ik);
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
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(sv[i], reinterpret_cast<floatx4*>(S + (long)(ty + i * RG) * DV) + tx);
}

template <typename TIn, typename TOut, int DK, int DV>
static hipError_t launch_decode(const DecodeArgs& a) {
    const long nh = (long)a.N * a.H;
    if (a.T == 1)
        hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, 1024>), dim3((unsigned)nh), dim3(1024), 0,
                           a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.beta,
                           a.state, (TOut*)a.o, a.H, a.T, a.gate | a.pre);
    else
        hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, 256>), dim3((unsigned)nh), dim3(256), 0,
                           a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.beta,
                           a.state, (TOut*)a.o, a.H, a.T, a.gate | a.pre);
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
