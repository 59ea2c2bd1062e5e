// kda_pre_bwd.hip -- the backward pass through the fused pre-processing: the
// steps that produce q, k and the log-gate in the method's workloads (each q and
// k row divided by its Euclidean norm; the log-gate -softplus(a) of a
// pre-activation a).  Before the backward stages, the pre-processed q, k and
// log-gate are written to the workspace; after them, the chain rule turns the
// gradients of those into gradients of the raw inputs, in place:
//   y = x / |x|:          dx = (dy - y (y . dy)) / |x|    (zero row: dx = 0)
//   g = -softplus(a):     da = -dg * sigmoid(a)
// All four are HBM-bound passes.  Each lane moves 8 consecutive values (16-byte
// loads and stores); a row of dk values is spread over dk/8 lanes and reduced
// with lane exchanges.  Pointers without the 16-byte alignment that needs (an
// output, or a gate tensor, given with element alignment only) take the
// one-value-per-lane forms.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

// sigmoid(a) without overflow on either side
__device__ __forceinline__ float sigmoid_stable(float a) {
    const float e = expf(-fabsf(a));
    return a >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// One wave per row of DK values: rows of q (blockIdx.y = 0) or k (1).
// xn = x / |x| in the input dtype, inv = 1 / |x| (0 for a zero row).
template <typename T, int DK>
__global__ __launch_bounds__(256) void pre_rows_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       T* __restrict__ qn, T* __restrict__ kn,
                                                       float* __restrict__ inv, long rows) {
    constexpr int PER = DK / 64;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const bool isk = blockIdx.y == 1;
    const T* x = (isk ? k : q) + row * DK;
    T* xn = (isk ? kn : qn) + row * DK;
    float v[PER], ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = to_f32<T>(x[lane + 64 * i]);
        ss += v[i] * v[i];
    }
    const float r = inv_norm(wave_sum(ss));
#pragma unroll
    for (int i = 0; i < PER; ++i) xn[lane + 64 * i] = from_f32<T>(v[i] * r);
    if (lane == 0) inv[(isk ? rows : 0) + row] = r;
}

// The log-gate as the backward stages read it: fp32, activated.
__global__ __launch_bounds__(256) void pre_gate_kernel(const void* __restrict__ g, int mode,
                                                       float* __restrict__ out, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = gate_load(g, mode, i);
}

// In place: dy (the gradient of the normalised row) -> dx (of the raw row).
template <typename T, int DK>
__global__ __launch_bounds__(256) void post_rows_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        float* __restrict__ dq, float* __restrict__ dk,
                                                        const float* __restrict__ inv, long rows) {
    constexpr int PER = DK / 64;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const bool isk = blockIdx.y == 1;
    const T* x = (isk ? k : q) + row * DK;
    float* d = (isk ? dk : dq) + row * DK;
    const float r = inv[(isk ? rows : 0) + row];
    float y[PER], dy[PER], dot = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        y[i] = to_f32<T>(x[lane + 64 * i]) * r;
        dy[i] = d[lane + 64 * i];
        dot += y[i] * dy[i];
    }
    dot = wave_sum(dot);
#pragma unroll
    for (int i = 0; i < PER; ++i) d[lane + 64 * i] = (dy[i] - y[i] * dot) * r;
}

// In place: dg (of the log-gate) -> da (of the pre-activation a).
__global__ __launch_bounds__(256) void post_gate_kernel(const void* __restrict__ g, int mode,
                                                        float* __restrict__ dg, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float a = (mode & MODE_GATE_BF16) ? (float)reinterpret_cast<const bf16*>(g)[i]
                                            : reinterpret_cast<const float*>(g)[i];
    dg[i] = -dg[i] * sigmoid_stable(a);
}

// Eight channels per lane, DK / 8 lanes per row: rows of q (blockIdx.y = 0) or k (1).
template <typename T, int DK>
__global__ __launch_bounds__(256) void pre_rows_vec_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           T* __restrict__ qn, T* __restrict__ kn,
                                                           float* __restrict__ inv, long rows) {
    constexpr int G = DK / 8, RPB = 256 / G;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / G;
    const int c = 8 * (threadIdx.x % G);
    if (row >= rows) return;                          // whole lane groups: the exchanges stay inside one
    const bool isk = blockIdx.y == 1;
    float x[8];
    Vec8<T>::load((isk ? k : q) + row * DK + c, x);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = inv_norm(ss);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] *= r;
    Vec8<T>::store((isk ? kn : qn) + row * DK + c, x);
    if (c == 0) inv[(isk ? rows : 0) + row] = r;
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void post_rows_vec_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            float* __restrict__ dq, float* __restrict__ dk,
                                                            const float* __restrict__ inv, long rows) {
    constexpr int G = DK / 8, RPB = 256 / G;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / G;
    const int c = 8 * (threadIdx.x % G);
    if (row >= rows) return;
    const bool isk = blockIdx.y == 1;
    float* d = (isk ? dk : dq) + row * DK + c;
    float y[8], dy[8];
    Vec8<T>::load((isk ? k : q) + row * DK + c, y);
    Vec8<float>::load(d, dy);
    const float r = inv[(isk ? rows : 0) + row];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        y[i] *= r;
        dot += y[i] * dy[i];
    }
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) dy[i] = (dy[i] - y[i] * dot) * r;
    Vec8<float>::store(d, dy);
}

// Eight gate values per lane (n a multiple of 8).
template <bool BF>
__global__ __launch_bounds__(256) void pre_gate_vec_kernel(const void* __restrict__ g, int mode,
                                                           float* __restrict__ out, long n) {
    const long i = 8 * ((long)blockIdx.x * 256 + threadIdx.x);
    if (i >= n) return;
    float a[8];
    if constexpr (BF) Vec8<bf16>::load(reinterpret_cast<const bf16*>(g) + i, a);
    else Vec8<float>::load(reinterpret_cast<const float*>(g) + i, a);
    if (mode & MODE_GATE_SOFTPLUS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = neg_softplus(a[j]);
    }
    Vec8<float>::store(out + i, a);
}

template <bool BF>
__global__ __launch_bounds__(256) void post_gate_vec_kernel(const void* __restrict__ g, float* __restrict__ dg,
                                                            long n) {
    const long i = 8 * ((long)blockIdx.x * 256 + threadIdx.x);
    if (i >= n) return;
    float a[8], d[8];
    if constexpr (BF) Vec8<bf16>::load(reinterpret_cast<const bf16*>(g) + i, a);
    else Vec8<float>::load(reinterpret_cast<const float*>(g) + i, a);
    Vec8<float>::load(dg + i, d);
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = -d[j] * sigmoid_stable(a[j]);
    Vec8<float>::store(dg + i, d);
}

bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename T, int DK>
hipError_t rows_launch_scalar(const PreBwdArgs& p, bool post) {
    const dim3 grid((unsigned)((p.rows + 3) / 4), 2);
    if (post)
        hipLaunchKernelGGL((post_rows_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q, (const T*)p.k,
                           p.dq, p.dk, p.inv, p.rows);
    else
        hipLaunchKernelGGL((pre_rows_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q, (const T*)p.k,
                           (T*)p.qn, (T*)p.kn, p.inv, p.rows);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t rows_launch(const PreBwdArgs& p, bool post) {
    constexpr int RPB = 256 / (DK / 8);
    // q, k and the workspace are 16-byte aligned by the entry points' checks
    if (!post || (al16(p.dq) && al16(p.dk))) {
        const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB), 2);
        if (post)
            hipLaunchKernelGGL((post_rows_vec_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q,
                               (const T*)p.k, p.dq, p.dk, p.inv, p.rows);
        else
            hipLaunchKernelGGL((pre_rows_vec_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q,
                               (const T*)p.k, (T*)p.qn, (T*)p.kn, p.inv, p.rows);
        return hipGetLastError();
    }
    return rows_launch_scalar<T, DK>(p, post);
}

hipError_t rows_dispatch(const PreBwdArgs& p, bool post) {
    if (p.in_bf16) return p.dk_size == 64 ? rows_launch<bf16, 64>(p, post) : rows_launch<bf16, 128>(p, post);
    return p.dk_size == 64 ? rows_launch<float, 64>(p, post) : rows_launch<float, 128>(p, post);
}

long gate_elems(const PreBwdArgs& p) {
    return p.gate == GATE_CHANNEL ? p.rows * p.dk_size : p.gate == GATE_HEAD ? p.rows : 0;
}

}  // namespace

hipError_t run_pre_bwd_inputs(const PreBwdArgs& p) {
    if (p.rows == 0) return hipSuccess;
    if (p.mode & MODE_QK_L2NORM) {
        const hipError_t e = rows_dispatch(p, false);
        if (e != hipSuccess) return e;
    }
    const long n = gate_elems(p);
    if (n > 0 && (p.mode & (MODE_GATE_SOFTPLUS | MODE_GATE_BF16))) {
        const dim3 grid8((unsigned)((n / 8 + 255) / 256));
        if (n % 8 == 0 && al16(p.g) && (p.mode & MODE_GATE_BF16))
            hipLaunchKernelGGL(pre_gate_vec_kernel<true>, grid8, dim3(256), 0, p.stream, p.g, p.mode, p.g_act, n);
        else if (n % 8 == 0 && al16(p.g))
            hipLaunchKernelGGL(pre_gate_vec_kernel<false>, grid8, dim3(256), 0, p.stream, p.g, p.mode, p.g_act, n);
        else
            hipLaunchKernelGGL(pre_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, p.stream, p.g,
                               p.mode, p.g_act, n);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t run_pre_bwd_grads(const PreBwdArgs& p) {
    if (p.rows == 0) return hipSuccess;
    if (p.mode & MODE_QK_L2NORM) {
        const hipError_t e = rows_dispatch(p, true);
        if (e != hipSuccess) return e;
    }
    const long n = gate_elems(p);
    if (n > 0 && (p.mode & MODE_GATE_SOFTPLUS)) {
        const dim3 grid8((unsigned)((n / 8 + 255) / 256));
        const bool vec = n % 8 == 0 && al16(p.g) && al16(p.dg);
        if (vec && (p.mode & MODE_GATE_BF16))
            hipLaunchKernelGGL(post_gate_vec_kernel<true>, grid8, dim3(256), 0, p.stream, p.g, p.dg, n);
        else if (vec)
            hipLaunchKernelGGL(post_gate_vec_kernel<false>, grid8, dim3(256), 0, p.stream, p.g, p.dg, n);
        else
            hipLaunchKernelGGL(post_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, p.stream, p.g,
                               p.mode, p.dg, n);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
