// kda_pre_bwd.hip -- the backward pass through the fused pre-processing: the
// steps that produce q, k and the log-gate in the method's workloads (each q and
// k row divided by its Euclidean norm; the log-gate -softplus(a) of a
// pre-activation a).  Before the backward stages, the pre-processed q, k and
// log-gate are written to the workspace; after them, the chain rule turns the
// gradients of those into gradients of the raw inputs, in place:
//   y = x / |x|:          dx = (dy - y (y . dy)) / |x|    (zero row: dx = 0)
//   g = -softplus(a):     da = -dg * sigmoid(a)
// All four kernels are elementwise or one wave per row: HBM-bound passes.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

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
    const float e = expf(-fabsf(a));                 // sigmoid without overflow on either side
    const float sig = a >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
    dg[i] = -dg[i] * sig;
}

template <typename T, int DK>
hipError_t rows_launch(const PreBwdArgs& p, bool post) {
    const dim3 grid((unsigned)((p.rows + 3) / 4), 2);
    if (post)
        hipLaunchKernelGGL((post_rows_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q, (const T*)p.k,
                           p.dq, p.dk, p.inv, p.rows);
    else
        hipLaunchKernelGGL((pre_rows_kernel<T, DK>), grid, dim3(256), 0, p.stream, (const T*)p.q, (const T*)p.k,
                           (T*)p.qn, (T*)p.kn, p.inv, p.rows);
    return hipGetLastError();
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
        hipLaunchKernelGGL(post_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, p.stream, p.g,
                           p.mode, p.dg, n);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
