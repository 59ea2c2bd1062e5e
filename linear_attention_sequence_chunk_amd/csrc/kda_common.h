// kda_common.h -- device-side building blocks shared by the libkda kernels (gfx950).
//
// MFMA conventions used everywhere (16x16 output tiles, wave64):
//   accumulator element e (0..3) of lane l  <->  tile row 4*(l/16)+e, tile column l%16
//   A operand: lane l supplies row l%16, k-slots kg*KPL .. kg*KPL+KPL-1 with kg = l/16
//   B operand: lane l supplies column l%16, the same k-slots
// A and B fragments are read from LDS buffers in which the contraction index k is
// contiguous (A row-major [row][k], B stored transposed [col][k]).  Since A and B
// use the same slot -> k assignment, the contraction is exact whatever order the
// hardware pairs the slots in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Log-gates are clamped to this floor inside the chunk kernels so that every
// exponent difference stays finite (alpha >= exp(-20) ~ 2e-9 instead of 0).
constexpr float G_FLOOR = -20.0f;
// A 16-token sub-block whose log-gate sum (on any channel) is below -SAFE_SPAN is
// handled by the direct (unfactored) path; above it, exp(+-span) stays a normal
// fp32/bf16 number with room for the products.
constexpr float SAFE_SPAN = 64.0f;

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int KPL = 8;          // k values per lane per instruction
    static constexpr int KSTEP = 32;       // k per instruction
    typedef bf16x8 frag;
    __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 4;
    typedef float frag;
    __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ inline floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// acc += A[16 x K] * B[K x 16]; A at a (row stride lda), B^T at bt (row stride ldb).
// K must be a multiple of Mma<T>::KSTEP.
template <typename T>
__device__ inline floatx4 mma_tile(floatx4 acc, const T* __restrict__ a, int lda,
                                   const T* __restrict__ bt, int ldb, int K, int lane) {
    typedef typename Mma<T>::frag frag;
    const int r = lane & 15, kg = lane >> 4;
    const T* pa = a + r * lda + kg * Mma<T>::KPL;
    const T* pb = bt + r * ldb + kg * Mma<T>::KPL;
    for (int k0 = 0; k0 < K; k0 += Mma<T>::KSTEP) {
        frag fa = *reinterpret_cast<const frag*>(pa + k0);
        frag fb = *reinterpret_cast<const frag*>(pb + k0);
        acc = Mma<T>::mma(fa, fb, acc);
    }
    return acc;
}

// ---------------------------------------------------------------- conversions
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ inline float to_f32(T x);
template <> __device__ inline float to_f32<float>(float x) { return x; }
template <> __device__ inline float to_f32<bf16>(bf16 x) { return (float)x; }

// 8 consecutive elements of type T, loaded from global memory to fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    __device__ static inline void load(const bf16* p, float* out) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
    __device__ static inline void store(bf16* p, const float* in) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
        *reinterpret_cast<bf16x8*>(p) = v;
    }
    // the same as a streaming (nontemporal) store: for data read back only by a
    // later launch, so that it leaves the caches while this kernel still runs
    __device__ static inline void store_nt(bf16* p, const float* in) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
    }
};
template <> struct Vec8<float> {
    __device__ static inline void load(const float* p, float* out) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
    __device__ static inline void store(float* p, const float* in) {
        *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(in[4], in[5], in[6], in[7]);
    }
};

// NaN stays NaN (the comparison is false), -inf becomes G_FLOOR.
__device__ inline float clamp_g(float g) { return g < G_FLOOR ? G_FLOOR : g; }

// ---------------------------------------------------------------- gate and pre-processing
// Kernels that read q, k or g take a mode word: the gate layout (GateLayout in
// kda_launch.h) in bits 0-3 and pre-processing flags above it.
constexpr int MODE_QK_L2NORM = 1 << 4;       // q and k rows are L2-normalised in the kernel
constexpr int MODE_GATE_SOFTPLUS = 1 << 5;   // the gate tensor holds a; the log-gate is -softplus(a)
constexpr int MODE_GATE_BF16 = 1 << 6;       // the gate tensor is bf16

__device__ inline int gate_layout(int mode) { return mode & 15; }

// -softplus(a) = -log(1 + e^a) = -(max(a, 0) + log(1 + e^{-|a|})): no overflow, and
// the hardware exp2 / log2 (~1 ulp); the absolute error of the log-gate stays
// below ~1e-7, also where e^{-|a|} is small and 1 + e^{-|a|} rounds.
__device__ inline float neg_softplus(float a) {
    return -(fmaxf(a, 0.f) + __logf(1.f + __expf(-fabsf(a))));
}

__device__ inline float gate_load(const void* __restrict__ g, int mode, long idx) {
    const float a = (mode & MODE_GATE_BF16) ? (float)reinterpret_cast<const bf16*>(g)[idx]
                                            : reinterpret_cast<const float*>(g)[idx];
    return (mode & MODE_GATE_SOFTPLUS) ? neg_softplus(a) : a;
}

// The log-gate of (row, channel c): per channel g[row * dk + c], per head g[row],
// or none (0).
__device__ inline float gate_at(const void* __restrict__ g, int mode, long row, int dk, int c) {
    const int layout = gate_layout(mode);
    if (layout == 0) return gate_load(g, mode, row * dk + c);
    if (layout == 1) return gate_load(g, mode, row);
    return 0.f;
}
// Two consecutive channels c, c + 1 (c even) of the same row.
__device__ inline float2 gate_pair(const void* __restrict__ g, int mode, long row, int dk, int c) {
    const int layout = gate_layout(mode);
    if (layout == 0) {
        float2 x;
        if (mode & MODE_GATE_BF16) {
            const bf16x2 b = *reinterpret_cast<const bf16x2*>(reinterpret_cast<const bf16*>(g) + row * dk + c);
            x = make_float2((float)b[0], (float)b[1]);
        } else {
            x = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(g) + row * dk + c);
        }
        if (mode & MODE_GATE_SOFTPLUS) { x.x = neg_softplus(x.x); x.y = neg_softplus(x.y); }
        return x;
    }
    if (layout == 1) { const float x = gate_load(g, mode, row); return make_float2(x, x); }
    return make_float2(0.f, 0.f);
}

// The log-gates of N rows (row indices rows[i]) at channels c, c + 1 (c even),
// decided once for the mode so that every load is issued before any is used.
template <int N>
__device__ inline void gate_pair_rows(const void* __restrict__ g, int mode, const long* rows, int dk, int c,
                                      float2* out) {
    const int layout = gate_layout(mode);
    if (layout == 0 && (mode & MODE_GATE_BF16)) {
        const bf16* gb = reinterpret_cast<const bf16*>(g);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const bf16x2 b = *reinterpret_cast<const bf16x2*>(gb + rows[i] * dk + c);
            out[i] = make_float2((float)b[0], (float)b[1]);
        }
    } else if (layout == 0) {
        const float* gf = reinterpret_cast<const float*>(g);
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = *reinterpret_cast<const float2*>(gf + rows[i] * dk + c);
    } else if (layout == 1 && (mode & MODE_GATE_BF16)) {
        const bf16* gb = reinterpret_cast<const bf16*>(g);
#pragma unroll
        for (int i = 0; i < N; ++i) { const float x = (float)gb[rows[i]]; out[i] = make_float2(x, x); }
    } else if (layout == 1) {
        const float* gf = reinterpret_cast<const float*>(g);
#pragma unroll
        for (int i = 0; i < N; ++i) { const float x = gf[rows[i]]; out[i] = make_float2(x, x); }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = make_float2(0.f, 0.f);
    }
    if (mode & MODE_GATE_SOFTPLUS) {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = make_float2(neg_softplus(out[i].x), neg_softplus(out[i].y));
    }
}

// 1 / ||x|| from the sum of squares, with a zero row mapped to zero.
__device__ inline float inv_norm(float sumsq) { return sumsq > 0.f ? rsqrtf(sumsq) : 0.f; }

}  // namespace kda
