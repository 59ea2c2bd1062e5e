// kda_launch.h -- host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// Layout of the log-gate g (same values as kda_gate_layout_t in kda.h).
enum GateLayout : int {
    GATE_CHANNEL = 0,   // g[row * dk + c]: one gate per key channel
    GATE_HEAD = 1,      // g[row]: one gate per token and head, shared by all channels
    GATE_NONE = 2       // no decay (alpha = 1); g is not read
};

struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    float* state; void* o;
    int N, H, dk, dv;
    int T;              // tokens per sequence (1 for a single step)
    bool in_bf16, out_bf16;
    int gate;
    hipStream_t stream;
    int pre = 0;        // pre-processing flags (MODE_* in kda_common.h)
};

struct ChunkArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const float* s0; void* o; float* sT;
    int B, T, H, dk, dv, C;
    bool in_bf16, out_bf16;
    int gate;
    void* ws; size_t ws_bytes;
    hipStream_t stream;
    int pre = 0;        // pre-processing flags (MODE_* in kda_common.h): intra stage only
    // packed variable-length batch: B = 1, T = total tokens, N sequences with
    // token offsets cu_seqlens[N+1] (device memory); NULL for [B,T,H,d] batches
    const int* cu_seqlens = nullptr;
    int N = 0;
    // backward pass only: the stages also keep fp32 checkpoints (below), and the
    // chain runs without segments
    bool checkpoints = false;
    float* ck_state = nullptr;   // chain: state at each chunk start, [unit][dk][dv]
    float* ck_w = nullptr;       // chain: W of each chunk, [unit][C][dv]
    float* ck_t = nullptr;       // intra: T = (I + Diag(beta) A)^-1, [unit][C][C]
    float* ck_a = nullptr;       // intra: A (strictly lower), [unit][C][C]
    // (of T and A only the 16x16 blocks on and below the diagonal are read; the
    // hot intra kernel does not write the others)
};

// The hot configuration (bf16 inputs, C = 64, dk = 128) has its own pair of
// kernels and its own workspace format: contents in MFMA fragment order, U in bf16.
inline bool hot_config(bool in_bf16, int dk, int C) { return in_bf16 && dk == 128 && C == 64; }

// Workspace of the split chunk path: struct of arrays, each indexed by the
// chunk-major unit id n * (B*H) + (b*H + h); per unit
//   Qt [C][dk] in, Wk [C][dk] in, Kb^T [dk][C] in, P [C][C] in, U [C][dv], gam [dk] fp32
// with U in fp32, except in the hot configuration (bf16)
// Fixed-length batches whose chain would run on too few workgroups (long
// sequences, few heads) in the hot configuration also hold, per (sequence,
// head) pair and segment, the segment-affine chain's E, M and start states
// (fp32 [DK][DV], [DK][DK], [DK][DV]); seg_* are 0-sized otherwise.
struct WsLayout {
    size_t cu, qt, wk, kb, p, u, gam, seg_e, seg_m, seg_s, total;   // byte offsets of each array, total bytes
};
// Segments of the hot chain per (sequence, head): segment 0 of L0 chunks, then
// nseg - 1 segments of L chunks (the last may have fewer); nseg = 1 is the plain
// sequential chain.
struct SegPlan {
    int L, nseg, L0;
};
SegPlan seg_plan(int B, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints);
constexpr int SEG_DVS = 128;         // value columns per workgroup of the segmented chain
constexpr int SEG_TARGET_WG = 256;   // segments enough for this many workgroups per launch
constexpr int SEG_MIN_CHUNKS = 32;   // no segment after the first shorter than this
constexpr int SEG_MIN_LATER = 4;     // fewer segments after the first: the plain chain is faster
// checkpoints = true: the backward pass's layout (no segment arrays)
WsLayout ws_layout(int B, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints = false);
// Packed variable-length batch of N sequences, T tokens in all: room for every
// possible chunk (at most ceil(T/C) + N) and, first, the chunk offsets int [N+1].
WsLayout ws_layout_packed(int N, int T, int H, int dk, int dv, bool in_bf16, int C, bool checkpoints = false);
// The layout for a call's arguments (fixed-length or packed).
WsLayout ws_layout_of(const ChunkArgs& a);
SegPlan seg_plan_of(const ChunkArgs& a);

// True when an instantiation exists for these sizes (dk, dv, C, dtype).
bool chunk_supported(int dk, int dv, int C, bool in_bf16);

// Backward pass (kda_chunk_bwd.hip).  fwd: the forward arguments with
// checkpoints = true and the four checkpoint arrays; the rest is the backward's.
struct BwdArgs {
    ChunkArgs fwd;
    const float* dO;            // [B,T,H,dv] cotangent of o
    const float* dST;           // [B,H,dk,dv] cotangent of the final state, or NULL
    float *dq, *dk, *dv;        // [B,T,H,dk], [B,T,H,dk], [B,T,H,dv]
    float* dg;                  // [B,T,H,dk] / [B,T,H] by gate layout, NULL without gates
    float* dbeta;               // [B,T,H]
    float* dS0;                 // [B,H,dk,dv] or NULL
    float* ck_dS;               // cotangent of each chunk's end state, [unit][dk][dv]
    float* ck_dW;               // dW of each chunk, [unit][C][dv]
};
// Workspace of the backward pass: the forward workspace then the checkpoints,
// per unit.
struct BwdLayout {
    WsLayout fwd;
    size_t t, a, state, w, dS, dW, total;
};
BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, bool in_bf16, int C);
// Packed variable-length batch of N sequences, T tokens in all (units as ws_layout_packed).
BwdLayout bwd_layout_packed(int N, int T, int H, int dk, int dv, bool in_bf16, int C);
bool bwd_supported(int dk, int dv, int C, bool in_bf16);
hipError_t run_chunk_bwd_stages(const BwdArgs& b);

// Backward pass through the fused pre-processing (kda_pre_bwd.hip).  mode: the
// MODE_* bits of kda_common.h.  The inputs pass writes the pre-processed q, k
// (input dtype) and log-gate (fp32) to the workspace; the grads pass turns the
// gradients of those into gradients of the raw q, k and gate tensor, in place.
struct PreBwdArgs {
    const void *q, *k, *g;       // raw inputs, [rows][dk] (g by gate layout, fp32 or bf16 by mode)
    void *qn, *kn;               // [rows][dk] input dtype (L2-normalised), or unused
    float* g_act;                // [rows][dk] / [rows] fp32 log-gate, or unused
    float* inv;                  // [2][rows]: 1/|q row|, 1/|k row| (0 for a zero row)
    float *dq, *dk, *dg;         // gradients, updated in place
    long rows;                   // token-heads
    int dk_size;
    bool in_bf16;
    int gate, mode;
    hipStream_t stream;
};
hipError_t run_pre_bwd_inputs(const PreBwdArgs& p);
hipError_t run_pre_bwd_grads(const PreBwdArgs& p);

hipError_t run_decode_step(const DecodeArgs& a);
// Threads per decode workgroup for T tokens per call (one workgroup per
// (sequence, head)), as measured: 1024 for one token, 512 for two, 256 from three on.
inline int decode_block_threads(int T) { return T == 1 ? 1024 : (T == 2 ? 512 : 256); }
hipError_t run_chunk_intra(const ChunkArgs& a);
hipError_t run_chunk_chain(const ChunkArgs& a);

}  // namespace kda
