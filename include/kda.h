/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) / gated delta-rule
 * state update on AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   Per (batch b, head h) a d_k x d_v state S is kept; key channels index rows,
 *   value channels index columns.  For each token t, in the order given in
 *   section 八 of "我终于看懂了 KDA：百万 Token 的关键，不是记得更多，而是会修改记忆":
 *     decay   S' = Diag(alpha_t) S, alpha_t = exp(g_t) per key channel
 *             (per-channel gate: Kimi Linear paragraph of
 *             "一个KimiK3装下22580个GPT-2，七年缩放真正改变的是记忆与检索");
 *     read    r  = S'^T k_t                 (delta rule: section 六 of the
 *     error   u  = beta_t (v_t - r)          explainer and the delta-rule
 *     write   S  = S' + k_t u^T              paragraph of the KimiK3 essay)
 *     output  o_t = S^T q_t                 (read after the token's own write)
 *   kda_chunk_fwd evaluates this over a whole sequence with the chunkwise form
 *   (chunk paragraph of the KimiK3 essay; sections 十六 and 十七 of the
 *   explainer: recurrence between chunks, parallel work inside a chunk, the
 *   chunk's rank-1 updates folded into matrix products).  kda_decode_step is the
 *   single-token step of section 十五 (read state, compute output, update state).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     keeps no pointer after the call returns and allocates nothing.
 *   - Layouts are contiguous row-major.  Sequence tensors are [B,T,H,d];
 *     states are [B,H,dk,dv] with dv fastest.
 *   - q, k, v have dtype in_dtype; o has dtype out_dtype; g, beta and every
 *     state are fp32.  g is the log-gate: g <= 0, -inf allowed (alpha = 0).
 *     g > 0 (alpha > 1) is outside the method's domain; results are unspecified.
 *     NaN/Inf inputs propagate; nothing is checked on the device.
 *   - Supported: dk, dv in {64, 128}; chunk size C in {16, 32, 64, 128}; any
 *     T >= 0 (a last partial chunk is allowed); B, H >= 0.  The chunkwise form
 *     gives the recurrence's result for every C, so C only groups the work
 *     (kda_chunk_size_used reports the chunk the kernels run).  C = 128 runs as
 *     64-token chunks for fp32 inputs (the 128 x 128 fp32 blocks exceed the
 *     160 KB of LDS a workgroup has), for bf16 inputs with dk = 128 (the 64-token
 *     kernels move fewer bytes per token) and in the backward pass.
 *   - Alignment: kda_chunk_fwd needs q, k, v, o, the workspace and a
 *     per-channel g 16-byte aligned (true of any [..., dk] row of a tensor whose
 *     storage is 16-byte aligned); kda_decode_step needs the state 16-byte
 *     aligned; every other pointer needs the alignment of its element type.
 *   - Validation happens on the host before any HIP call; on error nothing is
 *     launched and nothing is written.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; the return value only reports validation and launch
 *     errors.  Setting KDA_DEBUG_SYNC=1 in the environment makes each call
 *     synchronise the stream and report execution errors too.
 *   - Stateless and re-entrant; concurrent calls on different streams with
 *     disjoint outputs and workspaces are safe.  Identical inputs give
 *     bitwise-identical outputs (no floating-point atomics).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/*
 * Layout of the log-gate g, for the _ex entry points.  The plain entry points
 * use KDA_GATE_CHANNEL.
 *   KDA_GATE_CHANNEL  g holds one gate per key channel: [..., dk] fp32.  This is
 *                     Kimi Delta Attention's fine-grained gate (Kimi Linear
 *                     paragraph of the KimiK3 essay; section 九 of the explainer).
 *   KDA_GATE_HEAD     g holds one gate per token and head, [...] fp32 without
 *                     the channel axis, applied to every channel: the scalar
 *                     decay of Gated DeltaNet (Gated DeltaNet paragraph of the
 *                     KimiK3 essay).
 *   KDA_GATE_NONE     no decay, alpha = 1: the plain delta rule (DeltaNet); g is
 *                     not read and may be NULL.
 */
typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1, KDA_GATE_NONE = 2 } kda_gate_layout_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                       */
    KDA_ERR_SHAPE = 2,       /* a size is negative or inconsistent               */
    KDA_ERR_UNSUPPORTED = 3, /* dk, dv, C or a dtype outside the supported set   */
    KDA_ERR_MISALIGNED = 4,  /* a pointer lacks the alignment it needs          */
    KDA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
    KDA_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap   */
    KDA_ERR_HIP = 7          /* no usable device, or a HIP launch/execution error */
} kda_status_t;

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *kda_status_string(int status);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if the
 * sizes are unsupported).  Host-only; never touches the device. */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv,
                                     int in_dtype, int C);

/*
 * Segments the chain stage of kda_chunk_fwd / kda_chunk_fwd_ex runs each
 * sequence in, for these sizes (0 if unsupported); host-only.  The recurrence
 * across chunks is serial (section 十五 of the explainer: one step at a time);
 * when B*H is too small to fill the GPU and T is long, each sequence is cut
 * into segments: the first runs from the initial state while the affine state
 * maps S -> M S + E of the others are computed side by side; the maps are
 * composed in order, and every later segment then runs from its true start
 * state.
 * 1 means the plain sequential chain.  The result equals the sequential chain
 * up to rounding; the workspace (kda_chunk_fwd_workspace_bytes) includes the
 * segments' maps and start states.
 */
int kda_chunk_fwd_segments(int B, int T, int H, int dk, int dv, int in_dtype, int C);

/*
 * The chunk size the kernels run for a requested C (forward: backward = 0;
 * kda_chunk_bwd: backward = 1), or 0 for unsupported sizes; host-only.  The
 * chunk paragraph of the KimiK3 essay has the chunk size fitted to the matrix
 * units, and section 十八 of the explainer lists a chunk size suited to the
 * target GPU among what decides a kernel's speed: C = 128 is computed as
 * 64-token chunks where that is what fits gfx950 (see the supported sizes
 * above).  Results differ only by rounding.
 */
int kda_chunk_size_used(int dk, int dv, int in_dtype, int C, int backward);

/*
 * kda_chunk_fwd -- chunkwise-parallel forward over a whole sequence.
 *   q, k          [B,T,H,dk] in_dtype         queries, keys (not normalised here)
 *   v             [B,T,H,dv] in_dtype         values
 *   g             [B,T,H,dk] fp32             log-gate per key channel
 *   beta          [B,T,H]    fp32             write strength (learning rate)
 *   initial_state [B,H,dk,dv] fp32 or NULL    NULL means zeros
 *   o             [B,T,H,dv] out_dtype        outputs o_t = S_t^T q_t
 *   final_state   [B,H,dk,dv] fp32 or NULL    state after token T-1; may be the
 *                                             same pointer as initial_state
 *                                             (updated in place)
 *   workspace     device buffer of >= kda_chunk_fwd_workspace_bytes(...) bytes
 *   C             chunk size (tokens per chunk)
 * o must not overlap any other argument; final_state may equal initial_state
 * but not partially overlap it or any other argument.
 * Intermediate values use bf16 MFMA operands with fp32 accumulation when
 * in_dtype is BF16, fp32 MFMA operands when in_dtype is F32; the state is
 * carried in fp32.  Log-gates below -20 are treated as -20 (alpha >= 2e-9).
 * A call of 2^31 or more (chunk, head) units, B * ceil(T/C) * H (packed
 * batches: (ceil(T/C) + N) * H, with C the chunk that runs), returns
 * KDA_ERR_SHAPE; the kernels index units with 32-bit arithmetic.  The same
 * limit holds for every kda_chunk_* call, the backward ones included.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta,
                  const float *initial_state,
                  void *o, float *final_state,
                  int B, int T, int H, int dk, int dv,
                  int in_dtype, int out_dtype,
                  void *workspace, size_t workspace_bytes,
                  void *stream, int C);

/*
 * The two stages kda_chunk_fwd runs, exposed so that callers can schedule or
 * time them separately.  Same arguments and rules as kda_chunk_fwd.
 *   kda_chunk_intra: everything that does not depend on the carried state
 *     (gate prefix sums, decayed operands, the intra-chunk score matrices and
 *     the triangular solve), for all chunks in parallel, into the workspace.
 *     Reads q, k, v, g, beta; writes only the workspace.
 *   kda_chunk_chain: the sequential state recurrence across chunks and the
 *     outputs.  Reads the workspace and initial_state; writes o and final_state.
 *     It does not read g, which may be NULL.
 * kda_chunk_chain must run after kda_chunk_intra on the same workspace with the
 * same sizes (stream order suffices).
 */
int kda_chunk_intra(const void *q, const void *k, const void *v,
                    const float *g, const float *beta,
                    const float *initial_state,
                    void *o, float *final_state,
                    int B, int T, int H, int dk, int dv,
                    int in_dtype, int out_dtype,
                    void *workspace, size_t workspace_bytes,
                    void *stream, int C);
int kda_chunk_chain(const void *q, const void *k, const void *v,
                    const float *g, const float *beta,
                    const float *initial_state,
                    void *o, float *final_state,
                    int B, int T, int H, int dk, int dv,
                    int in_dtype, int out_dtype,
                    void *workspace, size_t workspace_bytes,
                    void *stream, int C);

/*
 * kda_chunk_fwd_ex, kda_chunk_intra_ex -- kda_chunk_fwd and kda_chunk_intra
 * with the gate layout as an argument (kda_gate_layout_t).  g is [B,T,H,dk] for
 * KDA_GATE_CHANNEL, [B,T,H] for KDA_GATE_HEAD (fp32, 4-byte aligned) and ignored
 * (NULL allowed) for KDA_GATE_NONE.  The chain stage, kda_chunk_chain, does not
 * read g and serves every layout.  An unknown layout returns KDA_ERR_UNSUPPORTED.
 */
int kda_chunk_fwd_ex(const void *q, const void *k, const void *v,
                     const float *g, const float *beta,
                     const float *initial_state,
                     void *o, float *final_state,
                     int B, int T, int H, int dk, int dv,
                     int in_dtype, int out_dtype,
                     void *workspace, size_t workspace_bytes,
                     void *stream, int C, int gate_layout);
int kda_chunk_intra_ex(const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *initial_state,
                       void *o, float *final_state,
                       int B, int T, int H, int dk, int dv,
                       int in_dtype, int out_dtype,
                       void *workspace, size_t workspace_bytes,
                       void *stream, int C, int gate_layout);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd_ex without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  It allocates
 * nothing: its workspace is a static device array of
 * KDA_NOALLOC_WORKSPACE_MAX bytes inside the library, one per GPU, held until
 * the process ends.  Sizes whose workspace (kda_chunk_fwd_workspace_bytes)
 * exceeds it return KDA_ERR_WORKSPACE before any HIP call; at d = 128 and
 * C = 64 that is about 1,800 (batch, head, chunk) units, e.g. 16 heads of
 * 7,000 tokens.  The work runs on the current device, and `stream` must belong
 * to it.  Nothing in the array needs to start at zero (every call writes what it
 * reads), but every call on a GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams, other host threads) race and give undefined
 * results; calls ordered on one stream are safe.  Arguments, results and
 * errors otherwise as kda_chunk_fwd_ex, bitwise the same results.
 */
#define KDA_NOALLOC_WORKSPACE_MAX ((size_t)128 << 20)
int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *initial_state,
                          void *o, float *final_state,
                          int B, int T, int H, int dk, int dv,
                          int in_dtype, int out_dtype,
                          void *stream, int C, int gate_layout);

/*
 * kda_chunk_fwd_varlen -- kda_chunk_fwd_ex over a packed batch of N sequences
 * of different lengths (the chunkwise form of the chunk paragraph of the KimiK3
 * essay and section 十六 of the explainer, applied to each sequence on its own:
 * no chunk spans two sequences, and each sequence starts from its own state).
 *   q, k          [T,H,dk] in_dtype   the N sequences one after another
 *   v             [T,H,dv] in_dtype
 *   g             [T,H,dk] / [T,H] fp32 or ignored, by gate_layout
 *   beta          [T,H]    fp32
 *   cu_seqlens    [N+1]    int32, DEVICE memory: sequence s is tokens
 *                          cu_seqlens[s] .. cu_seqlens[s+1]-1; cu_seqlens[0] = 0,
 *                          non-decreasing, cu_seqlens[N] = T.  Other values give
 *                          unspecified results but every access stays in bounds:
 *                          on the device each offset becomes the running maximum
 *                          of the offsets so far, clamped to [0, T], so sequences
 *                          never overlap.
 *   initial_state [N,H,dk,dv] fp32 or NULL;  final_state [N,H,dk,dv] fp32 or NULL
 *   o             [T,H,dv] out_dtype
 *   workspace     >= kda_chunk_varlen_workspace_bytes(N, T, H, dk, dv, in_dtype, C)
 * Sequences of length 0 are allowed (their final state is their initial state).
 * The result for each sequence is bitwise the same as a kda_chunk_fwd_ex call on
 * that sequence alone.  Same rules as kda_chunk_fwd otherwise; cu_seqlens must
 * not overlap o or final_state.
 */
int kda_chunk_fwd_varlen(const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state,
                         void *o, float *final_state,
                         const int *cu_seqlens, int N, int T, int H, int dk, int dv,
                         int in_dtype, int out_dtype,
                         void *workspace, size_t workspace_bytes,
                         void *stream, int C, int gate_layout);

/* Bytes of device workspace kda_chunk_fwd_varlen needs (0 if unsupported);
 * host-only.  Depends on N and T only, not on the individual lengths. */
size_t kda_chunk_varlen_workspace_bytes(int N, int T, int H, int dk, int dv,
                                        int in_dtype, int C);

/*
 * kda_chunk_bwd -- the backward pass of kda_chunk_fwd_ex (training): for the
 * scalar L = sum(dO * o) + sum(dST * final_state) it returns the gradients of L
 * with respect to every input.  The chunkwise form is trained by the same
 * chunking (chunk paragraph of the KimiK3 essay; sections 十六 and 十七 of the
 * explainer): a recurrence over the chunks in reverse order carries the
 * cotangent of the state, and every chunk's gradients are then formed in
 * parallel.  The forward stages are run again inside the call.
 *   q, k, v, g, beta, initial_state   as for kda_chunk_fwd_ex (initial_state may be NULL)
 *   dO            [B,T,H,dv] fp32     cotangent of o
 *   dST           [B,H,dk,dv] fp32    cotangent of the final state, or NULL (zeros)
 *   dq, dk        [B,T,H,dk] fp32     outputs
 *   dv            [B,T,H,dv] fp32
 *   dg            [B,T,H,dk] / [B,T,H] fp32 by gate_layout (NULL allowed without gates);
 *                                    zero where the forward floored the log-gate
 *   dbeta         [B,T,H]    fp32
 *   dS0           [B,H,dk,dv] fp32 or NULL
 *   workspace     >= kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, in_dtype, C)
 * Supported: C in {16, 32, 64, 128} (C = 128 runs as 64-token chunks); dk, dv
 * in {64, 128}; in_dtype BF16 or F32.  Gradients accumulate in fp32; products of fp32
 * operands run on bf16 MFMA with each operand split into bf16 hi + lo parts (about
 * 16 significant bits, the lo x lo term dropped).  Outputs must not overlap any input, the
 * workspace or each other.  Alignment: q, k, v and the workspace 16 bytes,
 * per-channel g 16 bytes, everything else 4 bytes.  Deterministic (no
 * floating-point atomics).
 */
int kda_chunk_bwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta, const float *initial_state,
                  const float *dO, const float *dST,
                  float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                  int B, int T, int H, int dk_size, int dv_size, int in_dtype,
                  void *workspace, size_t workspace_bytes,
                  void *stream, int C, int gate_layout);

/* Bytes of device workspace kda_chunk_bwd needs (0 if unsupported); host-only. */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv,
                                     int in_dtype, int C);

/*
 * kda_chunk_bwd_varlen -- the backward pass of kda_chunk_fwd_varlen: kda_chunk_bwd
 * over a packed batch of N sequences of different lengths.  Each sequence is
 * differentiated on its own (no chunk spans two sequences; the reverse
 * recurrence over the chunks starts from each sequence's own dST and ends in its
 * own dS0), as in the chunkwise training form of the chunk paragraph of the
 * KimiK3 essay and sections 十六 and 十七 of the explainer.
 *   q, k, v, g, beta, initial_state, cu_seqlens   as for kda_chunk_fwd_varlen
 *   dO            [T,H,dv] fp32       cotangent of o
 *   dST           [N,H,dk,dv] fp32    cotangent of the final states, or NULL (zeros)
 *   dq, dk        [T,H,dk] fp32;  dv [T,H,dv] fp32;  dbeta [T,H] fp32
 *   dg            [T,H,dk] / [T,H] fp32 by gate_layout (NULL allowed without gates)
 *   dS0           [N,H,dk,dv] fp32 or NULL
 *   workspace     >= kda_chunk_bwd_varlen_workspace_bytes(N, T, H, dk, dv, in_dtype, C)
 * Tokens outside every sequence (cu_seqlens[N] < T) are not written.  The result
 * for each sequence equals a kda_chunk_bwd call on that sequence alone.  Same
 * rules as kda_chunk_bwd otherwise; cu_seqlens must not overlap an output or the
 * workspace.
 */
int kda_chunk_bwd_varlen(const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *initial_state,
                         const float *dO, const float *dST,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                         const int *cu_seqlens, int N, int T, int H, int dk_size, int dv_size,
                         int in_dtype, void *workspace, size_t workspace_bytes,
                         void *stream, int C, int gate_layout);

/* Bytes of device workspace kda_chunk_bwd_varlen needs (0 if unsupported);
 * host-only.  Depends on N and T only, not on the individual lengths. */
size_t kda_chunk_bwd_varlen_workspace_bytes(int N, int T, int H, int dk, int dv,
                                            int in_dtype, int C);

/*
 * kda_decode_step -- one token per sequence, state updated IN PLACE.
 *   q, k   [N,H,dk] in_dtype;  v [N,H,dv] in_dtype
 *   g      [N,H,dk] fp32 log-gate;  beta [N,H] fp32
 *   state  [N,H,dk,dv] fp32, read and overwritten with the new state
 *   o      [N,H,dv] out_dtype
 * Each state element is read once and written once.  o must not overlap any
 * other argument; state must not overlap the inputs.  One workgroup of 1024
 * threads runs per sequence and head (512 for two tokens per call, 256 for
 * more, in kda_decode_tokens); N*H beyond 2^32 - 1 work-items at that size
 * (4,194,303 pairs for one token) returns KDA_ERR_SHAPE.
 */
int kda_decode_step(const void *q, const void *k, const void *v,
                    const float *g, const float *beta,
                    float *state, void *o,
                    int N, int H, int dk, int dv,
                    int in_dtype, int out_dtype, void *stream);

/*
 * kda_decode_step_ex -- kda_decode_step with the gate layout as an argument:
 * g is [N,H,dk] (KDA_GATE_CHANNEL), [N,H] (KDA_GATE_HEAD) or ignored
 * (KDA_GATE_NONE, NULL allowed).
 */
int kda_decode_step_ex(const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       float *state, void *o,
                       int N, int H, int dk, int dv,
                       int in_dtype, int out_dtype, void *stream, int gate_layout);

/*
 * kda_decode_tokens -- T consecutive tokens per sequence in one call, the state
 * updated IN PLACE: the same result, bitwise, as T kda_decode_step_ex calls, with
 * the state read and written once instead of T times (a short prefill that
 * continues a decoded sequence, or several tokens accepted at once).
 *   q, k  [N,T,H,dk] in_dtype;  v [N,T,H,dv] in_dtype;  beta [N,T,H] fp32
 *   g     [N,T,H,dk] / [N,T,H] fp32 or ignored, by gate_layout
 *   state [N,H,dk,dv] fp32, read and overwritten;  o [N,T,H,dv] out_dtype
 * T = 0 leaves the state unchanged.  Same rules as kda_decode_step otherwise.
 */
int kda_decode_tokens(const void *q, const void *k, const void *v,
                      const float *g, const float *beta,
                      float *state, void *o,
                      int N, int T, int H, int dk, int dv,
                      int in_dtype, int out_dtype, void *stream, int gate_layout);

/*
 * Fused pre-processing (the steps that produce the path's inputs in the recipe
 * of the method's workloads: q and k L2-normalised per token and head, the
 * log-gate g = -softplus(a) of a pre-activation a).  Flags, OR-ed together:
 *   KDA_PRE_QK_L2NORM      q and k are raw; each [dk] row is divided by its L2
 *                          norm inside the kernels (a zero row stays zero)
 *   KDA_PRE_GATE_SOFTPLUS  g holds a, and the log-gate is -softplus(a) =
 *                          -log(1 + e^a) (alpha = sigmoid(-a) in (0, 1))
 *   KDA_PRE_GATE_BF16      g (log-gate or a) is bf16 instead of fp32; a per-channel
 *                          bf16 g must be 16-byte aligned, a per-head one 2-byte
 * The normalised q, k and the activated gate exist only inside the kernels; the
 * result equals the plain call on the pre-processed inputs up to rounding.
 * Unknown flag bits return KDA_ERR_UNSUPPORTED.  kda_chunk_bwd takes
 * pre-processed inputs; kda_chunk_bwd_pre differentiates through the flags.
 */
typedef enum {
    KDA_PRE_NONE = 0,
    KDA_PRE_QK_L2NORM = 1,
    KDA_PRE_GATE_SOFTPLUS = 2,
    KDA_PRE_GATE_BF16 = 4
} kda_pre_flags_t;

/*
 * kda_chunk_fwd_pre, kda_chunk_intra_pre -- kda_chunk_fwd_ex / kda_chunk_intra_ex
 * with pre-processing flags (kda_pre_flags_t).  g points to fp32 or bf16 data by
 * KDA_PRE_GATE_BF16.  The chain stage (kda_chunk_chain) reads none of q, k, g
 * and serves these calls unchanged.  Arguments and errors as kda_chunk_fwd_ex.
 */
int kda_chunk_fwd_pre(const void *q, const void *k, const void *v,
                      const void *g, const float *beta,
                      const float *initial_state,
                      void *o, float *final_state,
                      int B, int T, int H, int dk, int dv,
                      int in_dtype, int out_dtype,
                      void *workspace, size_t workspace_bytes,
                      void *stream, int C, int gate_layout, int pre_flags);
int kda_chunk_intra_pre(const void *q, const void *k, const void *v,
                        const void *g, const float *beta,
                        const float *initial_state,
                        void *o, float *final_state,
                        int B, int T, int H, int dk, int dv,
                        int in_dtype, int out_dtype,
                        void *workspace, size_t workspace_bytes,
                        void *stream, int C, int gate_layout, int pre_flags);

/*
 * kda_decode_tokens_pre -- kda_decode_tokens with pre-processing flags; T = 1 is
 * the single decode step.  Arguments and errors as kda_decode_tokens.
 */
int kda_decode_tokens_pre(const void *q, const void *k, const void *v,
                          const void *g, const float *beta,
                          float *state, void *o,
                          int N, int T, int H, int dk, int dv,
                          int in_dtype, int out_dtype, void *stream,
                          int gate_layout, int pre_flags);

/*
 * kda_chunk_bwd_pre -- kda_chunk_bwd with pre-processing flags: the backward
 * pass of kda_chunk_fwd_pre.  The gradients are those of the raw inputs: dq and
 * dk of the rows before L2 normalisation (KDA_PRE_QK_L2NORM), dg of the gate
 * tensor as given, i.e. of the pre-activation a under KDA_PRE_GATE_SOFTPLUS
 * (dg is fp32 whatever the gate tensor's storage).  The pre-processed q, k and
 * log-gate are formed in the workspace, the backward stages run on them, and
 * the chain rule of the two steps is applied to the gradients in place:
 *   y = x/|x|:         dx = (dy - y (y . dy)) / |x|    (a zero row gets zero)
 *   g = -softplus(a):  da = -dg * sigmoid(a)
 *   workspace  >= kda_chunk_bwd_pre_workspace_bytes(B, T, H, dk, dv, in_dtype, C,
 *                                                   gate_layout, pre_flags)
 * A gate tensor that the flags transform needs only its element's alignment.
 * Arguments and errors as kda_chunk_bwd and kda_chunk_fwd_pre otherwise.
 */
int kda_chunk_bwd_pre(const void *q, const void *k, const void *v,
                      const void *g, const float *beta, const float *initial_state,
                      const float *dO, const float *dST,
                      float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                      int B, int T, int H, int dk_size, int dv_size, int in_dtype,
                      void *workspace, size_t workspace_bytes,
                      void *stream, int C, int gate_layout, int pre_flags);

/* Bytes of device workspace kda_chunk_bwd_pre needs (0 if unsupported); host-only. */
size_t kda_chunk_bwd_pre_workspace_bytes(int B, int T, int H, int dk, int dv,
                                         int in_dtype, int C, int gate_layout,
                                         int pre_flags);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
