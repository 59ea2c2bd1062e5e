// kda_api.cpp -- the C ABI of libkda: argument validation (host only, before any
// HIP call), dispatch to the kernels, status codes.  See include/kda.h.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kda_common.h"
#include "kda_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;                 // [lo, hi); empty when lo == hi
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return Range{a, p ? a + bytes : a};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool debug_sync() {
    static const bool on = [] {                       // read once, thread-safe initialisation
        const char* e = getenv("KDA_DEBUG_SYNC");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

int device_ready() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int finish(hipError_t e, hipStream_t s) {
    if (e != hipSuccess) return KDA_ERR_HIP;
    if (debug_sync()) {
        if (hipStreamSynchronize(s) != hipSuccess) return KDA_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

struct ChunkCall {
    const void *q, *k, *v;
    const float *g, *beta, *s0;
    void* o;
    float* sT;
    int B, T, H, dk, dv, in_dtype, out_dtype;
    void* ws;
    size_t ws_bytes;
    void* stream;
    int C;
    int gate;
    const int* cu_seqlens = nullptr;   // packed variable-length batch (B = 1, N sequences)
    int N = 0;
    bool packed = false;
    int pre = 0;                       // kda_pre_flags_t
    bool static_ws = false;            // workspace: the library's static device array (ws is ignored)
};

bool gate_ok(int g) { return g == KDA_GATE_CHANNEL || g == KDA_GATE_HEAD || g == KDA_GATE_NONE; }
constexpr int PRE_ALL = KDA_PRE_QK_L2NORM | KDA_PRE_GATE_SOFTPLUS | KDA_PRE_GATE_BF16;
bool pre_ok(int pre) { return (pre & ~PRE_ALL) == 0; }
// bytes of g per token-head for a gate layout (bf16 gates: half)
size_t gate_bytes(int gate, int dk, int pre = 0) {
    const size_t e = (pre & KDA_PRE_GATE_BF16) ? 2 : 4;
    return gate == KDA_GATE_CHANNEL ? (size_t)dk * e : gate == KDA_GATE_HEAD ? e : 0;
}
// the kernels' mode bits for the ABI's pre-processing flags
int pre_mode(int pre) {
    return ((pre & KDA_PRE_QK_L2NORM) ? kda::MODE_QK_L2NORM : 0) |
           ((pre & KDA_PRE_GATE_SOFTPLUS) ? kda::MODE_GATE_SOFTPLUS : 0) |
           ((pre & KDA_PRE_GATE_BF16) ? kda::MODE_GATE_BF16 : 0);
}

bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }
size_t esize(int d) { return d == KDA_BF16 ? 2 : 4; }

// The chunk the kernels run for a requested chunk size.  The chunkwise form
// gives the recurrence's result for every C (only rounding differs), so C is a
// grouping choice.  C = 128 runs as 64-token chunks: with fp32 inputs (the
// 128 x 128 fp32 blocks of both stages exceed the 160 KB of LDS), with bf16
// inputs and dk = 128 (the C = 64 kernels, built for the gfx950 matrix cores,
// move fewer bytes per token: P grows with C, and the segmented chain removes
// the serial length that a longer chunk would shorten), and in the backward
// pass (its per-chunk kernel holds 158 KB of LDS at C = 64).
int fwd_chunk(int C, int dk, int in_dtype) { return C == 128 && (in_dtype != KDA_BF16 || dk == 128) ? 64 : C; }
int bwd_chunk(int C) { return C == 128 ? 64 : C; }

// (chunk, head) units of a call: the kernels index them with 32-bit arithmetic,
// so a call has fewer than 2^31 of them (72.5 KB of workspace each at d = 128,
// far beyond any device's memory well before that)
bool units_ok(bool packed, int B, int N, int T, int H, int C) {
    const size_t nc = ((size_t)T + C - 1) / C;
    const size_t units = (packed ? nc + (size_t)N : (size_t)B * nc) * (size_t)H;
    return units < (size_t(1) << 31);
}

int validate_chunk(const ChunkCall& c) {
    if (c.B < 0 || c.T < 0 || c.H < 0 || c.N < 0) return KDA_ERR_SHAPE;
    if (!dtype_ok(c.in_dtype) || !dtype_ok(c.out_dtype) || !gate_ok(c.gate) || !pre_ok(c.pre))
        return KDA_ERR_UNSUPPORTED;
    if ((c.dk != 64 && c.dk != 128) || (c.dv != 64 && c.dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (c.C != 16 && c.C != 32 && c.C != 64 && c.C != 128) return KDA_ERR_UNSUPPORTED;
    if (!kda::chunk_supported(c.dk, c.dv, c.C, c.in_dtype == KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if (!units_ok(c.packed, c.B, c.N, c.T, c.H, c.C)) return KDA_ERR_SHAPE;

    // token rows: [B,T,H] (fixed-length) or [T,H] (packed); states: [B,H] or [N,H]
    const size_t tok = (size_t)(c.packed ? 1 : c.B) * c.T * c.H;
    const size_t nst = (size_t)(c.packed ? c.N : c.B) * c.H * c.dk * c.dv;
    if (c.packed && c.N > 0 && c.H > 0 && !c.cu_seqlens) return KDA_ERR_NULL;
    if (c.packed && c.cu_seqlens && !aligned(c.cu_seqlens, 4)) return KDA_ERR_MISALIGNED;
    const bool need_g = c.gate != KDA_GATE_NONE;
    if (tok > 0 && (!c.q || !c.k || !c.v || (need_g && !c.g) || !c.beta || !c.o)) return KDA_ERR_NULL;
    const float* g = need_g ? c.g : nullptr;            // g is not read without gates

    // q, k, v, o, the workspace and a per-channel g move in 16-byte vectors (the
    // C = 64 intra kernel reads four fp32 or eight bf16 gates at once); per-head g,
    // beta and the states only need their element's alignment.
    const void* p16[5] = {c.q, c.k, c.v, c.o, c.ws};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    if (g && !aligned(g, c.gate == KDA_GATE_CHANNEL ? 16 : ((c.pre & KDA_PRE_GATE_BF16) ? 2 : 4)))
        return KDA_ERR_MISALIGNED;
    const void* p4[3] = {c.beta, c.s0, c.sT};
    for (const void* p : p4)
        if (p && !aligned(p, 4)) return KDA_ERR_MISALIGNED;

    const size_t need = c.packed ? kda::ws_layout_packed(c.N, c.T, c.H, c.dk, c.dv, c.in_dtype == KDA_BF16, c.C).total
                                 : kda::ws_layout(c.B, c.T, c.H, c.dk, c.dv, c.in_dtype == KDA_BF16, c.C).total;
    const bool uses_ws = c.packed ? (size_t)c.N * c.H > 0 : tok > 0;
    if (c.static_ws) {
        // the library's own array: nothing of the caller's can overlap it
        if (uses_ws && need > KDA_NOALLOC_WORKSPACE_MAX) return KDA_ERR_WORKSPACE;
    } else if (uses_ws && (!c.ws || c.ws_bytes < need)) {
        return KDA_ERR_WORKSPACE;
    }

    const size_t ei = esize(c.in_dtype), eo = esize(c.out_dtype);
    const Range rq = range_of(c.q, tok * c.dk * ei), rk = range_of(c.k, tok * c.dk * ei),
                rv = range_of(c.v, tok * c.dv * ei), rg = range_of(g, tok * gate_bytes(c.gate, c.dk, c.pre)),
                rb = range_of(c.beta, tok * 4), rs0 = range_of(c.s0, nst * 4),
                ro = range_of(c.o, tok * c.dv * eo), rsT = range_of(c.sT, nst * 4),
                rw = range_of(c.static_ws ? nullptr : c.ws, uses_ws ? need : 0),
                rcu = range_of(c.packed ? c.cu_seqlens : nullptr, ((size_t)c.N + 1) * 4);
    const Range others_o[] = {rq, rk, rv, rg, rb, rs0, rsT, rw, rcu};
    for (const Range& r : others_o)
        if (overlap(ro, r)) return KDA_ERR_ALIAS;
    const Range others_s[] = {rq, rk, rv, rg, rb, rw, rcu};
    for (const Range& r : others_s)
        if (overlap(rsT, r)) return KDA_ERR_ALIAS;
    if (c.sT && c.s0 && c.sT != c.s0 && overlap(rsT, rs0)) return KDA_ERR_ALIAS;
    const Range others_w[] = {rq, rk, rv, rg, rb, rs0, rcu};
    for (const Range& r : others_w)
        if (overlap(rw, r)) return KDA_ERR_ALIAS;
    return KDA_OK;
}

kda::ChunkArgs to_args(const ChunkCall& c) {
    kda::ChunkArgs a;
    a.q = c.q; a.k = c.k; a.v = c.v; a.g = c.gate == KDA_GATE_NONE ? nullptr : c.g; a.beta = c.beta;
    a.gate = c.gate;
    a.pre = pre_mode(c.pre);
    a.s0 = c.s0; a.o = c.o; a.sT = c.sT;
    a.B = c.packed ? 1 : c.B; a.T = c.T; a.H = c.H; a.dk = c.dk; a.dv = c.dv; a.C = c.C;
    a.cu_seqlens = c.packed ? c.cu_seqlens : nullptr;
    a.N = c.packed ? c.N : 0;
    a.in_bf16 = c.in_dtype == KDA_BF16; a.out_bf16 = c.out_dtype == KDA_BF16;
    a.ws = c.ws; a.ws_bytes = c.ws_bytes;
    a.stream = (hipStream_t)c.stream;
    return a;
}

enum Stages { STAGE_INTRA = 1, STAGE_CHAIN = 2 };

}  // namespace

// Workspace of kda_chunk_fwd_noalloc: one array per device, held until the
// process ends.  Host code uses only the device address hipGetSymbolAddress
// returns for the current device (the name alone is a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_WORKSPACE_MAX];

namespace {

constexpr int MAX_DEVICES = 64;

// The current device's address of `scratch`, looked up once per device with
// that device current; NULL on failure.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[MAX_DEVICES] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

int run_chunk(ChunkCall c, int stages) {
    c.C = fwd_chunk(c.C, c.dk, c.in_dtype);
    int st = validate_chunk(c);
    if (st != KDA_OK) return st;
    const long nseqh = (long)(c.packed ? c.N : c.B) * c.H;
    const long nstate = nseqh * c.dk * c.dv;
    if (nseqh == 0) return KDA_OK;                      // nothing to do: no device needed
    st = device_ready();
    if (st != KDA_OK) return st;
    if (c.static_ws) {
        c.ws = scratch_address();
        c.ws_bytes = KDA_NOALLOC_WORKSPACE_MAX;
        if (!c.ws) return KDA_ERR_HIP;
    }
    const kda::ChunkArgs a = to_args(c);
    if (c.T == 0) {
        // Empty sequence: the final state is the initial state (or zeros).
        if ((stages & STAGE_CHAIN) && c.sT && c.sT != c.s0) {
            hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0,
                               a.stream, c.s0, c.sT, nstate);
            return finish(hipGetLastError(), a.stream);
        }
        return KDA_OK;
    }
    if (stages & STAGE_INTRA) {
        hipError_t e = kda::run_chunk_intra(a);
        if (e != hipSuccess) return KDA_ERR_HIP;
    }
    if (stages & STAGE_CHAIN) {
        hipError_t e = kda::run_chunk_chain(a);
        if (e != hipSuccess) return KDA_ERR_HIP;
    }
    return finish(hipSuccess, a.stream);
}

struct BwdCall {
    const void *q, *k, *v, *g;
    const float *beta, *s0, *dO, *dST;
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    int B, T, H, dk_size, dv_size, in_dtype;
    void* ws;
    size_t ws_bytes;
    void* stream;
    int C, gate;
    const int* cu_seqlens = nullptr;   // packed variable-length batch (B = 1, N sequences)
    int N = 0;
    bool packed = false;
    int pre = 0;                       // kda_pre_flags_t: raw q, k and gate tensor
};

// Room after the backward's workspace for the pre-processed inputs (pre != 0):
// normalised q and k in the input dtype, their inverse row norms, the fp32 log-gate.
struct PreLayout {
    size_t qn, kn, inv, gact, total;
};
bool pre_gate_materialised(int gate, int pre) {
    return gate != KDA_GATE_NONE && (pre & (KDA_PRE_GATE_SOFTPLUS | KDA_PRE_GATE_BF16));
}
PreLayout pre_layout(size_t base, size_t tok, int dk, int in_dtype, int gate, int pre) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const bool qk = pre & KDA_PRE_QK_L2NORM;
    PreLayout P{};
    size_t off = al(base);
    P.qn = off;   off = al(off + (qk ? tok * dk * esize(in_dtype) : 0));
    P.kn = off;   off = al(off + (qk ? tok * dk * esize(in_dtype) : 0));
    P.inv = off;  off = al(off + (qk ? 2 * tok * 4 : 0));
    P.gact = off; off = al(off + (pre_gate_materialised(gate, pre) ? tok * gate_bytes(gate, dk) : 0));
    P.total = pre ? off : base;
    return P;
}

// The backward pass: validation, the forward stages again (with checkpoints),
// then the backward stages.
int run_bwd(BwdCall c) {
    const int dk = c.dk_size, dv = c.dv_size;
    c.C = bwd_chunk(c.C);
    if (c.B < 0 || c.T < 0 || c.H < 0 || c.N < 0) return KDA_ERR_SHAPE;
    if (!dtype_ok(c.in_dtype) || !gate_ok(c.gate) || !pre_ok(c.pre)) return KDA_ERR_UNSUPPORTED;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    const bool bf = c.in_dtype == KDA_BF16;
    if (!kda::bwd_supported(dk, dv, c.C, bf) || !kda::chunk_supported(dk, dv, c.C, bf)) return KDA_ERR_UNSUPPORTED;
    if (!units_ok(c.packed, c.B, c.N, c.T, c.H, c.C)) return KDA_ERR_SHAPE;
    // token rows: [B,T,H] (fixed-length) or [T,H] (packed); states: [B,H] or [N,H]
    const long nseqh = (long)(c.packed ? c.N : c.B) * c.H;
    const size_t tok = (size_t)(c.packed ? 1 : c.B) * c.T * c.H, nst = (size_t)nseqh * dk * dv;
    const bool need_g = c.gate != KDA_GATE_NONE;
    if (!need_g) c.g = nullptr;
    if (!need_g) c.dg = nullptr;
    if (c.packed && nseqh > 0 && !c.cu_seqlens) return KDA_ERR_NULL;
    if (c.packed && c.cu_seqlens && !aligned(c.cu_seqlens, 4)) return KDA_ERR_MISALIGNED;
    if (tok > 0 && (!c.q || !c.k || !c.v || (need_g && (!c.g || !c.dg)) || !c.beta || !c.dO || !c.dq || !c.dk ||
                    !c.dv || !c.dbeta))
        return KDA_ERR_NULL;
    const void* p16[4] = {c.q, c.k, c.v, c.ws};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    // a gate tensor read only by the elementwise pre-processing needs its element's
    // alignment; one the forward stages read directly, as kda_chunk_fwd_ex
    const bool g_mat = pre_gate_materialised(c.gate, c.pre);
    if (c.g && !aligned(c.g, g_mat ? ((c.pre & KDA_PRE_GATE_BF16) ? 2 : 4) : (c.gate == KDA_GATE_CHANNEL ? 16 : 4)))
        return KDA_ERR_MISALIGNED;
    const void* p4[10] = {c.beta, c.s0, c.dO, c.dST, c.dq, c.dk, c.dv, c.dg, c.dbeta, c.dS0};
    for (const void* p : p4)
        if (p && !aligned(p, 4)) return KDA_ERR_MISALIGNED;
    const kda::BwdLayout L = c.packed ? kda::bwd_layout_packed(c.N, c.T, c.H, dk, dv, bf, c.C)
                                      : kda::bwd_layout(c.B, c.T, c.H, dk, dv, bf, c.C);
    const PreLayout P = pre_layout(L.total, tok, dk, c.in_dtype, c.gate, c.pre);
    const bool uses_ws = tok > 0 && nseqh > 0;
    if (uses_ws && (!c.ws || c.ws_bytes < P.total)) return KDA_ERR_WORKSPACE;
    const size_t ei = esize(c.in_dtype), gb = gate_bytes(c.gate, dk);
    const Range rq = range_of(c.q, tok * dk * ei), rk = range_of(c.k, tok * dk * ei), rv = range_of(c.v, tok * dv * ei),
                rg = range_of(c.g, tok * gate_bytes(c.gate, dk, c.pre)), rb = range_of(c.beta, tok * 4),
                rs0 = range_of(c.s0, nst * 4), rdo = range_of(c.dO, tok * dv * 4), rdst = range_of(c.dST, nst * 4),
                rw = range_of(c.ws, uses_ws ? P.total : 0),
                rcu = range_of(c.packed ? c.cu_seqlens : nullptr, ((size_t)c.N + 1) * 4);
    const Range outs[] = {range_of(c.dq, tok * dk * 4), range_of(c.dk, tok * dk * 4), range_of(c.dv, tok * dv * 4),
                          range_of(c.dg, tok * gb), range_of(c.dbeta, tok * 4), range_of(c.dS0, nst * 4)};
    const Range ins[] = {rq, rk, rv, rg, rb, rs0, rdo, rdst, rw, rcu};
    for (int i = 0; i < 6; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return KDA_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return KDA_ERR_ALIAS;
    }
    const Range fwd_in[] = {rq, rk, rv, rg, rb, rs0, rdo, rdst, rcu};
    for (const Range& r : fwd_in)
        if (overlap(rw, r)) return KDA_ERR_ALIAS;

    if (nseqh == 0) return KDA_OK;
    int st = device_ready();
    if (st != KDA_OK) return st;
    if (c.T == 0) {                                        // dS0 = dS_T: nothing happens in between
        if (c.dS0) {
            hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0,
                               (hipStream_t)c.stream, c.dST, c.dS0, (long)nst);
            return finish(hipGetLastError(), (hipStream_t)c.stream);
        }
        return KDA_OK;
    }
    char* ws = (char*)c.ws;
    kda::ChunkArgs a;
    a.q = c.q; a.k = c.k; a.v = c.v; a.g = (const float*)c.g; a.beta = c.beta; a.s0 = c.s0;
    a.o = nullptr; a.sT = nullptr;
    // pre-processing: the stages below see the normalised q, k and the fp32 log-gate
    kda::PreBwdArgs pb{};
    if (c.pre) {
        pb.q = c.q; pb.k = c.k; pb.g = c.g;
        pb.qn = ws + P.qn; pb.kn = ws + P.kn; pb.inv = (float*)(ws + P.inv); pb.g_act = (float*)(ws + P.gact);
        pb.dq = c.dq; pb.dk = c.dk; pb.dg = c.dg;
        pb.rows = (long)tok; pb.dk_size = dk; pb.in_bf16 = bf; pb.gate = c.gate; pb.mode = pre_mode(c.pre);
        pb.stream = (hipStream_t)c.stream;
        if (kda::run_pre_bwd_inputs(pb) != hipSuccess) return KDA_ERR_HIP;
        if (c.pre & KDA_PRE_QK_L2NORM) { a.q = pb.qn; a.k = pb.kn; }
        if (g_mat) a.g = pb.g_act;
    }
    a.B = c.packed ? 1 : c.B; a.T = c.T; a.H = c.H; a.dk = dk; a.dv = dv; a.C = c.C;
    a.in_bf16 = bf; a.out_bf16 = false; a.gate = c.gate;
    a.ws = ws; a.ws_bytes = L.fwd.total; a.stream = (hipStream_t)c.stream;
    a.cu_seqlens = c.packed ? c.cu_seqlens : nullptr;
    a.N = c.packed ? c.N : 0;
    a.checkpoints = true;
    a.ck_t = (float*)(ws + L.t); a.ck_a = (float*)(ws + L.a);
    a.ck_state = (float*)(ws + L.state); a.ck_w = (float*)(ws + L.w);
    if (kda::run_chunk_intra(a) != hipSuccess) return KDA_ERR_HIP;
    if (kda::run_chunk_chain(a) != hipSuccess) return KDA_ERR_HIP;
    kda::BwdArgs bw;
    bw.fwd = a; bw.dO = c.dO; bw.dST = c.dST;
    bw.dq = c.dq; bw.dk = c.dk; bw.dv = c.dv; bw.dg = c.dg; bw.dbeta = c.dbeta; bw.dS0 = c.dS0;
    bw.ck_dS = (float*)(ws + L.dS); bw.ck_dW = (float*)(ws + L.dW);
    if (kda::run_chunk_bwd_stages(bw) != hipSuccess) return KDA_ERR_HIP;
    if (c.pre && kda::run_pre_bwd_grads(pb) != hipSuccess) return KDA_ERR_HIP;
    return finish(hipSuccess, (hipStream_t)c.stream);
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "a size is negative or inconsistent";
        case KDA_ERR_UNSUPPORTED: return "unsupported dk, dv, chunk size or dtype";
        case KDA_ERR_MISALIGNED: return "a pointer lacks the alignment its argument needs";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_ALIAS: return "an output overlaps an argument it may not overlap";
        case KDA_ERR_HIP: return "no usable HIP device, or a HIP launch/execution error";
        default: return "unknown status";
    }
}

size_t kda_chunk_varlen_workspace_bytes(int N, int T, int H, int dk, int dv, int in_dtype, int C) {
    if (N < 0 || T < 0 || H < 0 || !dtype_ok(in_dtype)) return 0;
    C = fwd_chunk(C, dk, in_dtype);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    if (C != 16 && C != 32 && C != 64 && C != 128) return 0;
    if (!kda::chunk_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    return kda::ws_layout_packed(N, T, H, dk, dv, in_dtype == KDA_BF16, C).total;
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* initial_state, void* o, float* final_state, const int* cu_seqlens,
                         int N, int T, int H, int dk, int dv, int in_dtype, int out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream, int C, int gate_layout) {
    ChunkCall c{q, k, v, g, beta, initial_state, o, final_state, 1, T, H, dk, dv, in_dtype,
                out_dtype, workspace, workspace_bytes, stream, C, gate_layout};
    c.cu_seqlens = cu_seqlens;
    c.N = N;
    c.packed = true;
    return run_chunk(c, STAGE_INTRA | STAGE_CHAIN);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype, int C) {
    if (B < 0 || T < 0 || H < 0 || !dtype_ok(in_dtype)) return 0;
    C = bwd_chunk(C);
    if (!kda::bwd_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    if (!kda::chunk_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    return kda::bwd_layout(B, T, H, dk, dv, in_dtype == KDA_BF16, C).total;
}

size_t kda_chunk_bwd_varlen_workspace_bytes(int N, int T, int H, int dk, int dv, int in_dtype, int C) {
    if (N < 0 || T < 0 || H < 0 || !dtype_ok(in_dtype)) return 0;
    C = bwd_chunk(C);
    if (!kda::bwd_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    if (!kda::chunk_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    return kda::bwd_layout_packed(N, T, H, dk, dv, in_dtype == KDA_BF16, C).total;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* initial_state, const float* dO, const float* dST, float* dq, float* dk_out,
                  float* dv_out, float* dg, float* dbeta, float* dS0, int B, int T, int H, int dk, int dv,
                  int in_dtype, void* workspace, size_t workspace_bytes, void* stream, int C, int gate_layout) {
    BwdCall c{q, k, v, g, beta, initial_state, dO, dST, dq, dk_out, dv_out, dg, dbeta, dS0,
              B, T, H, dk, dv, in_dtype, workspace, workspace_bytes, stream, C, gate_layout};
    return run_bwd(c);
}

size_t kda_chunk_bwd_pre_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype, int C, int gate_layout,
                                         int pre_flags) {
    if (!gate_ok(gate_layout) || !pre_ok(pre_flags)) return 0;
    const size_t base = kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, in_dtype, C);
    if (base == 0) return 0;
    return pre_layout(base, (size_t)B * T * H, dk, in_dtype, gate_layout, pre_flags).total;
}

int kda_chunk_bwd_pre(const void* q, const void* k, const void* v, const void* g, const float* beta,
                      const float* initial_state, const float* dO, const float* dST, float* dq, float* dk_out,
                      float* dv_out, float* dg, float* dbeta, float* dS0, int B, int T, int H, int dk, int dv,
                      int in_dtype, void* workspace, size_t workspace_bytes, void* stream, int C, int gate_layout,
                      int pre_flags) {
    BwdCall c{q, k, v, g, beta, initial_state, dO, dST, dq, dk_out, dv_out, dg, dbeta, dS0,
              B, T, H, dk, dv, in_dtype, workspace, workspace_bytes, stream, C, gate_layout};
    c.pre = pre_flags;
    return run_bwd(c);
}

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* initial_state, const float* dO, const float* dST, float* dq,
                         float* dk_out, float* dv_out, float* dg, float* dbeta, float* dS0,
                         const int* cu_seqlens, int N, int T, int H, int dk, int dv, int in_dtype,
                         void* workspace, size_t workspace_bytes, void* stream, int C, int gate_layout) {
    BwdCall c{q, k, v, g, beta, initial_state, dO, dST, dq, dk_out, dv_out, dg, dbeta, dS0,
              1, T, H, dk, dv, in_dtype, workspace, workspace_bytes, stream, C, gate_layout};
    c.cu_seqlens = cu_seqlens;
    c.N = N;
    c.packed = true;
    return run_bwd(c);
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype, int C) {
    if (B < 0 || T < 0 || H < 0 || !dtype_ok(in_dtype)) return 0;
    C = fwd_chunk(C, dk, in_dtype);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    if (C != 16 && C != 32 && C != 64 && C != 128) return 0;
    if (!kda::chunk_supported(dk, dv, C, in_dtype == KDA_BF16)) return 0;
    return kda::ws_layout(B, T, H, dk, dv, in_dtype == KDA_BF16, C).total;
}

int kda_chunk_fwd_segments(int B, int T, int H, int dk, int dv, int in_dtype, int C) {
    if (kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, in_dtype, C) == 0) return 0;
    return kda::seg_plan(B, T, H, dk, dv, in_dtype == KDA_BF16, fwd_chunk(C, dk, in_dtype), false).nseg;
}

int kda_chunk_size_used(int dk, int dv, int in_dtype, int C, int backward) {
    if (!dtype_ok(in_dtype) || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    if (C != 16 && C != 32 && C != 64 && C != 128) return 0;
    const int used = backward ? bwd_chunk(C) : fwd_chunk(C, dk, in_dtype);
    const bool bf = in_dtype == KDA_BF16;
    if (!kda::chunk_supported(dk, dv, used, bf) || (backward && !kda::bwd_supported(dk, dv, used, bf))) return 0;
    return used;
}

#define KDA_CHUNK_PARAMS                                                                    \
    const void *q, const void *k, const void *v, const float *g, const float *beta,         \
        const float *initial_state, void *o, float *final_state, int B, int T, int H, int dk, \
        int dv, int in_dtype, int out_dtype, void *workspace, size_t workspace_bytes,        \
        void *stream, int C
#define KDA_CHUNK_CALL(GATE)                                                                \
    ChunkCall { q, k, v, g, beta, initial_state, o, final_state, B, T, H, dk, dv, in_dtype,  \
                out_dtype, workspace, workspace_bytes, stream, C, GATE }

int kda_chunk_fwd(KDA_CHUNK_PARAMS) { return run_chunk(KDA_CHUNK_CALL(KDA_GATE_CHANNEL), STAGE_INTRA | STAGE_CHAIN); }
int kda_chunk_intra(KDA_CHUNK_PARAMS) { return run_chunk(KDA_CHUNK_CALL(KDA_GATE_CHANNEL), STAGE_INTRA); }
// the chain stage does not read g (any layout, NULL allowed)
int kda_chunk_chain(KDA_CHUNK_PARAMS) { return run_chunk(KDA_CHUNK_CALL(KDA_GATE_NONE), STAGE_CHAIN); }
int kda_chunk_fwd_ex(KDA_CHUNK_PARAMS, int gate_layout) {
    return run_chunk(KDA_CHUNK_CALL(gate_layout), STAGE_INTRA | STAGE_CHAIN);
}
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* initial_state, void* o, float* final_state, int B, int T, int H, int dk,
                          int dv, int in_dtype, int out_dtype, void* stream, int C, int gate_layout) {
    ChunkCall c{q, k, v, g, beta, initial_state, o, final_state, B, T, H, dk, dv, in_dtype,
                out_dtype, nullptr, 0, stream, C, gate_layout};
    c.static_ws = true;
    return run_chunk(c, STAGE_INTRA | STAGE_CHAIN);
}
int kda_chunk_intra_ex(KDA_CHUNK_PARAMS, int gate_layout) {
    return run_chunk(KDA_CHUNK_CALL(gate_layout), STAGE_INTRA);
}
#define KDA_CHUNK_PRE_CALL(GATE, PRE)                                                       \
    [&] {                                                                                   \
        ChunkCall c_ = KDA_CHUNK_CALL(GATE);                                                \
        c_.pre = (PRE);                                                                     \
        return c_;                                                                          \
    }()
int kda_chunk_fwd_pre(const void* q, const void* k, const void* v, const void* g_any, const float* beta,
                      const float* initial_state, void* o, float* final_state, int B, int T, int H, int dk,
                      int dv, int in_dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream, int C, int gate_layout, int pre_flags) {
    const float* g = static_cast<const float*>(g_any);
    return run_chunk(KDA_CHUNK_PRE_CALL(gate_layout, pre_flags), STAGE_INTRA | STAGE_CHAIN);
}
int kda_chunk_intra_pre(const void* q, const void* k, const void* v, const void* g_any, const float* beta,
                        const float* initial_state, void* o, float* final_state, int B, int T, int H, int dk,
                        int dv, int in_dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                        void* stream, int C, int gate_layout, int pre_flags) {
    const float* g = static_cast<const float*>(g_any);
    return run_chunk(KDA_CHUNK_PRE_CALL(gate_layout, pre_flags), STAGE_INTRA);
}
#undef KDA_CHUNK_PRE_CALL

}  // extern "C"

namespace {

int decode_call(const void* q, const void* k, const void* v, const float* g, const float* beta,
                float* state, void* o, int N, int T, int H, int dk, int dv, int in_dtype, int out_dtype,
                void* stream, int gate_layout, int pre = 0) {
    if (N < 0 || T < 0 || H < 0) return KDA_ERR_SHAPE;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype) || !gate_ok(gate_layout) || !pre_ok(pre))
        return KDA_ERR_UNSUPPORTED;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    const size_t nh = (size_t)N * H, tok = nh * (size_t)T;
    if (tok == 0) return KDA_OK;
    // one workgroup per (n, h) in a 1-D grid: the work-items, nh times the
    // workgroup size the token count selects, must fit in 32 bits
    if (nh > 0xffffffffull / (size_t)kda::decode_block_threads(T)) return KDA_ERR_SHAPE;
    const bool need_g = gate_layout != KDA_GATE_NONE;
    if (!q || !k || !v || (need_g && !g) || !beta || !state || !o) return KDA_ERR_NULL;
    if (!need_g) g = nullptr;                            // g is not read without gates
    // the state is streamed in 16-byte vectors; the rest is read element-wise
    if (!aligned(state, 16)) return KDA_ERR_MISALIGNED;
    const void* pe[6] = {q, k, v, g, beta, o};
    const uintptr_t ae[6] = {esize(in_dtype), esize(in_dtype), esize(in_dtype),
                             (uintptr_t)((pre & KDA_PRE_GATE_BF16) ? 2 : 4), 4, esize(out_dtype)};
    for (int i = 0; i < 6; ++i)
        if (pe[i] && !aligned(pe[i], ae[i])) return KDA_ERR_MISALIGNED;
    const size_t ei = esize(in_dtype), eo = esize(out_dtype);
    const Range rq = range_of(q, tok * dk * ei), rk = range_of(k, tok * dk * ei),
                rv = range_of(v, tok * dv * ei), rg = range_of(g, tok * gate_bytes(gate_layout, dk, pre)),
                rb = range_of(beta, tok * 4),
                rs = range_of(state, nh * dk * dv * 4), ro = range_of(o, tok * dv * eo);
    const Range in[] = {rq, rk, rv, rg, rb};
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_ALIAS;
    if (overlap(ro, rs)) return KDA_ERR_ALIAS;

    int st = device_ready();
    if (st != KDA_OK) return st;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.N = N; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.gate = gate_layout;
    a.pre = pre_mode(pre);
    a.stream = (hipStream_t)stream;
    return finish(kda::run_decode_step(a), a.stream);
}

}  // namespace

extern "C" {

int kda_decode_step_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       float* state, void* o, int N, int H, int dk, int dv, int in_dtype, int out_dtype,
                       void* stream, int gate_layout) {
    return decode_call(q, k, v, g, beta, state, o, N, 1, H, dk, dv, in_dtype, out_dtype, stream, gate_layout);
}

int kda_decode_tokens(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      float* state, void* o, int N, int T, int H, int dk, int dv, int in_dtype,
                      int out_dtype, void* stream, int gate_layout) {
    return decode_call(q, k, v, g, beta, state, o, N, T, H, dk, dv, in_dtype, out_dtype, stream, gate_layout);
}

int kda_decode_tokens_pre(const void* q, const void* k, const void* v, const void* g, const float* beta,
                          float* state, void* o, int N, int T, int H, int dk, int dv, int in_dtype,
                          int out_dtype, void* stream, int gate_layout, int pre_flags) {
    return decode_call(q, k, v, static_cast<const float*>(g), beta, state, o, N, T, H, dk, dv, in_dtype,
                       out_dtype, stream, gate_layout, pre_flags);
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    float* state, void* o, int N, int H, int dk, int dv, int in_dtype, int out_dtype,
                    void* stream) {
    return kda_decode_step_ex(q, k, v, g, beta, state, o, N, H, dk, dv, in_dtype, out_dtype, stream,
                              KDA_GATE_CHANNEL);
}

}  // extern "C"
