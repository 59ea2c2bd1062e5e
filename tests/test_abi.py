"""The C ABI: exported symbols, host-side validation and status codes (CPU).

No compute runs here: valid calls stop at the device check (KDA_ERR_HIP on a
machine without a GPU), invalid ones are rejected before any HIP call, so fake
(never dereferenced) pointers are enough."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from linear_attention_sequence_chunk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
HAS_GPU = torch.cuda.is_available()

OK, NULL, SHAPE, UNSUP, MISAL, WS, ALIAS, HIP = range(8)


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = declared()
    assert set(names) == set(_lib.SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = _lib.lib()
    for n in names:
        getattr(L, n)


def test_version_and_strings():
    L = _lib.lib()
    assert L.kda_abi_version() == 1
    for s in range(8):
        assert len(_lib.status_string(s)) >= 2
    assert _lib.status_string(99) == "unknown status"


def test_workspace_bytes():
    L = _lib.lib()
    ws = L.kda_chunk_fwd_workspace_bytes
    # per chunk-head: 3*C*dk + C*C elements in the input dtype, C*dv + dk fp32
    n = ws(1, 64, 1, 64, 64, _lib.F32, 64)
    assert n >= (3 * 64 * 64 + 64 * 64) * 4 + (64 * 64 + 64) * 4
    assert ws(4, 8192, 16, 128, 128, _lib.BF16, 64) > ws(4, 8192, 16, 128, 128, _lib.BF16, 128) // 2
    assert ws(1, 10, 1, 96, 64, _lib.F32, 64) == 0       # unsupported dk
    assert ws(1, 10, 1, 64, 64, _lib.F32, 48) == 0       # unsupported C
    assert ws(1, 10, 1, 64, 64, 7, 64) == 0              # bad dtype
    assert ws(1, 100, 1, 64, 64, _lib.F32, 64) == ws(1, 128, 1, 64, 64, _lib.F32, 64)  # partial chunk


class Fake:
    """Non-overlapping fake device addresses (never dereferenced)."""
    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return p


def chunk_args(B=2, T=100, H=3, dk=64, dv=64, ind=_lib.F32, outd=_lib.F32, C=64):
    f = Fake()
    e = 4 if ind == _lib.F32 else 2
    eo = 4 if outd == _lib.F32 else 2
    tok = B * T * H
    a = dict(q=f(tok * dk * e), k=f(tok * dk * e), v=f(tok * dv * e), g=f(tok * dk * 4),
             beta=f(tok * 4), s0=f(B * H * dk * dv * 4), o=f(tok * dv * eo),
             sT=f(B * H * dk * dv * 4))
    wsb = _lib.lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, ind, C)
    a.update(ws=f(wsb), wsb=wsb, B=B, T=T, H=H, dk=dk, dv=dv, ind=ind, outd=outd, C=C)
    return a


def call_chunk(a, fn="kda_chunk_fwd", gate=None):
    L = _lib.lib()
    args = [a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"], a["sT"],
            a["B"], a["T"], a["H"], a["dk"], a["dv"], a["ind"], a["outd"], a["ws"], a["wsb"], None, a["C"]]
    if gate is not None:
        return getattr(L, fn + "_ex")(*args, gate)
    return getattr(L, fn)(*args)


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_intra", "kda_chunk_chain"])
def test_chunk_validation_codes(fn):
    a = chunk_args()
    cases = [
        (dict(B=-1), SHAPE), (dict(T=-5), SHAPE), (dict(T=2**31 - 1, H=64), SHAPE),   # 2^31 (chunk, head) units
        (dict(dk=96), UNSUP), (dict(dv=32), UNSUP), (dict(C=48), UNSUP), (dict(C=256), UNSUP),
        (dict(ind=5), UNSUP), (dict(outd=-1), UNSUP),
        (dict(q=None), NULL), (dict(beta=None), NULL), (dict(o=None), NULL),
        (dict(k=a["k"] + 8), MISAL), (dict(g=a["g"] + 4), MISAL), (dict(g=a["g"] + 8), MISAL),
        (dict(s0=a["s0"] + 2), MISAL),
        (dict(ws=a["ws"] + 8), MISAL), (dict(o=a["o"] + 4), MISAL),
        (dict(ws=None), WS), (dict(wsb=a["wsb"] - 1), WS),
        (dict(o=a["q"]), ALIAS), (dict(o=a["ws"]), ALIAS), (dict(sT=a["v"]), ALIAS),
        (dict(sT=a["s0"] + 256), ALIAS), (dict(ws=a["g"]), ALIAS), (dict(o=a["sT"]), ALIAS),
    ]
    for change, code in cases:
        if fn == "kda_chunk_chain" and "g" in change or (fn == "kda_chunk_chain" and change.get("ws") == a["g"]):
            continue                      # the chain stage does not read g
        b = dict(a)
        b.update(change)
        assert call_chunk(b, fn) == code, (change, code)


@pytest.mark.skipif(HAS_GPU, reason="valid calls with fake pointers would reach a real device")
@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_intra"])
def test_gate_layout_codes(fn):
    a = chunk_args(ind=_lib.BF16, outd=_lib.BF16, dk=128, dv=128)
    CH, HEAD, NONE = _lib.GATE["channel"], _lib.GATE["head"], _lib.GATE["none"]
    tok = a["B"] * a["T"] * a["H"]
    cases = [
        (dict(), 3, UNSUP), (dict(), -1, UNSUP),
        (dict(g=None), CH, NULL), (dict(g=None), HEAD, NULL), (dict(g=None), NONE, HIP),
        (dict(g=a["g"] + 4), CH, MISAL), (dict(g=a["g"] + 8), CH, MISAL), (dict(g=a["g"] + 16), CH, HIP),
        (dict(g=a["g"] + 4), HEAD, HIP), (dict(g=a["g"] + 2), HEAD, MISAL),
        (dict(g=a["g"] + 2), NONE, HIP),                     # g is not read without gates
        (dict(g=a["ws"] - tok * 4), HEAD, HIP),              # a per-head g is [B,T,H] only
        (dict(g=a["ws"] - tok * 4), CH, ALIAS), (dict(g=a["ws"]), NONE, HIP),
        (dict(), CH, HIP), (dict(), HEAD, HIP), (dict(), NONE, HIP),
    ]
    for change, gate, code in cases:
        b = dict(a)
        b.update(change)
        assert call_chunk(b, fn, gate) == code, (change, gate, code)
    b = dict(a); b["g"] = None
    assert call_chunk(b, "kda_chunk_chain") == HIP        # the chain stage takes NULL g


def test_noalloc_rejects_sizes_beyond_its_array():
    """kda_chunk_fwd_noalloc: a workspace larger than the static array is refused
    on the host (KDA_ERR_WORKSPACE) before any HIP call; sizes within it reach
    the device check; the usual argument checks apply."""
    L = _lib.lib()
    big = chunk_args(B=1, T=9000, H=16, dk=128, dv=128, ind=_lib.BF16, outd=_lib.BF16)
    assert big["wsb"] > _lib.NOALLOC_WORKSPACE_MAX

    def call(a, gate=0):
        return L.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"], a["sT"],
                                       a["B"], a["T"], a["H"], a["dk"], a["dv"], a["ind"], a["outd"], None,
                                       a["C"], gate)
    assert call(big) == WS
    small = chunk_args(B=2, T=300, H=3, dk=128, dv=128, ind=_lib.BF16, outd=_lib.BF16)
    assert call(dict(small, C=48)) == UNSUP
    assert call(dict(small, q=None)) == NULL
    assert call(dict(small, o=small["q"])) == ALIAS
    assert call(dict(small, g=small["g"] + 8)) == MISAL
    assert call(dict(small, B=0)) == OK
    if not HAS_GPU:
        assert call(small) == HIP


def test_segment_plan():
    """kda_chunk_fwd_segments: the chain runs in segments only in the hot
    configuration (bf16, dk = 128, 64-token chunks), for fixed-length batches
    whose sequential chain would have fewer than 256 workgroups of 32 columns,
    with at least four segments after the first and none of them shorter than 32
    chunks; each of the two segment launches takes (segments - 1) workgroups
    per pair, at most 256."""
    seg = _lib.lib().kda_chunk_fwd_segments
    B16, F = _lib.BF16, _lib.F32
    assert seg(1, 1 << 20, 16, 128, 128, B16, 64) == 17          # the 1M-token workload
    assert seg(4, 8192, 16, 128, 128, B16, 64) == 1              # 64 pairs x 4 slices fill the GPU
    assert seg(1, 65536, 32, 128, 128, B16, 128) == 9            # C = 128 runs as 64-token chunks
    assert seg(1, 10240, 1, 128, 128, B16, 64) == 5              # 160 chunks: the fewest segments
    assert seg(1, 10239, 1, 128, 128, B16, 64) == 5              # 160 chunks, the last one partial
    assert seg(1, 10176, 1, 128, 128, B16, 64) == 1              # 159 chunks: sequential
    assert seg(1, 4096, 1, 128, 128, B16, 64) == 1
    assert seg(2, 12352, 1, 128, 64, B16, 64) == 6
    assert seg(1, 1 << 20, 16, 64, 64, B16, 64) == 1             # generic kernels: sequential chain
    assert seg(1, 1 << 20, 16, 128, 128, F, 64) == 1
    assert seg(1, 100, 1, 96, 128, B16, 64) == 0                 # unsupported
    L = _lib.lib()
    # segments add E, M and a start state per pair and segment to the workspace
    per_pair = lambda b, h, t: L.kda_chunk_fwd_workspace_bytes(b, t, h, 128, 128, B16, 64) // (b * h)
    assert per_pair(1, 1, 10240) - per_pair(1, 64, 10240) >= 5 * 3 * 128 * 128 * 4


def test_chunk_size_used():
    """C = 128 runs as 64-token chunks for fp32 inputs, for bf16 inputs with
    dk = 128 and in the backward pass; other sizes run as asked.  The workspace
    follows the chunk that runs."""
    L = _lib.lib()
    used = L.kda_chunk_size_used
    F, B16 = _lib.F32, _lib.BF16
    assert used(64, 64, F, 128, 0) == 64 and used(128, 128, F, 128, 0) == 64
    assert used(128, 128, B16, 128, 0) == 64 and used(128, 64, B16, 128, 0) == 64
    assert used(64, 64, B16, 128, 0) == 128 and used(64, 128, B16, 128, 0) == 128
    assert used(64, 128, B16, 128, 1) == 64 and used(128, 128, F, 128, 1) == 64
    for C in (16, 32, 64):
        assert used(128, 128, F, C, 0) == C and used(64, 64, B16, C, 1) == C
    assert used(96, 64, F, 64, 0) == 0 and used(64, 64, F, 48, 0) == 0 and used(64, 64, 9, 64, 0) == 0
    ws = L.kda_chunk_fwd_workspace_bytes
    assert ws(2, 300, 3, 64, 128, F, 128) == ws(2, 300, 3, 64, 128, F, 64) > 0
    assert ws(2, 300, 3, 128, 128, B16, 128) == ws(2, 300, 3, 128, 128, B16, 64)
    assert ws(2, 300, 3, 64, 64, B16, 128) != ws(2, 300, 3, 64, 64, B16, 64)
    bws = L.kda_chunk_bwd_workspace_bytes
    assert bws(2, 300, 3, 64, 64, B16, 128) == bws(2, 300, 3, 64, 64, B16, 64) > 0


@pytest.mark.parametrize("dk", [64, 128])
def test_fp32_c128_is_supported(dk):
    a = chunk_args(dk=dk, dv=128, C=128)
    assert a["wsb"] > 0
    assert call_chunk(a) == (OK if HAS_GPU else HIP) or HAS_GPU


def test_valid_chunk_call_reaches_device_check():
    a = chunk_args(ind=_lib.BF16, outd=_lib.BF16, dk=128, dv=128)
    b = dict(a); b["sT"] = b["s0"]                      # in-place state is allowed
    b2 = dict(a); b2["s0"] = None; b2["sT"] = None      # no states is allowed
    for x in (a, b, b2):
        st = call_chunk(x)
        assert st == (OK if HAS_GPU else HIP) or (HAS_GPU and st == HIP)
    if not HAS_GPU:
        assert call_chunk(a) == HIP


def test_empty_sizes_return_ok_without_pointers():
    L = _lib.lib()
    st = L.kda_chunk_fwd(None, None, None, None, None, None, None, None, 0, 5, 3, 64, 64,
                         0, 0, None, 0, None, 64)
    assert st in (OK, HIP)
    assert L.kda_decode_step(None, None, None, None, None, None, None, 0, 4, 64, 64, 0, 0, None) == OK


def test_decode_validation_codes():
    L = _lib.lib()
    f = Fake()
    N, H, dk, dv = 3, 2, 128, 64
    a = dict(q=f(N * H * dk * 2), k=f(N * H * dk * 2), v=f(N * H * dv * 2), g=f(N * H * dk * 4),
             beta=f(N * H * 4), state=f(N * H * dk * dv * 4), o=f(N * H * dv * 2),
             N=N, H=H, dk=dk, dv=dv, ind=_lib.BF16, outd=_lib.BF16)

    def call(x):
        return L.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], x["o"],
                                 x["N"], x["H"], x["dk"], x["dv"], x["ind"], x["outd"], None)
    cases = [(dict(N=-1), SHAPE), (dict(dk=100), UNSUP), (dict(ind=3), UNSUP),
             (dict(state=None), NULL), (dict(v=a["v"] + 1), MISAL), (dict(state=a["state"] + 8), MISAL),
             (dict(o=a["state"]), ALIAS), (dict(state=a["q"]), ALIAS), (dict(o=a["g"] + 16), ALIAS),
             (dict(N=1 << 16, H=(1 << 15) + 1), SHAPE)]                 # N*H beyond one grid dimension
    for change, code in cases:
        b = dict(a); b.update(change)
        assert call(b) == code, (change, code)
    if not HAS_GPU:
        assert call(a) == HIP

    def sized(n, T=1):
        g = Fake()
        return dict(q=g(n * T * dk * 2), k=g(n * T * dk * 2), v=g(n * T * dv * 2), g=g(n * T * dk * 4),
                    beta=g(n * T * 4), state=g(n * dk * dv * 4), o=g(n * T * dv * 2),
                    N=n, T=T, H=1, dk=dk, dv=dv, ind=_lib.BF16, outd=_lib.BF16)
    # one token per call: 1024-thread workgroups, so 2^22 pairs are 2^32 work-items
    assert call(sized(4194304)) == SHAPE
    if not HAS_GPU:
        assert call(sized(4194303)) == HIP              # the largest single-token grid

    def call_ex(x, gate):
        return L.kda_decode_step_ex(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], x["o"],
                                    x["N"], x["H"], x["dk"], x["dv"], x["ind"], x["outd"], None, gate)
    ex_cases = [(dict(), 3, UNSUP), (dict(g=None), 0, NULL), (dict(g=None), 1, NULL),
                (dict(g=a["g"] + 2), 1, MISAL), (dict(o=a["g"] + 16), 0, ALIAS)]
    if not HAS_GPU:
        ex_cases += [(dict(g=None), 2, HIP), (dict(o=a["g"] + 4 * N * H), 1, HIP), (dict(), 1, HIP)]
    for change, gate, code in ex_cases:
        b = dict(a); b.update(change)
        assert call_ex(b, gate) == code, (change, gate, code)

    # several tokens per call: inputs [N,T,H,d]
    T = 4
    t = dict(q=f(N * T * H * dk * 2), k=f(N * T * H * dk * 2), v=f(N * T * H * dv * 2),
             g=f(N * T * H * dk * 4), beta=f(N * T * H * 4), state=f(N * H * dk * dv * 4),
             o=f(N * T * H * dv * 2), N=N, T=T, H=H, dk=dk, dv=dv, ind=_lib.BF16, outd=_lib.BF16)

    def call_t(x, gate=0):
        return L.kda_decode_tokens(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], x["o"],
                                   x["N"], x["T"], x["H"], x["dk"], x["dv"], x["ind"], x["outd"], None, gate)
    t_cases = [(dict(T=-1), SHAPE), (dict(dv=96), UNSUP), (dict(beta=None), NULL),
               (dict(o=t["v"] + (N * T * H * dv * 2) // 2), ALIAS), (dict(o=t["o"] + 1), MISAL)]
    for change, code in t_cases:
        b = dict(t); b.update(change)
        assert call_t(b) == code, (change, code)
    assert L.kda_decode_tokens(None, None, None, None, None, None, None, 3, 0, 2, 64, 64, 0, 0, None, 0) == OK
    if not HAS_GPU:
        assert call_t(t) == HIP
        # several tokens per call run 256-thread workgroups: 2^22 pairs still fit
        assert call_t(sized(4194304, T)) == HIP
    assert call_t(sized(1 << 24, T)) == SHAPE


def test_python_binding_refuses_cpu_tensors():
    from linear_attention_sequence_chunk_amd import chunk_fwd, decode_step
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1))
    with pytest.raises(ValueError):
        decode_step(x[0], x[0], x[0], x[0], torch.zeros(4, 1), torch.zeros(4, 1, 64, 64))


def test_varlen_validation_codes():
    L = _lib.lib()
    f = Fake()
    N, T, H, dk, dv = 4, 300, 2, 128, 128
    tok = T * H
    wsb = L.kda_chunk_varlen_workspace_bytes(N, T, H, dk, dv, _lib.BF16, 64)
    assert wsb > L.kda_chunk_fwd_workspace_bytes(1, T, H, dk, dv, _lib.BF16, 64)   # room for N extra chunks
    assert L.kda_chunk_varlen_workspace_bytes(N, T, H, 96, dv, _lib.BF16, 64) == 0
    a = dict(q=f(tok * dk * 2), k=f(tok * dk * 2), v=f(tok * dv * 2), g=f(tok * dk * 4), beta=f(tok * 4),
             s0=f(N * H * dk * dv * 4), o=f(tok * dv * 2), sT=f(N * H * dk * dv * 4), cu=f((N + 1) * 4),
             N=N, T=T, H=H, ws=f(wsb), wsb=wsb, gate=0)

    def call(x):
        return L.kda_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], x["o"], x["sT"],
                                      x["cu"], x["N"], x["T"], x["H"], dk, dv, _lib.BF16, _lib.BF16,
                                      x["ws"], x["wsb"], None, 64, x["gate"])
    cases = [(dict(N=-1), SHAPE), (dict(gate=5), UNSUP), (dict(cu=None), NULL), (dict(cu=a["cu"] + 2), MISAL),
             (dict(wsb=wsb - 1), WS), (dict(o=a["cu"]), ALIAS), (dict(sT=a["cu"]), ALIAS),
             (dict(ws=a["cu"] - 16), ALIAS), (dict(g=None), NULL)]
    for change, code in cases:
        b = dict(a); b.update(change)
        assert call(b) == code, (change, code)
    # nothing to do: no sequences, or no heads
    assert L.kda_chunk_fwd_varlen(None, None, None, None, None, None, None, None, None, 0, 0, 2, dk, dv,
                                  1, 1, None, 0, None, 64, 0) == OK
    if not HAS_GPU:
        assert call(a) == HIP
        b = dict(a); b["g"] = None; b["gate"] = 2
        assert call(b) == HIP


@pytest.mark.parametrize("fn", ["kda_chunk_fwd_pre", "kda_chunk_intra_pre"])
def test_pre_flag_codes(fn):
    """Pre-processing flags: unknown bits, and the bf16 gate's size and alignment."""
    L = _lib.lib()
    a = chunk_args(ind=_lib.BF16, outd=_lib.BF16, dk=128, dv=128)
    CH, HEAD = _lib.GATE["channel"], _lib.GATE["head"]
    QK, SP, GB = _lib.PRE_QK_L2NORM, _lib.PRE_GATE_SOFTPLUS, _lib.PRE_GATE_BF16
    tok = a["B"] * a["T"] * a["H"]

    def call(x, gate, pre):
        args = [x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], x["o"], x["sT"], x["B"], x["T"], x["H"],
                x["dk"], x["dv"], x["ind"], x["outd"], x["ws"], x["wsb"], None, x["C"], gate, pre]
        return getattr(L, fn)(*args)
    cases = [(dict(), CH, 8, UNSUP), (dict(), CH, -1, UNSUP),
             (dict(g=a["g"] + 8), CH, GB, MISAL),            # a per-channel bf16 g needs 16 bytes
             (dict(g=a["g"] + 1), HEAD, GB, MISAL),
             (dict(g=None), CH, SP, NULL),
             (dict(q=None), CH, QK, NULL)]
    if not HAS_GPU:
        cases += [(dict(), CH, QK | SP | GB, HIP), (dict(g=a["g"] + 16), CH, GB, HIP),
                  (dict(g=a["g"] + 2), HEAD, GB | SP, HIP),
                  # a bf16 per-channel g covers half the bytes: o may follow it
                  (dict(o=a["g"] + tok * 128 * 2), CH, GB, HIP),
                  (dict(o=a["g"] + tok * 128 * 2), CH, 0, ALIAS)]
    for change, gate, pre, code in cases:
        b = dict(a)
        b.update(change)
        if pre == 0:
            assert call_chunk(b, fn.replace("_pre", ""), gate) == code, (change, gate, pre, code)
        else:
            assert call(b, gate, pre) == code, (change, gate, pre, code)


def test_decode_pre_flag_codes():
    L = _lib.lib()
    f = Fake()
    N, T, H, dk, dv = 3, 2, 2, 128, 64
    t = dict(q=f(N * T * H * dk * 2), k=f(N * T * H * dk * 2), v=f(N * T * H * dv * 2),
             g=f(N * T * H * dk * 2), beta=f(N * T * H * 4), state=f(N * H * dk * dv * 4),
             o=f(N * T * H * dv * 2))

    def call(x, gate, pre):
        return L.kda_decode_tokens_pre(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], x["o"],
                                       N, T, H, dk, dv, _lib.BF16, _lib.BF16, None, gate, pre)
    assert call(t, 0, 16) == UNSUP
    assert call(dict(t, g=t["g"] + 1), 0, _lib.PRE_GATE_BF16) == MISAL
    assert call(dict(t, g=t["g"] + 2), 0, 0) == MISAL          # fp32 g needs 4 bytes
    if not HAS_GPU:
        assert call(dict(t, g=t["g"] + 2), 0, _lib.PRE_GATE_BF16 | _lib.PRE_GATE_SOFTPLUS) == HIP
        assert call(t, 2, _lib.PRE_QK_L2NORM) == HIP


def test_backward_validation_codes():
    L = _lib.lib()
    f = Fake()
    B, T, H, dk, dv, C = 2, 100, 3, 128, 64, 64
    tok, nst = B * T * H, B * H * dk * dv
    wsb = L.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, _lib.BF16, C)
    assert wsb > L.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, _lib.BF16, C)   # + checkpoints
    # C = 128 runs as 64-token chunks
    assert L.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, _lib.BF16, 128) == wsb
    a = dict(q=f(tok * dk * 2), k=f(tok * dk * 2), v=f(tok * dv * 2), g=f(tok * dk * 4), beta=f(tok * 4),
             s0=f(nst * 4), dO=f(tok * dv * 4), dST=f(nst * 4), dq=f(tok * dk * 4), dk=f(tok * dk * 4),
             dv=f(tok * dv * 4), dg=f(tok * dk * 4), dbeta=f(tok * 4), dS0=f(nst * 4),
             B=B, T=T, H=H, dkk=dk, dvv=dv, ind=_lib.BF16, ws=f(wsb), wsb=wsb, C=C, gate=0)

    def call(x):
        return L.kda_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], x["dO"], x["dST"],
                               x["dq"], x["dk"], x["dv"], x["dg"], x["dbeta"], x["dS0"], x["B"], x["T"],
                               x["H"], x["dkk"], x["dvv"], x["ind"], x["ws"], x["wsb"], None, x["C"], x["gate"])
    cases = [(dict(T=-1), SHAPE), (dict(T=2**31 - 1, H=64), SHAPE), (dict(dkk=96), UNSUP), (dict(C=48), UNSUP), (dict(ind=7), UNSUP),
             (dict(gate=5), UNSUP), (dict(dq=None), NULL), (dict(dO=None), NULL), (dict(dg=None), NULL),
             (dict(q=a["q"] + 8), MISAL), (dict(g=a["g"] + 4), MISAL), (dict(g=a["g"] + 8), MISAL),
             (dict(dbeta=a["dbeta"] + 2), MISAL),
             (dict(ws=None), WS), (dict(wsb=wsb - 1), WS),
             (dict(dq=a["q"]), ALIAS), (dict(dk=a["dq"] + 256), ALIAS), (dict(dS0=a["dST"]), ALIAS),
             (dict(ws=a["dO"]), ALIAS), (dict(dg=a["ws"]), ALIAS)]
    if not HAS_GPU:
        cases += [(dict(), HIP), (dict(gate=2, g=None, dg=None), HIP),   # no gates: g and dg may be NULL
                  (dict(dST=None, s0=None, dS0=None), HIP)]
    for change, code in cases:
        b = dict(a)
        b.update(change)
        assert call(b) == code, (change, code)
    empty = dict(a, B=0)
    assert call(empty) == OK


def test_backward_varlen_validation_codes():
    """kda_chunk_bwd_varlen: sizes, NULLs, alignment, workspace and aliasing,
    including cu_seqlens, all decided on the host."""
    L = _lib.lib()
    f = Fake()
    N, T, H, dk, dv, C = 3, 250, 2, 128, 64, 64
    tok, nst = T * H, N * H * dk * dv
    wsb = L.kda_chunk_bwd_varlen_workspace_bytes(N, T, H, dk, dv, _lib.BF16, C)
    assert wsb > L.kda_chunk_bwd_workspace_bytes(1, T, H, dk, dv, _lib.BF16, C)   # room for N extra chunks
    assert L.kda_chunk_bwd_varlen_workspace_bytes(N, T, H, dk, dv, _lib.BF16, 128) == wsb   # 64-token chunks
    assert L.kda_chunk_bwd_varlen_workspace_bytes(-1, T, H, dk, dv, _lib.BF16, C) == 0
    a = dict(q=f(tok * dk * 2), k=f(tok * dk * 2), v=f(tok * dv * 2), g=f(tok * dk * 4), beta=f(tok * 4),
             s0=f(nst * 4), dO=f(tok * dv * 4), dST=f(nst * 4), dq=f(tok * dk * 4), dk=f(tok * dk * 4),
             dv=f(tok * dv * 4), dg=f(tok * dk * 4), dbeta=f(tok * 4), dS0=f(nst * 4), cu=f((N + 1) * 4),
             N=N, T=T, H=H, ws=f(wsb), wsb=wsb, C=C, gate=0)

    def call(x):
        return L.kda_chunk_bwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], x["dO"], x["dST"],
                                      x["dq"], x["dk"], x["dv"], x["dg"], x["dbeta"], x["dS0"], x["cu"],
                                      x["N"], x["T"], x["H"], dk, dv, _lib.BF16, x["ws"], x["wsb"], None,
                                      x["C"], x["gate"])
    cases = [(dict(N=-1), SHAPE), (dict(C=96), UNSUP), (dict(gate=5), UNSUP), (dict(cu=None), NULL),
             (dict(dO=None), NULL), (dict(cu=a["cu"] + 2), MISAL), (dict(wsb=wsb - 1), WS),
             (dict(ws=None), WS), (dict(dq=a["cu"]), ALIAS), (dict(dS0=a["cu"]), ALIAS),
             (dict(ws=a["cu"] - 16), ALIAS), (dict(dS0=a["dST"]), ALIAS), (dict(dg=None), NULL)]
    for change, code in cases:
        b = dict(a)
        b.update(change)
        assert call(b) == code, (change, code)
    # nothing to do: no sequences, or no heads
    assert call(dict(a, N=0, T=0)) == OK
    assert call(dict(a, H=0)) == OK
    if not HAS_GPU:
        assert call(a) == HIP
        assert call(dict(a, g=None, dg=None, gate=2)) == HIP
        assert call(dict(a, T=0)) == HIP          # the dS0 = dST copy still needs a device


def test_backward_pre_validation_codes():
    """kda_chunk_bwd_pre: flag bits, the larger workspace, the bf16 gate's size
    and alignment, all decided on the host."""
    L = _lib.lib()
    f = Fake()
    B, T, H, dk, dv, C = 2, 100, 3, 128, 64, 64
    tok, nst = B * T * H, B * H * dk * dv
    QK, SP, GB = _lib.PRE_QK_L2NORM, _lib.PRE_GATE_SOFTPLUS, _lib.PRE_GATE_BF16
    plain = L.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, _lib.BF16, C)
    ws_of = lambda gate, pre: L.kda_chunk_bwd_pre_workspace_bytes(B, T, H, dk, dv, _lib.BF16, C, gate, pre)
    assert ws_of(0, 0) == plain
    assert ws_of(0, QK) >= plain + 2 * tok * dk * 2 + 2 * tok * 4        # normalised q, k and 1/|row|
    assert ws_of(0, SP) >= plain + tok * dk * 4                          # the fp32 log-gate
    assert ws_of(1, SP) < ws_of(0, SP)                                   # per-head gate: [tok] only
    assert ws_of(2, SP | GB) == plain                                    # no gate: nothing to form
    assert ws_of(0, 8) == 0 and ws_of(5, 0) == 0
    wsb = ws_of(0, QK | SP | GB)
    # g's fake extent has room for a dg right after a bf16 gate tensor
    a = dict(q=f(tok * dk * 2), k=f(tok * dk * 2), v=f(tok * dv * 2), g=f(tok * dk * 6), beta=f(tok * 4),
             s0=f(nst * 4), dO=f(tok * dv * 4), dST=f(nst * 4), dq=f(tok * dk * 4), dk=f(tok * dk * 4),
             dv=f(tok * dv * 4), dg=f(tok * dk * 4), dbeta=f(tok * 4), dS0=f(nst * 4),
             ws=f(wsb), wsb=wsb, gate=0, pre=QK | SP | GB)

    def call(x):
        return L.kda_chunk_bwd_pre(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], x["dO"], x["dST"],
                                   x["dq"], x["dk"], x["dv"], x["dg"], x["dbeta"], x["dS0"], B, T, H, dk, dv,
                                   _lib.BF16, x["ws"], x["wsb"], None, C, x["gate"], x["pre"])
    cases = [(dict(pre=8), UNSUP), (dict(pre=QK | 16), UNSUP), (dict(wsb=plain), WS), (dict(wsb=wsb - 1), WS),
             (dict(g=a["g"] + 1), MISAL), (dict(g=None), NULL),
             (dict(dg=a["g"] + tok * dk * 2 - 4), ALIAS),       # the bf16 gate's last element
             (dict(pre=QK, g=a["g"] + 4), MISAL),              # fp32 gate read by the stages: 8 bytes
             (dict(pre=QK | SP, dg=a["g"] + tok * dk * 2), ALIAS)]   # an fp32 gate tensor is twice as long
    for change, code in cases:
        b = dict(a)
        b.update(change)
        assert call(b) == code, (change, code)
    if not HAS_GPU:
        assert call(a) == HIP
        assert call(dict(a, g=a["g"] + 2)) == HIP               # element alignment is enough here
        assert call(dict(a, dg=a["g"] + tok * dk * 2)) == HIP   # just past the bf16 gate: no overlap
        assert call(dict(a, pre=SP, g=a["g"] + 4)) == HIP       # fp32 a, only read elementwise
