"""Host model of the packed-batch offset pass (CPU).

The device pass turns the caller's cu_seqlens[N+1] into clamped token offsets
cu_tok[i] = min(T, max(0, cu_seqlens[0..i])) (a running maximum) and chunk
offsets cu_chunks; sequence s is tokens [cu_tok[s], cu_tok[s+1]).  The
workspace and the intra grid hold ceil(T/C) + N chunk units per head, so no
offsets, however malformed, may yield more chunks than that.  This module
restates the pass on the host and checks that bound, and that well-formed
offsets pass through unchanged, over random and adversarial inputs."""
import numpy as np
import pytest


def offsets_pass(cu, T, C):
    """The same arithmetic as the device pass, in 1024-wide blocks with carries."""
    n1 = len(cu)
    cu_tok = np.zeros(n1, np.int64)
    cu_chunks = np.zeros(n1, np.int64)
    carry_max, carry_sum = 0, 0
    for base in range(0, n1, 1024):
        blk = np.clip(np.asarray(cu[base:base + 1024], np.int64), 0, T)
        run = np.maximum(np.maximum.accumulate(blk), carry_max)
        prev = np.concatenate([[carry_max], run[:-1]])
        cnt = (run - prev + C - 1) // C
        if base == 0:
            cnt[0] = 0                      # index 0 ends no sequence
        cu_tok[base:base + len(blk)] = run
        cu_chunks[base:base + len(blk)] = carry_sum + np.cumsum(cnt)
        carry_sum = int(cu_chunks[base + len(blk) - 1])
        carry_max = int(run[-1])
    return cu_tok, cu_chunks


def check(cu, T, C):
    N = len(cu) - 1
    cu_tok, cu_chunks = offsets_pass(cu, T, C)
    assert cu_chunks[0] == 0
    assert np.all(np.diff(cu_tok) >= 0) and cu_tok.min() >= 0 and cu_tok.max() <= T
    lens = np.diff(cu_tok)
    assert np.array_equal(np.diff(cu_chunks), (lens + C - 1) // C)
    assert cu_chunks[-1] <= -(-T // C) + N, (cu_chunks[-1], T, C, N)
    return cu_tok, cu_chunks


@pytest.mark.parametrize("C", [16, 64, 128])
def test_malformed_offsets_stay_within_the_workspace(C):
    r = np.random.default_rng(C)
    T = 1000
    # the case that overlapped before: sequences that restart at 0
    check([0, T, 0, T], T, C)
    check([0, T] * 600 + [0], T, C)         # crosses a 1024-offset block boundary
    check([T + 5, -3, 2 * T, 0, 7], T, C)
    check(list(range(T, -1, -1)), T, C)     # decreasing
    for _ in range(300):
        n = int(r.integers(1, 2500))
        kind = r.integers(0, 3)
        if kind == 0:
            cu = r.integers(-50, T + 50, n + 1)
        elif kind == 1:
            cu = np.sort(r.integers(0, T + 1, n + 1))[::-1]
        else:
            cu = np.cumsum(r.integers(-C, 2 * C, n + 1))
        check(cu, T, C)


def test_well_formed_offsets_are_unchanged():
    r = np.random.default_rng(0)
    for _ in range(200):
        n = int(r.integers(1, 3000))
        T = int(r.integers(0, 100000))
        cu = np.sort(np.concatenate([[0, T], r.integers(0, T + 1, n - 1)]))
        cu_tok, cu_chunks = check(cu, T, 64)
        assert np.array_equal(cu_tok, cu)
        assert np.array_equal(np.diff(cu_chunks), (np.diff(cu) + 63) // 64)
