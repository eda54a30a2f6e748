"""Pins of the oracle's prefix top-k thresholds (CPU only).

thr(n) is the key of the k-th most important candidate of Cand(n) = {s ..
n - W}, 0 while fewer than k candidates exist, KEY_NONE when k = 0.  The
oracle computes it with a min-heap sweep; here it is checked against the
sorted prefix written from the definition, against the streaming cache's
scored set at every step, against closed forms, and the key encoding against
IEEE-754 facts.
"""
import struct

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import KEY_NONE, KVpopOracle, prefix_thresholds, score_key
from fixed_budget_learned_amd.inputs import bf16_bits_rne


def _thr_by_definition(scores_g, n_tokens, s, k, W):
    """Sorted prefix, k-th element: the definition written out."""
    out = []
    for n in range(n_tokens):
        cand = list(range(s, n - W + 1))
        if k == 0:
            out.append(KEY_NONE)
        elif len(cand) < k:
            out.append(0)
        else:
            ranked = sorted(cand, key=lambda t: (float(scores_g[t]), t), reverse=True)
            t = ranked[k - 1]
            out.append(score_key(scores_g[t], t))
    return out


def _f32(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


# ---------------------------------------------------------------------------
# Key encoding
# ---------------------------------------------------------------------------

def test_score_key_ieee_facts():
    # 1.0f is 0x3F800000: a non-negative float gets its sign bit set
    assert score_key(1.0, 0) == 0xBF800000 << 32
    # -1.0f is 0xBF800000: a negative float has every bit flipped
    assert score_key(-1.0, 5) == (0x407FFFFF << 32) | 5
    # -0 and +0 are the same score
    assert score_key(-0.0, 7) == score_key(0.0, 7) == (0x80000000 << 32) | 7
    # +inf 0x7F800000 and -inf 0xFF800000
    assert score_key(float("inf"), 0) == 0xFF800000 << 32
    assert score_key(float("-inf"), 0) == 0x007FFFFF << 32
    # the smallest positive subnormal sits just above zero
    assert score_key(_f32(1), 0) == 0x80000001 << 32


@settings(max_examples=300, deadline=None)
@given(a=st.floats(width=32, allow_nan=False), b=st.floats(width=32, allow_nan=False),
       pa=st.integers(0, 1000), pb=st.integers(0, 1000))
def test_score_key_orders_like_score_then_position(a, b, pa, pb):
    fa, fb = float(np.float32(a)), float(np.float32(b))
    assert ((fa, pa) < (fb, pb)) == (score_key(fa, pa) < score_key(fb, pb))
    assert ((fa, pa) == (fb, pb)) == (score_key(fa, pa) == score_key(fb, pb))


# ---------------------------------------------------------------------------
# Thresholds
# ---------------------------------------------------------------------------

@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(s=st.integers(0, 4), k=st.integers(0, 9), W=st.integers(1, 8),
       n=st.integers(0, 60), levels=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_thresholds_equal_sorted_prefix(s, k, W, n, levels, seed):
    rng = np.random.default_rng(seed)
    scores = (rng.integers(0, levels, size=n) - levels // 2).astype(np.float32)
    assert prefix_thresholds(scores, n, s, k, W) == _thr_by_definition(scores, n, s, k, W)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(s=st.integers(0, 3), k=st.integers(0, 6), W=st.integers(1, 6),
       n=st.integers(1, 50), seed=st.integers(0, 2**31 - 1))
def test_thresholds_give_the_streamed_scored_set(s, k, W, n, seed):
    """{t in Cand(n) : key(t) >= thr(n)} is the streaming cache's scored set."""
    rng = np.random.default_rng(seed)
    H = 2
    scores = rng.integers(0, 3, size=(H, n)).astype(np.float32)
    thr = [prefix_thresholds(scores[g], n, s, k, W) for g in range(H)]
    orc = KVpopOracle(1 * H, H, 8, s, k, W)
    for p in range(n):
        t = p - W
        sl = scores[:, t] if t >= 0 else np.zeros(H, np.float32)
        orc.decode(bf16_bits_rne(rng.standard_normal((H, 8), dtype=np.float32)),
                   bf16_bits_rne(rng.standard_normal((H, 8), dtype=np.float32)),
                   bf16_bits_rne(rng.standard_normal((H, 8), dtype=np.float32)), sl,
                   attend=False)
        for g in range(H):
            cand = range(s, p - W + 1)
            by_thr = {c for c in cand if score_key(scores[g][c], c) >= thr[g][p]}
            assert by_thr == set(orc.S[g]), (p, g)


def test_thresholds_closed_forms():
    s, k, W, n = 3, 5, 4, 40
    inc = np.arange(n, dtype=np.float32)
    thr = prefix_thresholds(inc, n, s, k, W)
    for p in range(n):
        m = p - W - s + 1
        if m < k:
            assert thr[p] == 0
        else:  # the newest k candidates are kept: the k-th is p - W - k + 1
            assert thr[p] == score_key(inc[p - W - k + 1], p - W - k + 1)
    dec = -np.arange(n, dtype=np.float32)
    thr = prefix_thresholds(dec, n, s, k, W)
    for p in range(n):
        if p - W - s + 1 >= k:  # the oldest k stay forever
            assert thr[p] == score_key(dec[s + k - 1], s + k - 1)
    assert prefix_thresholds(inc, n, s, 0, W) == [KEY_NONE] * n


def test_thresholds_never_decrease():
    rng = np.random.default_rng(3)
    sc = rng.standard_normal(3000).astype(np.float32)
    thr = prefix_thresholds(sc, 3000, 4, 100, 64)
    assert all(a <= b for a, b in zip(thr, thr[1:]))


def test_planted_tie_mistake_is_caught():
    """Thresholds with the tie order flipped (older wins) fail the definition."""
    scores = np.array([1, 1, 1, 1, 1, 1, 1, 1], np.float32)
    s, k, W, n = 0, 2, 1, 8
    ref = _thr_by_definition(scores, n, s, k, W)
    wrong = []
    for p in range(n):
        cand = list(range(s, p - W + 1))
        if len(cand) < k:
            wrong.append(0)
        else:
            ranked = sorted(cand, key=lambda t: (float(scores[t]), -t), reverse=True)
            wrong.append(score_key(scores[ranked[k - 1]], ranked[k - 1]))
    assert wrong != ref
    assert prefix_thresholds(scores, n, s, k, W) == ref
