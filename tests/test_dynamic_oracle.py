"""Pins of the oracle's Dynamic backend (CPU only).

The Dynamic backend holds every token that leaves the window and, at each
prune, cuts the scored region back to its top-k.  Checked against a stream
derived by hand (tests/golden/dynamic_hand_stream.json), against the held
set written from its definition at every step and the Static kept set at
every prune, against the Static oracle when a prune follows every step, and
against masked dense attention over the held set.  Planted mistakes at the
bottom fail these pins.
"""
import json
import os

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import (KVpopOracle, bf16_to_f64, held_dynamic_by_definition,
                    kept_by_definition, kv_head_of, masked_dense_attention)
from fixed_budget_learned_amd.inputs import bf16_bits_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(rng, shape):
    return bf16_bits_rne(rng.standard_normal(shape, dtype=np.float32))


def _stream(orc, scores, rng, n_tokens, prune_every, prompt=0, on_step=None):
    """Optionally prefill `prompt` tokens, then decode up to position
    n_tokens - 1, pruning after every prune_every-th decode step.  Calls
    on_step(n, pruned, before) after each step, `before` being the held sets
    just before the prune."""
    if prompt:
        orc.prefill(_bits(rng, (orc.Hkv, prompt, orc.D)), _bits(rng, (orc.Hkv, prompt, orc.D)),
                    scores[:, :prompt])
    for m, n in enumerate(range(prompt, n_tokens), start=1):
        t = n - orc.W
        sl = scores[:, t] if t >= 0 else np.zeros(orc.Hkv, np.float32)
        orc.decode(_bits(rng, (orc.Hq, orc.D)), _bits(rng, (orc.Hkv, orc.D)),
                   _bits(rng, (orc.Hkv, orc.D)), sl, attend=False)
        before = [orc.kept(g) for g in range(orc.Hkv)]
        pruned = m % prune_every == 0
        if pruned:
            orc.prune()
        if on_step is not None:
            on_step(n, pruned, before)


def _hand_case():
    with open(os.path.join(GOLDEN, "dynamic_hand_stream.json")) as f:
        return json.load(f)


def test_dynamic_hand_stream():
    c = _hand_case()
    s, k, W, d = c["n_sink"], c["n_scored"], c["n_recent"], c["prune_every"]
    scores = np.asarray(c["scores"], np.float32)[None, :]
    orc = KVpopOracle(1, 1, 8, s, k, W, dynamic=True)
    last = [-1]

    def check(n, pruned, before):
        assert orc.kept(0) == c["held"][n], f"step {n}"
        if pruned:
            assert before[0] == c["before_prune"][str(n)], f"before prune, step {n}"
            assert kept_by_definition(scores[0], n, s, k, W) == c["held"][n]
            last[0] = n
        assert held_dynamic_by_definition(scores[0], n, last[0], s, k, W) == c["held"][n]

    _stream(orc, scores, np.random.default_rng(0), len(c["held"]), d, on_step=check)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(s=st.integers(0, 3), k=st.integers(0, 6), W=st.integers(1, 6), d=st.integers(1, 7),
       n_tok=st.integers(1, 45), prompt=st.integers(0, 20), Hkv=st.integers(1, 2),
       ties=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_dynamic_streaming_matches_definition(s, k, W, d, n_tok, prompt, Hkv, ties, seed):
    rng = np.random.default_rng(seed)
    prompt = min(prompt, n_tok)
    if ties:
        scores = rng.integers(0, 3, size=(Hkv, n_tok)).astype(np.float32)
    else:
        scores = rng.random((Hkv, n_tok), dtype=np.float32)
    orc = KVpopOracle(2 * Hkv, Hkv, 8, s, k, W, dynamic=True)
    last = [prompt - 1]

    def check(n, pruned, before):
        if pruned:
            last[0] = n
        for g in range(Hkv):
            want = held_dynamic_by_definition(scores[g], n, last[0], s, k, W)
            assert orc.kept(g) == want, (n, g)
            if pruned:
                assert orc.kept(g) == kept_by_definition(scores[g], n, s, k, W)
            # never more than the budget plus the growth since the last prune
            assert len(orc.kept(g)) <= s + k + W + (n - last[0])

    _stream(orc, scores, rng, n_tok, d, prompt=prompt, on_step=check)
    if prompt:
        # right after a prefill the held set is the Static one
        o2 = KVpopOracle(2 * Hkv, Hkv, 8, s, k, W, dynamic=True)
        o2.prefill(_bits(rng, (Hkv, prompt, 8)), _bits(rng, (Hkv, prompt, 8)), scores[:, :prompt])
        for g in range(Hkv):
            assert o2.kept(g) == kept_by_definition(scores[g], prompt - 1, s, k, W)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(s=st.integers(0, 3), k=st.integers(0, 5), W=st.integers(1, 5), n_tok=st.integers(1, 40),
       prompt=st.integers(0, 12), seed=st.integers(0, 2 ** 31 - 1))
def test_prune_every_step_is_the_static_cache(s, k, W, n_tok, prompt, seed):
    """With a prune after every step the Dynamic cache holds exactly what the
    Static one keeps (its replacement rule is separate code), and attends
    identically."""
    Hq, Hkv, D = 4, 2, 8
    prompt = min(prompt, n_tok)
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, 4, size=(Hkv, n_tok)).astype(np.float32)
    dyn = KVpopOracle(Hq, Hkv, D, s, k, W, dynamic=True)
    sta = KVpopOracle(Hq, Hkv, D, s, k, W)
    if prompt:
        kp, vp = _bits(rng, (Hkv, prompt, D)), _bits(rng, (Hkv, prompt, D))
        dyn.prefill(kp, vp, scores[:, :prompt])
        sta.prefill(kp, vp, scores[:, :prompt])
    for n in range(prompt, n_tok):
        q, kn, vn = _bits(rng, (Hq, D)), _bits(rng, (Hkv, D)), _bits(rng, (Hkv, D))
        t = n - W
        sl = scores[:, t] if t >= 0 else np.zeros(Hkv, np.float32)
        dyn.decode(q, kn, vn, sl, attend=False)
        dyn.prune()
        o_sta = sta.decode(q, kn, vn, sl)
        for g in range(Hkv):
            assert dyn.kept(g) == sta.kept(g), (n, g)
        assert np.array_equal(dyn.attend(q), o_sta)


def test_dynamic_attention_is_masked_dense_attention_over_the_held_set():
    """Between prunes the output covers every held row, the grown ones too."""
    Hq, Hkv, D, s, k, W, d, T = 4, 2, 16, 2, 5, 4, 6, 40
    rng = np.random.default_rng(3)
    scores = rng.random((Hkv, T), dtype=np.float32)
    orc = KVpopOracle(Hq, Hkv, D, s, k, W, dynamic=True)
    Ks, Vs = [], []
    last = -1
    for n in range(T):
        q, kn, vn = _bits(rng, (Hq, D)), _bits(rng, (Hkv, D)), _bits(rng, (Hkv, D))
        Ks.append(kn)
        Vs.append(vn)
        t = n - W
        sl = scores[:, t] if t >= 0 else np.zeros(Hkv, np.float32)
        out = orc.decode(q, kn, vn, sl)
        Kall = np.stack(Ks, axis=1)
        Vall = np.stack(Vs, axis=1)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            held = held_dynamic_by_definition(scores[g], n, last, s, k, W)
            want = masked_dense_attention(bf16_to_f64(q[h]), bf16_to_f64(Kall[g]),
                                          bf16_to_f64(Vall[g]), held, orc.scale)
            assert np.abs(out[h] - want).max() < 1e-12
        if (n + 1) % d == 0:
            orc.prune()
            last = n


# ---------------------------------------------------------------------------
# Planted mistakes (in copies of the oracle, on the CPU)
# ---------------------------------------------------------------------------

class _OlderWinsTies(KVpopOracle):
    def prune(self):
        for g in range(self.Hkv):
            S = self.S[g]
            ranked = sorted(S, key=lambda p: (S[p], -p), reverse=True)
            self.S[g] = {p: S[p] for p in ranked[:self.k]}


class _GrowsWithComparison(KVpopOracle):
    """Uses the Static admission rule while growing."""
    def _admit_leaving(self, g, t, score):
        self.dynamic = False
        try:
            super()._admit_leaving(g, t, score)
        finally:
            self.dynamic = True


def _hand_stream_held(cls):
    c = _hand_case()
    scores = np.asarray(c["scores"], np.float32)[None, :]
    orc = cls(1, 1, 8, c["n_sink"], c["n_scored"], c["n_recent"], dynamic=True)
    held = []
    _stream(orc, scores, np.random.default_rng(0), len(c["held"]), c["prune_every"],
            on_step=lambda n, p, b: held.append(orc.kept(0)))
    return held, c["held"]


def test_planted_tie_order_mistake_is_caught():
    got, want = _hand_stream_held(_OlderWinsTies)
    assert got != want


def test_planted_comparison_while_growing_is_caught():
    got, want = _hand_stream_held(_GrowsWithComparison)
    assert got != want
