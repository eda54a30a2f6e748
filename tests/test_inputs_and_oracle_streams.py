"""Seeded inputs and the oracle on the tiny single-head workload at full size."""
import numpy as np

from fixed_budget_learned_amd.configs import TINY, BATCH64_SERVING, WORKLOADS
from fixed_budget_learned_amd.inputs import TokenStream, prompt_lengths
from oracle import KVpopOracle, kept_by_definition


def test_inputs_are_deterministic_and_distinct():
    a = TokenStream(TINY, 0, 0, 0, 64)
    b = TokenStream(TINY, 0, 0, 0, 64)
    c = TokenStream(TINY, 1, 0, 0, 64)
    for x, y in ((a.k, b.k), (a.v, b.v), (a.scores, b.scores), (a.q, b.q)):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.k, c.k)
    assert not np.array_equal(a.k, a.v)


def test_leaving_scores_are_delayed_by_the_window():
    """Decode step i hands over the score of position P + i - W (delayed readout)."""
    w = WORKLOADS[2]
    ts = TokenStream(w, 0, 0, 300, 40)
    sl = ts.step_leaving_scores()
    for i in range(40):
        t = 300 + i - w.n_recent
        assert np.array_equal(sl[i], ts.scores[:, t])


def test_prompt_lengths_batched_workload():
    P = prompt_lengths(BATCH64_SERVING)
    assert P.shape == (64,) and P.min() >= 4096 and P.max() <= 32768
    assert len(set(P.tolist())) > 50


def test_quantized_lognormal_scores_have_256_levels():
    from fixed_budget_learned_amd.inputs import draw_scores, rng_for
    x = draw_scores(rng_for(5, 0, 0, 2), "qlognormal256", (8, 20000))
    lv = np.unique(x)
    assert lv.min() >= 0 and lv.max() <= 255 / 32 and len(lv) <= 256
    assert np.array_equal(lv * 32, np.round(lv * 32))


def test_tiny_workload_full_stream_matches_definition():
    w = TINY
    ts = TokenStream(w, 0, 0, 0, w.decode_steps)
    orc = KVpopOracle(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_scored, w.n_recent)
    sl = ts.step_leaving_scores()
    kv_k, kv_v = ts.step_kv()
    for n in range(w.decode_steps):
        orc.decode(ts.q[n], kv_k[n], kv_v[n], sl[n])
        assert orc.kept(0) == kept_by_definition(ts.scores[0], n, w.n_sink, w.n_scored, w.n_recent)
        assert len(orc.kept(0)) == min(w.budget, n + 1)
