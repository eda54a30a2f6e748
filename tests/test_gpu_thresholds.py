"""Parity of the prefix top-k thresholds kernel (through the C ABI) with the
oracle: every position's threshold key must match bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Geo, log, make_cache, to_dev_bf16, to_dev_f32
from fixed_budget_learned_amd import abi
from fixed_budget_learned_amd.inputs import bf16_bits_rne
from oracle import prefix_thresholds, score_key

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


def _scores(kind, H, P, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((H, P), dtype=np.float32)
    if kind == "ties":
        return rng.integers(0, 5, size=(H, P)).astype(np.float32)
    if kind == "increasing":
        return np.tile(np.arange(P, dtype=np.float32), (H, 1))
    if kind == "decreasing":
        return np.tile(-np.arange(P, dtype=np.float32), (H, 1))
    if kind == "qlog":
        z = rng.standard_normal((H, P))
        return (np.minimum(255.0, np.floor(32.0 * np.exp(z))) / 32.0).astype(np.float32)
    raise ValueError(kind)


def _gpu_thresholds(geo, sc):
    H, P = sc.shape
    cache = make_cache(geo, max_positions=max(P, 1))
    thr = torch.empty((H, P), dtype=torch.int64, device="cuda")
    cache.prefix_thresholds(to_dev_f32(sc), thr)
    got = thr.cpu().numpy().view(np.uint64)
    cache.close()
    return got


CASES = [
    # name, (Hkv, s, k, W), P, scores
    ("one_chunk_ties", (2, 4, 44, 16), 600, "ties"),
    ("multi_chunk_normal", (2, 4, 100, 32), 5000, "normal"),
    ("k_above_candidates", (1, 4, 3000, 16), 2000, "normal"),
    ("prompt_inside_window", (1, 4, 10, 16), 19, "normal"),
    ("no_sink_window_one", (1, 0, 5, 1), 3000, "normal"),
    ("ties_across_chunks", (2, 4, 2000, 64), 9000, "ties"),
    ("largest_k", (1, 4, 4096, 64), 10000, "qlog"),
    ("increasing", (1, 4, 300, 16), 4000, "increasing"),
    ("decreasing", (1, 4, 300, 16), 4000, "decreasing"),
    ("exact_chunk_multiple", (1, 4, 500, 12), 4 + 12 + 3 * 1024, "normal"),
    ("k_one_long", (1, 4, 1, 16), 20000, "normal"),               # 4,096-candidate chunks
    ("k_two_ties", (2, 4, 2, 8), 9000, "ties"),
    ("increasing_overflow", (1, 4, 100, 16), 12000, "increasing"),  # every candidate enters
    ("decreasing_segments", (1, 4, 300, 16), 12000, "decreasing"),   # every segment starts from the first k
    ("largest_k_32_segments", (1, 4, 4096, 64), 40000, "normal"),
    ("qwen3_8b_layer_4x", (8, 4, 3772, 256), 16384, "normal"),
    ("long_context_131k", (8, 4, 1788, 256), 131072, "normal"),
    # segment starts over prefixes of 16k+ candidates with a small kept
    # fraction keep the candidates at or above a sampled threshold; ties
    # (a fifth of the scores share the top value) overflow that and take
    # the exact select, monotone scores put the whole top k at one end
    ("sampled_starts_ties", (2, 4, 700, 64), 60000, "ties"),
    ("sampled_starts_increasing", (1, 4, 700, 16), 60000, "increasing"),
    ("sampled_starts_decreasing", (1, 4, 700, 16), 60000, "decreasing"),
    ("sampled_starts_qlog", (2, 0, 1500, 1), 90000, "qlog"),
]


@pytest.mark.parametrize("name,g,P,kind", CASES, ids=[c[0] for c in CASES])
def test_thresholds_match_oracle(name, g, P, kind):
    H, s, k, W = g
    geo = Geo(H, H, 64, s, k, W)
    sc = _scores(kind, H, P, seed=len(name) * 7919 + P)
    log(f"thresholds {name}: Hkv={H} s={s} k={k} W={W} P={P} scores={kind}")
    got = _gpu_thresholds(geo, sc)
    for h in range(H):
        want = np.array(prefix_thresholds(sc[h], P, s, k, W), dtype=np.uint64)
        bad = np.nonzero(got[h] != want)[0]
        assert bad.size == 0, (f"head {h}: {bad.size} positions differ, first at {bad[0]}: "
                               f"got {got[h][bad[0]]:#x} want {want[bad[0]]:#x}")


def test_no_scored_slots_gives_key_none():
    geo = Geo(2, 2, 64, 2, 0, 8)
    got = _gpu_thresholds(geo, _scores("normal", 2, 300, 1))
    assert (got == np.uint64(0xFFFFFFFFFFFFFFFF)).all()


def test_thresholds_reproduce_the_prefilled_kept_set():
    """Bulk check: after a prefill of P tokens the cache holds the sinks, the
    window and the candidates whose key reaches thr[P-1]."""
    H, s, k, W, P = 4, 4, 700, 64, 12000
    geo = Geo(2 * H, H, 64, s, k, W)
    rng = np.random.default_rng(11)
    sc = rng.standard_normal((H, P), dtype=np.float32)
    kk = bf16_bits_rne(rng.standard_normal((H, P, 64), dtype=np.float32))
    vv = bf16_bits_rne(rng.standard_normal((H, P, 64), dtype=np.float32))
    got = _gpu_thresholds(geo, sc)
    cache = make_cache(geo, max_positions=P)
    cache.prefill_compact(0, 0, to_dev_bf16(kk), to_dev_bf16(vv), to_dev_f32(sc))
    st = cache.state(0, 0)
    cache.close()
    for h in range(H):
        t = int(got[h][P - 1])
        want = set(range(s)) | set(range(P - W, P))
        want |= {c for c in range(s, P - W) if score_key(sc[h][c], c) >= t}
        assert set(st.kept[h].tolist()) == want
