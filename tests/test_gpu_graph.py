"""Captured HIP graphs replay the hot path exactly.

A pass of reset + prefill + decode steps (and the prefix thresholds and the
future-attention target) is captured once and replayed several times, with
eager work and synchronisations in between.  Every replay must reproduce the
eager pass bit for bit: every step's output, the final kept sets, and the
thresholds and targets.  The kernels are deterministic (fixed merge orders),
and no library call records a memset into the graph.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Geo, Stream, log, make_cache, to_dev_bf16, to_dev_f32
from fixed_budget_learned_amd import abi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


CASES = [
    # name, geo, prompt, steps, decode_splits, prune_interval
    ("static_multi_split", Geo(8, 2, 128, 4, 300, 32), 2000, 40, 0, 0),
    ("static_single_split", Geo(8, 2, 64, 4, 300, 32), 1500, 40, 1, 0),
    ("dynamic_prunes_in_graph", Geo(8, 2, 128, 4, 200, 16), 1200, 48, 0, 16),
]


@pytest.mark.parametrize("name,geo,P,steps,splits,every", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, geo, P, steps, splits, every):
    log(f"graph {name}: geo={geo} P={P} steps={steps} splits={splits} prune_every={every}")
    s = Stream(geo, P + steps, 31, "ties")
    Hq, Hkv, D = geo.n_q_heads, geo.n_kv_heads, geo.head_dim
    pk, pv, ps = to_dev_bf16(s.k[:, :P]), to_dev_bf16(s.v[:, :P]), to_dev_f32(s.scores[:, :P])
    q = to_dev_bf16(np.stack([s.q[P + i] for i in range(steps)])[:, None])
    kn = to_dev_bf16(np.stack([s.k[:, P + i] for i in range(steps)])[:, None])
    vn = to_dev_bf16(np.stack([s.v[:, P + i] for i in range(steps)])[:, None])
    sl = to_dev_f32(np.stack([s.leaving(P + i) for i in range(steps)])[:, None])
    qf, kf = to_dev_bf16(s.q[:P].transpose(1, 0, 2)), pk
    out = torch.zeros((steps, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    thr = torch.zeros((Hkv, P), dtype=torch.int64, device="cuda")
    work = torch.zeros((2, Hq, P), dtype=torch.float32, device="cuda")
    y = torch.zeros((Hkv, P), dtype=torch.float32, device="cuda")
    # the Dynamic prune clock counts every decode step of the cache's life:
    # eager pass and capture each take `steps` steps, so with steps a multiple
    # of the interval every pass sees the prunes at the same steps
    assert every == 0 or steps % every == 0
    cache = make_cache(geo, decode_splits=splits, prune_interval=every, max_positions=P + steps)

    def one_pass():
        cache.reset(0, 0)
        cache.prefill_compact(0, 0, pk, pv, ps)
        for i in range(steps):
            cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out[i])
        cache.prefix_thresholds(ps, thr)
        cache.future_attention_target(qf, kf, work, y)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        one_pass()
    torch.cuda.synchronize()
    want_out = out.clone()
    want_thr, want_y = thr.clone(), y.clone()
    want_kept = cache.state(0, 0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        one_pass()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        thr.zero_()
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), f"replay {rep}: outputs"
        assert torch.equal(thr, want_thr), f"replay {rep}: thresholds"
        assert torch.equal(y, want_y), f"replay {rep}: future target"
        st = cache.state(0, 0)
        assert st.n == want_kept.n == P + steps - 1
        for h in range(Hkv):
            assert st.kept[h].tolist() == want_kept.kept[h].tolist(), f"replay {rep}: head {h}"
        # eager work between replays
        junk = torch.randn(1 << 20, device="cuda")
        junk.mul_(2.0).sum().item()
    del g
    cache.close()
    log("  replays identical")
