"""The one-launch decode of several layers (kvpop_decode_step_layers) against
the oracle, and against one kvpop_decode_step per layer.

Each (layer, sequence) is an independent stream with its own seeded inputs
and prompt length, as the call requires; the oracle follows each one on its
own.  Kept sets must match bit for bit at every step, outputs within the
acceptance bar of gpu_harness.  With the split count and the merge forced to
the same values, the one-launch step and the per-layer steps run the same
arithmetic per head, so their outputs must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_harness import (Geo, Stream, check_output, log, make_cache, make_oracle, out_to_f64,
                         to_dev_bf16, to_dev_f32)
from fixed_budget_learned_amd import abi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


def _streams(geo, L, prompts, steps, kind, seed):
    """prompts[l][b]: prompt length of (layer l, sequence b)."""
    return [[Stream(geo, prompts[l][b] + steps, seed * 10007 + l * 101 + b, kind)
             for b in range(len(prompts[l]))] for l in range(L)]


def _step_inputs(streams, prompts, i):
    L, B = len(streams), len(streams[0])
    q = np.stack([np.stack([streams[l][b].q[prompts[l][b] + i] for b in range(B)]) for l in range(L)])
    kn = np.stack([np.stack([streams[l][b].k[:, prompts[l][b] + i] for b in range(B)]) for l in range(L)])
    vn = np.stack([np.stack([streams[l][b].v[:, prompts[l][b] + i] for b in range(B)]) for l in range(L)])
    sl = np.stack([np.stack([streams[l][b].leaving(prompts[l][b] + i) for b in range(B)]) for l in range(L)])
    return q, kn, vn, sl


def _prefill_all(cache, streams, prompts, layer0=0):
    items = []
    for l, row in enumerate(streams):
        for b, s in enumerate(row):
            P = prompts[l][b]
            if P > 0:
                items.append((layer0 + l, b, to_dev_bf16(s.k[:, :P]), to_dev_bf16(s.v[:, :P]),
                              to_dev_f32(s.scores[:, :P])))
    cache.prefill_compact_batch(items)


CASES = [
    # name, geo, prompts [layer][seq], steps, score kind, prune interval
    ("g4_d128_ragged", Geo(8, 2, 128, 4, 60, 16), [[0, 37], [150, 3], [300, 64], [20, 500]], 80,
     "normal", 0),
    ("g1_d64_ties", Geo(2, 2, 64, 2, 40, 8), [[100, 0, 9], [41, 260, 5]], 70, "ties", 0),
    ("g8_d128_signed_zero", Geo(16, 2, 128, 4, 30, 12), [[64, 200], [0, 33], [90, 1]], 50,
     "signed_zero_ties", 0),
    ("dynamic_prunes", Geo(8, 2, 128, 4, 50, 16), [[120, 0], [300, 45], [80, 200]], 64,
     "normal", 9),
    # more heads than the stream-order launch has workgroups (4 x 80 x 2 = 640)
    ("many_heads_d64", Geo(4, 2, 64, 2, 40, 8),
     [[int(x) for x in np.random.default_rng(l).integers(0, 120, 80)] for l in range(4)], 12,
     "normal", 0),
    # few heads with long slot ranges: every chunk its own workgroup, 25 partials per head
    ("few_heads_long", Geo(8, 2, 128, 4, 1500, 64), [[3000], [1800]], 20, "normal", 0),
]


@pytest.mark.parametrize("name,geo,prompts,steps,kind,every", CASES, ids=[c[0] for c in CASES])
def test_layers_against_oracle(name, geo, prompts, steps, kind, every):
    L, B = len(prompts), len(prompts[0])
    log(f"layers {name}: L={L} B={B} geo={geo} steps={steps} prune_every={every}")
    streams = _streams(geo, L, prompts, steps, kind, seed=len(name))
    # one layer more than the launch covers, so the call works on a sub-range
    cache = make_cache(geo, n_layers=L + 1, batch=B, prune_interval=every)
    _prefill_all(cache, streams, prompts, layer0=1)
    Hq, D = geo.n_q_heads, geo.head_dim
    out = torch.empty((L, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs, kept = [], []
    for i in range(steps):
        q, kn, vn, sl = _step_inputs(streams, prompts, i)
        cache.decode_step_layers(1, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn),
                                 to_dev_f32(sl), out)
        outs.append(out_to_f64(out))
        kept.append([[cache.state(1 + l, b) for b in range(B)] for l in range(L)])
    assert cache.state(0, 0).n == -1, "the layer outside the range was touched"
    cache.close()
    worst = 0.0
    for l in range(L):
        for b in range(B):
            s, P = streams[l][b], prompts[l][b]
            orc = make_oracle(geo, dynamic=every > 0)
            if P > 0:
                orc.prefill(s.k[:, :P], s.v[:, :P], s.scores[:, :P])
            for i in range(steps):
                n = P + i
                ref = orc.decode(s.q[n], s.k[:, n], s.v[:, n], s.leaving(n))
                if every > 0 and (i + 1) % every == 0:
                    orc.prune()
                st = kept[i][l][b]
                assert st.n == orc.n
                for g in range(geo.n_kv_heads):
                    assert st.kept[g].tolist() == orc.kept(g), f"layer {l} seq {b} step {i} head {g}"
                worst = max(worst, check_output(outs[i][l, b], ref, f"layer {l} seq {b} step {i}")[0])
    log(f"  ok, worst max|err| {worst:.2e}")


def test_layers_bit_identical_to_per_layer_steps():
    """Same split count and merge for both: identical bits."""
    geo = Geo(32, 8, 128, 4, 3772, 256)
    L, P, steps = 3, 5000, 40
    prompts = [[P] for _ in range(L)]
    streams = _streams(geo, L, prompts, steps, "normal", seed=3)
    runs = {}
    for mode in ("layers", "per_layer"):
        cache = make_cache(geo, n_layers=L, batch=1, decode_splits=6, decode_finish=2)
        _prefill_all(cache, streams, prompts)
        out = torch.empty((L, 1, geo.n_q_heads, geo.head_dim), dtype=torch.bfloat16, device="cuda")
        outs = []
        for i in range(steps):
            q, kn, vn, sl = (to_dev_bf16(x) if x.dtype == np.uint16 else to_dev_f32(x)
                             for x in _step_inputs(streams, prompts, i))
            if mode == "layers":
                cache.decode_step_layers(0, q, kn, vn, sl, out)
            else:
                for l in range(L):
                    cache.decode_step(l, q[l], kn[l], vn[l], sl[l], out[l])
            outs.append(out.view(torch.int16).cpu().numpy().copy())
        runs[mode] = (outs, [[k.tolist() for k in cache.state(l, 0).kept] for l in range(L)])
        cache.close()
    assert runs["layers"][1] == runs["per_layer"][1]
    for i, (x, y) in enumerate(zip(runs["layers"][0], runs["per_layer"][0])):
        assert np.array_equal(x, y), f"step {i}: outputs differ"


def test_layers_errors():
    geo = Geo(4, 1, 64, 2, 10, 4)
    cache = make_cache(geo, n_layers=2, max_positions=8)
    q = torch.zeros((2, 1, 4, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((2, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    sl = torch.zeros((2, 1, 1), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(abi.KVpopError) as e:     # layers 1 .. 2 of a 2-layer cache
        cache.decode_step_layers(1, q, kv, kv, sl, out)
    assert e.value.code == abi.KVPOP_EINVAL
    for _ in range(8):                            # positions 0 .. 7
        cache.decode_step_layers(0, q, kv, kv, sl, out)
    with pytest.raises(abi.KVpopError) as e:      # position 8 is past max_positions - 1
        cache.decode_step_layers(0, q, kv, kv, sl, out)
    assert e.value.code == abi.KVPOP_ESTATE
    assert cache.state(0, 0).n == 7 and cache.state(1, 0).n == 7
    cache.close()
