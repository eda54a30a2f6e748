"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Kept sets must match bit-exactly; attention outputs within
max|err| <= 2e-2 and relative L2 err <= 1e-2 (see gpu_harness).  The GPU
side runs first and its results are copied to the host; the oracle then
replays the same seeded inputs.
"""
import zlib

import numpy as np
import pytest
import torch

from gpu_harness import (Geo, Stream, check_kept, check_output, log, make_cache, make_oracle,
                         out_to_f64, to_dev_bf16, to_dev_f32)
from fixed_budget_learned_amd import abi
from fixed_budget_learned_amd.configs import (BATCH64_SERVING, LONG_131K_8X, QWEN3_8B_36L_4X,
                                              QWEN3_8B_LAYER_4X, TINY)
from fixed_budget_learned_amd.inputs import TokenStream, prompt_lengths
from oracle import KVpopOracle, bf16_to_f64, kept_by_definition

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


def _geo(w):
    return Geo(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_scored, w.n_recent)


# ---------------------------------------------------------------------------
# Generic driver: B sequences with ragged prompts, then `steps` decode steps
# ---------------------------------------------------------------------------

def run_case(geo: Geo, prompts, steps, score_kind="uniform", seed=0, splits=0,
             check_every=1, out_every=1, layer=0, n_layers=1):
    B = len(prompts)
    streams = [Stream(geo, P + steps, seed * 1000 + b, score_kind) for b, P in enumerate(prompts)]
    cache = make_cache(geo, n_layers=n_layers, batch=B, decode_splits=splits)
    log(f"case geo={geo} prompts={prompts} steps={steps} scores={score_kind} splits={splits}")
    for b, P in enumerate(prompts):
        if P > 0:
            cache.prefill_compact(layer, b, to_dev_bf16(streams[b].k[:, :P]),
                                  to_dev_bf16(streams[b].v[:, :P]), to_dev_f32(streams[b].scores[:, :P]))
    torch.cuda.synchronize()
    gpu_kept = {}
    gpu_out = {}

    def snap_kept(i):
        for b in range(B):
            gpu_kept[(i, b)] = cache.state(layer, b)

    snap_kept(-1)
    H, Hq, D = geo.n_kv_heads, geo.n_q_heads, geo.head_dim
    q = np.stack([np.stack([s.q[P + i] for s, P in zip(streams, prompts)]) for i in range(steps)])
    kn = np.stack([np.stack([s.k[:, P + i] for s, P in zip(streams, prompts)]) for i in range(steps)])
    vn = np.stack([np.stack([s.v[:, P + i] for s, P in zip(streams, prompts)]) for i in range(steps)])
    sl = np.stack([np.stack([s.leaving(P + i) for s, P in zip(streams, prompts)]) for i in range(steps)])
    qd, kd, vd, sd = to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), to_dev_f32(sl)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    for i in range(steps):
        cache.decode_step(layer, qd[i], kd[i], vd[i], sd[i], out)
        if i % out_every == 0 or i == steps - 1:
            gpu_out[i] = out_to_f64(out)
        if i % check_every == 0 or i == steps - 1:
            snap_kept(i)
    torch.cuda.synchronize()
    cache.close()

    for b, P in enumerate(prompts):
        s = streams[b]
        orc = make_oracle(geo)
        if P > 0:
            orc.prefill(s.k[:, :P], s.v[:, :P], s.scores[:, :P])
        _cmp_kept(gpu_kept[(-1, b)], orc, f"b={b} after prefill")
        worst = 0.0
        for i in range(steps):
            n = P + i
            assert np.array_equal(sl[i, b], s.scores[:, n - geo.n_recent]) if n - geo.n_recent >= 0 else True
            ref = orc.decode(s.q[n], s.k[:, n], s.v[:, n], sl[i, b], attend=(i in gpu_out))
            if i in gpu_out:
                mx, _ = check_output(gpu_out[i][b], ref, f"b={b} step {i}")
                worst = max(worst, mx)
            if (i, b) in gpu_kept:
                _cmp_kept(gpu_kept[(i, b)], orc, f"b={b} step {i}")
        log(f"  seq {b}: P={P} ok, worst max|err| {worst:.2e}")


def _cmp_kept(st, orc, what):
    assert st.n == orc.n, f"{what}: n {st.n} != {orc.n}"
    assert st.flags == 0, f"{what}: flags {st.flags}"
    for g in range(orc.Hkv):
        want = orc.kept(g)
        got = st.kept[g].tolist()
        if got != want:
            raise AssertionError(f"{what}: head {g}: |got|={len(got)} |want|={len(want)} "
                                 f"missing {sorted(set(want) - set(got))[:8]} "
                                 f"extra {sorted(set(got) - set(want))[:8]}")


# ---------------------------------------------------------------------------
# Small and ragged cases, every step
# ---------------------------------------------------------------------------

CASES = [
    ("g1_d64_from_empty", Geo(1, 1, 64, 4, 44, 16), [0], 150, "uniform", 0),
    ("g4_d128_ragged_batch", Geo(8, 2, 128, 4, 100, 32), [0, 37, 500], 120, "uniform", 0),
    ("g8_d64_ties", Geo(16, 2, 64, 2, 50, 8), [300, 3], 100, "ties", 0),
    ("g2_d128_no_sink_signed_zero", Geo(4, 2, 128, 0, 20, 5), [100, 1], 60, "signed_zero_ties", 0),
    ("k0_sink_plus_window", Geo(4, 1, 128, 4, 0, 16), [64], 40, "uniform", 0),
    ("short_prompts", Geo(4, 1, 64, 4, 30, 16), [1, 2, 4, 5, 19, 20, 21, 50], 50, "normal", 0),
    ("increasing_scores", Geo(4, 2, 128, 4, 40, 16), [200], 60, "increasing", 0),
    ("decreasing_scores", Geo(4, 2, 128, 4, 40, 16), [200], 60, "decreasing", 0),
    ("infinite_scores", Geo(8, 1, 128, 3, 60, 12), [400], 60, "inf", 0),
    ("one_split", Geo(8, 2, 128, 4, 500, 64), [3000, 700], 40, "normal", 1),
    ("max_splits", Geo(8, 2, 128, 4, 500, 64), [3000, 700], 40, "normal", 256),
    ("odd_splits", Geo(8, 2, 128, 4, 500, 64), [3000, 700], 40, "ties", 7),
    ("big_budget_multi_chunk", Geo(32, 8, 128, 4, 6000, 256), [9000], 30, "normal", 0),
    ("gqa8_d128", Geo(64, 8, 128, 4, 200, 32), [1000], 30, "normal", 0),
    # a scored region that can hold every candidate never evicts: dense attention
    ("dense_no_eviction", Geo(8, 2, 128, 4, 10000, 32), [3000, 57, 0], 40, "normal", 0),
    ("dense_prompt_fills_region_exactly", Geo(8, 2, 128, 4, 200, 16), [220], 30, "ties", 0),
    # 256 KV heads in all: one workgroup per head, no cross-workgroup merge
    ("auto_single_split_256_heads", Geo(2, 2, 64, 4, 40, 16),
     [(37 * i) % 300 for i in range(128)], 30, "ties", 0),
    # slot ranges rounded up to whole passes leave the last split empty
    ("empty_last_split", Geo(4, 1, 128, 4, 64, 32), [150, 20], 40, "normal", 3),
    ("single_split_g8_d64", Geo(16, 2, 64, 4, 700, 64), [2000, 90], 30, "normal", 1),
    # prompts longer than one workgroup's registers hold: two-level select
    # (slices of 16k candidates, tie-heavy across slice borders; 32k slices),
    # and the streaming select when the union of the slices is too large
    ("two_level_16k_slices_ties", Geo(4, 1, 64, 4, 500, 16), [40000], 20, "ties", 0),
    ("two_level_32k_slices", Geo(8, 2, 128, 4, 5000, 32), [70000], 10, "normal", 0),
    ("long_prompt_streaming_select", Geo(4, 1, 64, 4, 20000, 16), [40000], 10, "normal", 0),
]


@pytest.mark.parametrize("name,geo,prompts,steps,kind,splits", CASES, ids=[c[0] for c in CASES])
def test_small_cases(name, geo, prompts, steps, kind, splits):
    run_case(geo, prompts, steps, kind, seed=zlib.crc32(name.encode()) % 1000, splits=splits)


def test_tiny_workload_every_step():
    """Tiny single head, 512 tokens decoded from an empty cache."""
    w = TINY
    geo = _geo(w)
    ts = TokenStream(w, 0, 0, 0, w.decode_steps)
    kk, vv = ts.step_kv()
    sl = ts.step_leaving_scores()
    cache = make_cache(geo)
    qd, kd, vd, sd = to_dev_bf16(ts.q), to_dev_bf16(kk), to_dev_bf16(vv), to_dev_f32(sl)
    out = torch.empty((1, 1, w.head_dim), dtype=torch.bfloat16, device="cuda")
    outs, kept = [], []
    for n in range(w.decode_steps):
        cache.decode_step(0, qd[n:n + 1], kd[n:n + 1], vd[n:n + 1], sd[n:n + 1], out)
        outs.append(out_to_f64(out)[0])
        kept.append(cache.state(0, 0).kept[0].tolist())
    cache.close()
    orc = make_oracle(geo)
    for n in range(w.decode_steps):
        ref = orc.decode(ts.q[n], kk[n], vv[n], sl[n])
        assert kept[n] == orc.kept(0) == kept_by_definition(ts.scores[0], n, w.n_sink, w.n_scored, w.n_recent)
        check_output(outs[n], ref, f"step {n}")


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def _full_layer(w, layer, steps, n_layers=1, cache=None, check_every=64, out_every=16, seq=0):
    geo = _geo(w)
    P = int(prompt_lengths(w)[seq])
    ts = TokenStream(w, layer, seq, P, steps)
    own = cache is None
    if own:
        cache = make_cache(geo, n_layers=n_layers, batch=1)
    log(f"{w.name} layer {layer}: P={P} steps={steps}")
    cache.prefill_compact(layer, 0, to_dev_bf16(ts.prompt_k()), to_dev_bf16(ts.prompt_v()),
                          to_dev_f32(ts.prompt_scores()))
    kk, vv = ts.step_kv()
    sl = ts.step_leaving_scores()
    qd, kd, vd, sd = to_dev_bf16(ts.q), to_dev_bf16(kk), to_dev_bf16(vv), to_dev_f32(sl)
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kept = {-1: cache.state(layer, 0)}
    outs = {}
    for i in range(steps):
        cache.decode_step(layer, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], sd[i:i + 1], out)
        if i % out_every == 0 or i == steps - 1:
            outs[i] = out_to_f64(out)[0]
        if i % check_every == 0 or i == steps - 1:
            kept[i] = cache.state(layer, 0)
    torch.cuda.synchronize()
    if own:
        cache.close()
    orc = make_oracle(geo)
    orc.prefill(ts.prompt_k(), ts.prompt_v(), ts.prompt_scores())
    _cmp_kept(kept[-1], orc, "after prefill")
    # the prefill kept set also equals the definition written out directly
    for g in (0, w.n_kv_heads - 1):
        assert kept[-1].kept[g].tolist() == kept_by_definition(ts.scores[g], P - 1, w.n_sink,
                                                                w.n_scored, w.n_recent)
    worst = worst_rel = 0.0
    for i in range(steps):
        ref = orc.decode(ts.q[i], kk[i], vv[i], sl[i], attend=(i in outs))
        if i in outs:
            mx, rel = check_output(outs[i], ref, f"step {i}")
            worst, worst_rel = max(worst, mx), max(worst_rel, rel)
        if i in kept:
            _cmp_kept(kept[i], orc, f"step {i}")
    log(f"  ok, worst max|err| {worst:.3e}, worst L2-rel {worst_rel:.3e}")


@pytest.mark.timeout(600)
def test_qwen3_8b_layer_full():
    """One Qwen3-8B layer at 4x: prefill 16,384 then 1,024 decode steps."""
    _full_layer(QWEN3_8B_LAYER_4X, 0, QWEN3_8B_LAYER_4X.decode_steps)


# Full-size workloads run past the window: with W = 256, a token appended
# by a decode step leaves the window (and competes for a scored slot) only
# after 256 more steps ("Qwen3-8B-KVpop-4x" model card, "Delayed scoring").
STEPS_PAST_WINDOW = 320
CHECKS = [63, 127, 191, 255, STEPS_PAST_WINDOW - 1]


def _decode_layer(cache, layer, step_inputs, out_steps, check_steps):
    """Decode one layer through kvpop_decode_step; returns outputs and states."""
    qd, kd, vd, sd = step_inputs
    w_hq, w_d = qd.shape[-2], qd.shape[-1]
    out = torch.empty((1, w_hq, w_d), dtype=torch.bfloat16, device="cuda")
    outs, kept = {}, {}
    for i in range(qd.shape[0]):
        cache.decode_step(layer, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], sd[i:i + 1], out)
        if i in out_steps:
            outs[i] = out_to_f64(out)[0]
        if i in check_steps:
            kept[i] = cache.state(layer, 0)
    return outs, kept


def _compare(what, kept_gpu, outs_gpu, kept_ref, outs_ref):
    """kept_gpu: {step: HeadState}; kept_ref: {step: [per-head sorted lists]}."""
    for i, st in kept_gpu.items():
        for g, want in enumerate(kept_ref[i]):
            got = st.kept[g].tolist()
            assert got == want, (f"{what} step {i} head {g}: |got|={len(got)} |want|={len(want)} "
                                 f"missing {sorted(set(want) - set(got))[:8]} "
                                 f"extra {sorted(set(got) - set(want))[:8]}")
    worst_mx = worst_rel = 0.0
    for i, o in outs_gpu.items():
        mx, rel = check_output(o, outs_ref[i], f"{what} step {i}")
        worst_mx, worst_rel = max(worst_mx, mx), max(worst_rel, rel)
    return worst_mx, worst_rel


def _stack_prefill(w, cache, steps):
    """Every layer's prompt of a 36-layer workload, compacted in one batched
    call (as bench.py times it); returns the step inputs of every layer."""
    items, step_in = [], []
    for layer in range(w.n_layers):
        ts = TokenStream(w, layer, 0, w.prompt_len, steps)
        items.append((layer, 0, to_dev_bf16(ts.prompt_k()), to_dev_bf16(ts.prompt_v()),
                      to_dev_f32(ts.prompt_scores())))
        kk, vv = ts.step_kv()
        step_in.append((ts.q, kk, vv, ts.step_leaving_scores()))
        del ts
    cache.prefill_compact_batch(items)
    torch.cuda.synchronize()
    return step_in


@pytest.mark.timeout(900)
def test_qwen3_8b_36_layer_stack():
    """36 layers at 4x: every layer's kept sets after one batched prefill,
    then 320 steps (one launch per layer-step) on layers 0, 17 and 35 with
    kept sets every 64 steps and outputs every 16."""
    from oracle_workers import pool, stream_oracle
    w = QWEN3_8B_36L_4X
    steps, sampled = STEPS_PAST_WINDOW, (0, 17, 35)
    out_steps = list(range(0, steps, 16)) + [steps - 1]
    log(f"{w.name}: batched prefill of {w.n_layers} layers, then {steps} steps on {sampled}")
    cache = make_cache(_geo(w), n_layers=w.n_layers, batch=1)
    step_in = _stack_prefill(w, cache, steps)
    after_prefill = [cache.state(l, 0) for l in range(w.n_layers)]
    gpu = {}
    for layer in sampled:
        q, kk, vv, sl = step_in[layer]
        gpu[layer] = _decode_layer(cache, layer, (to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(vv),
                                                  to_dev_f32(sl)), set(out_steps), set(CHECKS))
    cache.close()
    del step_in
    with pool() as pl:
        jobs = {layer: pl.apply_async(stream_oracle, (w.name, layer, 0, w.prompt_len, steps,
                                                      CHECKS if layer in sampled else [],
                                                      out_steps if layer in sampled else []))
                for layer in range(w.n_layers)}
        refs = {layer: j.get() for layer, j in jobs.items()}
    for layer in range(w.n_layers):
        kept_ref, outs_ref = refs[layer]
        _compare(f"layer {layer} after prefill", {-1: after_prefill[layer]}, {}, kept_ref, {})
        if layer in sampled:
            mx, rel = _compare(f"layer {layer}", gpu[layer][1], gpu[layer][0], kept_ref, outs_ref)
            log(f"  layer {layer}: {steps} steps ok, worst max|err| {mx:.3e}, worst L2-rel {rel:.3e}")
    log(f"  all {w.n_layers} layers' prefill kept sets ok")


@pytest.mark.timeout(900)
def test_qwen3_8b_36_layer_stack_one_launch():
    """36 layers at 4x decoded 320 steps with kvpop_decode_step_layers (every
    layer in one launch, the labelled benchmark path): every layer's kept
    sets after the last step against the definition, outputs of layers 0 and
    35 every 32 steps against the streaming oracle."""
    from oracle_workers import kept_at, pool, stream_oracle
    w = QWEN3_8B_36L_4X
    steps, sampled = STEPS_PAST_WINDOW, (0, 35)
    out_steps = list(range(0, steps, 32)) + [steps - 1]
    log(f"{w.name}: {steps} one-launch steps of all {w.n_layers} layers")
    cache = make_cache(_geo(w), n_layers=w.n_layers, batch=1)
    step_in = _stack_prefill(w, cache, steps)
    q = to_dev_bf16(np.stack([x[0] for x in step_in], axis=1)[:, :, None])
    kk = to_dev_bf16(np.stack([x[1] for x in step_in], axis=1)[:, :, None])
    vv = to_dev_bf16(np.stack([x[2] for x in step_in], axis=1)[:, :, None])
    sl = to_dev_f32(np.stack([x[3] for x in step_in], axis=1)[:, :, None])
    del step_in
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    outs = {layer: {} for layer in sampled}
    for i in range(steps):
        cache.decode_step_layers(0, q[i], kk[i], vv[i], sl[i], out)
        if i in out_steps:
            o = out_to_f64(out)
            for layer in sampled:
                outs[layer][i] = o[layer, 0]
    final = [cache.state(l, 0) for l in range(w.n_layers)]
    cache.close()
    n_last = w.prompt_len + steps - 1
    with pool() as pl:
        kjobs = {l: pl.apply_async(kept_at, (w.name, l, 0, w.prompt_len, steps, [n_last]))
                 for l in range(w.n_layers)}
        ojobs = {l: pl.apply_async(stream_oracle, (w.name, l, 0, w.prompt_len, steps, [], out_steps))
                 for l in sampled}
        kref = {l: j.get() for l, j in kjobs.items()}
        oref = {l: j.get()[1] for l, j in ojobs.items()}
    for l in range(w.n_layers):
        assert final[l].n == n_last
        _compare(f"layer {l} final", {n_last: final[l]}, {}, kref[l], {})
    for l in sampled:
        mx, rel = _compare(f"layer {l}", {}, outs[l], {}, oref[l])
        log(f"  layer {l}: outputs ok, worst max|err| {mx:.3e}, worst L2-rel {rel:.3e}")
    log(f"  all {w.n_layers} layers' kept sets after {steps} steps ok")


@pytest.mark.timeout(900)
def test_long_context_131k():
    """131,072-token prefill at 88 % compression, layers 0 and 35 of a
    36-layer cache, 320 steps each, kept sets every 64 steps, outputs every 16."""
    from oracle_workers import pool, stream_oracle
    w = LONG_131K_8X
    steps, sampled = STEPS_PAST_WINDOW, (0, 35)
    out_steps = list(range(0, steps, 16)) + [steps - 1]
    cache = make_cache(_geo(w), n_layers=w.n_layers, batch=1)
    gpu = {}
    with pool(2) as pl:
        jobs = {l: pl.apply_async(stream_oracle, (w.name, l, 0, w.prompt_len, steps, CHECKS, out_steps))
                for l in sampled}
        for layer in sampled:
            log(f"{w.name} layer {layer}: P={w.prompt_len} steps={steps}")
            ts = TokenStream(w, layer, 0, w.prompt_len, steps)
            cache.prefill_compact(layer, 0, to_dev_bf16(ts.prompt_k()), to_dev_bf16(ts.prompt_v()),
                                  to_dev_f32(ts.prompt_scores()))
            after = cache.state(layer, 0)
            kk, vv = ts.step_kv()
            o, k = _decode_layer(cache, layer, (to_dev_bf16(ts.q), to_dev_bf16(kk), to_dev_bf16(vv),
                                                to_dev_f32(ts.step_leaving_scores())),
                                 set(out_steps), set(CHECKS))
            k[-1] = after
            gpu[layer] = (o, k)
            del ts, kk, vv
            torch.cuda.empty_cache()
        refs = {l: j.get() for l, j in jobs.items()}
    cache.close()
    for layer in sampled:
        mx, rel = _compare(f"layer {layer}", gpu[layer][1], gpu[layer][0], *refs[layer])
        log(f"  layer {layer}: ok, worst max|err| {mx:.3e}, worst L2-rel {rel:.3e}")


@pytest.mark.timeout(900)
def test_batched_serving_b64():
    """64 sequences with drawn prompt lengths and quantized (tied) scores,
    compacted in one batched call, then 320 decode steps: every sequence's
    kept sets every 64 steps against the streaming oracle, outputs of every
    9th sequence every 32 steps."""
    from oracle_workers import pool, stream_oracle
    w = BATCH64_SERVING
    geo = _geo(w)
    steps = STEPS_PAST_WINDOW
    Ps = prompt_lengths(w)
    B = w.batch
    sample = set(range(0, B, 9)) | {B - 1}
    out_steps = list(range(0, steps, 32)) + [steps - 1]
    cache = make_cache(geo, batch=B)
    log(f"batched: prompts {Ps.min()}..{Ps.max()}, {steps} steps")
    pl = pool()
    jobs = {b: pl.apply_async(stream_oracle, (w.name, 0, b, int(Ps[b]), steps, CHECKS,
                                              out_steps if b in sample else []))
            for b in range(B)}
    q = np.zeros((steps, B, w.n_q_heads, w.head_dim), np.uint16)
    kn = np.zeros((steps, B, w.n_kv_heads, w.head_dim), np.uint16)
    vn = np.zeros_like(kn)
    sl = np.zeros((steps, B, w.n_kv_heads), np.float32)
    items = []  # all 64 prompts in one batched call, as bench.py times it
    for b in range(B):
        if b % 16 == 0:
            log(f"  inputs of sequence {b}")
        ts = TokenStream(w, 0, b, int(Ps[b]), steps)
        items.append((0, b, to_dev_bf16(ts.prompt_k()), to_dev_bf16(ts.prompt_v()),
                      to_dev_f32(ts.prompt_scores())))
        k_, v_ = ts.step_kv()
        q[:, b], kn[:, b], vn[:, b], sl[:, b] = ts.q, k_, v_, ts.step_leaving_scores()
        del ts
    cache.prefill_compact_batch(items)
    torch.cuda.synchronize()
    del items
    kept = {-1: [cache.state(0, b) for b in range(B)]}
    qd, kd, vd, sd = to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), to_dev_f32(sl)
    out = torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    outs = {}
    for i in range(steps):
        cache.decode_step(0, qd[i], kd[i], vd[i], sd[i], out)
        if i in out_steps:
            outs[i] = out_to_f64(out)
        if i in CHECKS:
            kept[i] = [cache.state(0, b) for b in range(B)]
    cache.close()
    worst_mx = worst_rel = 0.0
    for b in range(B):
        kept_ref, outs_ref = jobs[b].get()
        mx, rel = _compare(f"seq {b}", {i: kept[i][b] for i in kept},
                           {i: outs[i][b] for i in outs_ref}, kept_ref, outs_ref)
        worst_mx, worst_rel = max(worst_mx, mx), max(worst_rel, rel)
        if b % 16 == 15:
            log(f"  oracle checked sequences 0..{b}")
    pl.close()
    pl.join()
    log(f"  batched ok, worst max|err| {worst_mx:.3e}, worst L2-rel {worst_rel:.3e}")


@pytest.mark.timeout(600)
def test_dense_131k_context():
    """Dense decode (no eviction) over a 131,072-token prompt: every token is
    kept, so the output is plain softmax attention over all positions."""
    P, steps, Hq, Hkv, D, W = 131072, 12, 32, 8, 128, 256
    geo = Geo(Hq, Hkv, D, 4, P + steps, W)
    rng = np.random.default_rng(131072)
    from fixed_budget_learned_amd.inputs import bf16_bits_rne
    T = P + steps
    K = bf16_bits_rne(rng.standard_normal((Hkv, T, D), dtype=np.float32))
    V = bf16_bits_rne(rng.standard_normal((Hkv, T, D), dtype=np.float32))
    Q = bf16_bits_rne(rng.standard_normal((steps, Hq, D), dtype=np.float32))
    S = rng.standard_normal((Hkv, T), dtype=np.float32)
    cache = make_cache(geo, max_positions=T)
    cache.prefill_compact(0, 0, to_dev_bf16(K[:, :P]), to_dev_bf16(V[:, :P]), to_dev_f32(S[:, :P]))
    out = torch.empty((1, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs = []
    for i in range(steps):
        n = P + i
        cache.decode_step(0, to_dev_bf16(Q[i][None]), to_dev_bf16(K[:, n][None]),
                          to_dev_bf16(V[:, n][None]), to_dev_f32(S[:, n - W][None]), out)
        outs.append(out_to_f64(out)[0])
    st = cache.state(0, 0)
    cache.close()
    assert st.n == T - 1
    for g in range(Hkv):
        assert st.kept[g].tolist() == list(range(T))
    from oracle import softmax_attention
    import math
    Kf, Vf = bf16_to_f64(K), bf16_to_f64(V)
    for i in (0, steps - 1):
        n = P + i
        q = bf16_to_f64(Q[i])
        ref = np.stack([softmax_attention(q[h], Kf[h // 4, :n + 1], Vf[h // 4, :n + 1], 1 / math.sqrt(D))
                        for h in range(Hq)])
        check_output(outs[i], ref, f"dense step {i}")


# ---------------------------------------------------------------------------
# Determinism, split invariance, state machine
# ---------------------------------------------------------------------------

def _decode_run(geo, P, steps, splits, seed=7, kind="normal", finish=0):
    s = Stream(geo, P + steps, seed, kind)
    cache = make_cache(geo, decode_splits=splits, decode_finish=finish)
    cache.prefill_compact(0, 0, to_dev_bf16(s.k[:, :P]), to_dev_bf16(s.v[:, :P]),
                          to_dev_f32(s.scores[:, :P]))
    out = torch.empty((1, geo.n_q_heads, geo.head_dim), dtype=torch.bfloat16, device="cuda")
    outs = []
    for i in range(steps):
        n = P + i
        cache.decode_step(0, to_dev_bf16(s.q[n][None]), to_dev_bf16(s.k[:, n][None]),
                          to_dev_bf16(s.v[:, n][None]), to_dev_f32(s.leaving(n)[None]), out)
        outs.append(out.view(torch.int16).cpu().numpy().copy())
    st = cache.state(0, 0)
    cache.close()
    return outs, [k.tolist() for k in st.kept]


def test_deterministic_and_split_invariant():
    geo = Geo(32, 8, 128, 4, 3772, 256)
    a_out, a_kept = _decode_run(geo, 16384, 24, 0)
    b_out, b_kept = _decode_run(geo, 16384, 24, 0)
    assert a_kept == b_kept
    for x, y in zip(a_out, b_out):
        assert np.array_equal(x, y), "two identical runs differ"
    for splits in (1, 2, 33, 256):
        c_out, c_kept = _decode_run(geo, 16384, 24, splits)
        assert c_kept == a_kept
        for x, y in zip(a_out, c_out):
            xf = out_to_f64(torch.from_numpy(x).view(torch.bfloat16))
            yf = out_to_f64(torch.from_numpy(y).view(torch.bfloat16))
            assert np.abs(xf - yf).max() <= 2e-3


@pytest.mark.parametrize("geo,P,steps,splits,kind", [
    (Geo(32, 8, 128, 4, 3772, 256), 16384, 20, 0, "normal"),   # full grid, 128-slot splits
    (Geo(32, 8, 128, 4, 3772, 256), 16384, 20, 16, "ties"),    # 256-slot splits
    (Geo(4, 1, 128, 4, 3772, 256), 9000, 24, 0, "normal"),     # one KV head, 32 splits
    (Geo(16, 2, 64, 4, 7000, 64), 20000, 24, 0, "uniform"),    # D 64, long splits
    (Geo(8, 8, 128, 2, 900, 16), 1500, 40, 7, "ties"),         # odd split count
], ids=["4x_layer", "16_splits", "one_head", "d64_long", "odd"])
def test_split_finishes_identical(geo, P, steps, splits, kind):
    """Merging a head's splits in the last split's workgroup (decode_finish 1)
    and in a second launch (decode_finish 2) run the same arithmetic: outputs
    and kept sets must agree bit for bit, and with the oracle's kept set."""
    log(f"finishes geo={geo} P={P} steps={steps} splits={splits} kind={kind}")
    t_out, t_kept = _decode_run(geo, P, steps, splits, kind=kind, finish=1)
    l_out, l_kept = _decode_run(geo, P, steps, splits, kind=kind, finish=2)
    assert t_kept == l_kept
    for i, (x, y) in enumerate(zip(t_out, l_out)):
        assert np.array_equal(x, y), f"step {i}: the two finishes differ"
    s = Stream(geo, P + steps, 7, kind)
    orc = make_oracle(geo)
    orc.prefill(s.k[:, :P], s.v[:, :P], s.scores[:, :P])
    for n in range(P, P + steps):
        ref = orc.decode(s.q[n], s.k[:, n], s.v[:, n], s.leaving(n), attend=(n == P + steps - 1))
    check_output(out_to_f64(torch.from_numpy(t_out[-1]).view(torch.bfloat16))[0], ref, "last step")
    for g in range(geo.n_kv_heads):
        assert t_kept[g] == orc.kept(g), g


def test_state_machine_errors_and_reset():
    geo = Geo(4, 1, 64, 2, 10, 4)
    cache = make_cache(geo, max_positions=40)
    s = Stream(geo, 60, 3)
    k, v, sc = to_dev_bf16(s.k[:, :30]), to_dev_bf16(s.v[:, :30]), to_dev_f32(s.scores[:, :30])
    cache.prefill_compact(0, 0, k, v, sc)
    with pytest.raises(abi.KVpopError) as e:
        cache.prefill_compact(0, 0, k, v, sc)
    assert e.value.code == abi.KVPOP_ESTATE
    out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    for n in range(30, 40):                      # positions up to max_positions - 1
        cache.decode_step(0, to_dev_bf16(s.q[n][None]), to_dev_bf16(s.k[:, n][None]),
                          to_dev_bf16(s.v[:, n][None]), to_dev_f32(s.leaving(n)[None]), out)
    with pytest.raises(abi.KVpopError) as e:     # position 40 is past the limit
        n = 40
        cache.decode_step(0, to_dev_bf16(s.q[n][None]), to_dev_bf16(s.k[:, n][None]),
                          to_dev_bf16(s.v[:, n][None]), to_dev_f32(s.leaving(n)[None]), out)
    assert e.value.code == abi.KVPOP_ESTATE
    assert cache.state(0, 0).n == 39
    with pytest.raises(ValueError):
        cache.decode_step(0, to_dev_bf16(s.q[0]), to_dev_bf16(s.k[:, 0][None]),
                          to_dev_bf16(s.v[:, 0][None]), to_dev_f32(s.leaving(0)[None]), out)
    # reset, then the same prompt again gives the oracle's kept set
    cache.reset(0, 0)
    assert cache.state(0, 0).n == -1
    cache.prefill_compact(0, 0, k, v, sc)
    orc = make_oracle(geo)
    orc.prefill(s.k[:, :30], s.v[:, :30], s.scores[:, :30])
    _cmp_kept(cache.state(0, 0), orc, "after reset + prefill")
    # empty prompt is a no-op
    cache.reset(0, 0)
    cache.prefill_compact(0, 0, to_dev_bf16(s.k[:, :0]), to_dev_bf16(s.v[:, :0]),
                          to_dev_f32(s.scores[:, :0]))
    assert cache.state(0, 0).n == -1
    cache.close()


def test_reset_is_applied_by_the_next_reader():
    """A reset enqueues nothing: the next decode (or state read) of the layer
    initialises the sequence's control blocks, a non-empty prefill overwrites
    them.  Sequence 1 of a batch of 3 is reset mid-stream and restarts from an
    empty prompt while sequences 0 and 2 carry on; then sequence 2 is reset and
    refilled by a prefill."""
    geo = Geo(8, 2, 64, 2, 12, 6)
    B, P, T1, T2 = 3, 40, 25, 30
    cache = make_cache(geo, batch=B)
    streams = [Stream(geo, P + T1 + T2 + P, 40 + b) for b in range(B)]
    orcs = [make_oracle(geo) for _ in range(B)]
    for b in range(B):
        s = streams[b]
        cache.prefill_compact(0, b, to_dev_bf16(s.k[:, :P]), to_dev_bf16(s.v[:, :P]),
                              to_dev_f32(s.scores[:, :P]))
        orcs[b].prefill(s.k[:, :P], s.v[:, :P], s.scores[:, :P])
    pos = [P] * B  # next position of each sequence
    out = torch.empty((B, geo.n_q_heads, geo.head_dim), dtype=torch.bfloat16, device="cuda")

    def step(last):
        q = np.stack([streams[b].q[pos[b]] for b in range(B)])
        kn = np.stack([streams[b].k[:, pos[b]] for b in range(B)])
        vn = np.stack([streams[b].v[:, pos[b]] for b in range(B)])
        sl = np.stack([streams[b].leaving(pos[b]) for b in range(B)])
        cache.decode_step(0, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), to_dev_f32(sl), out)
        got = out_to_f64(out)
        for b in range(B):
            s = streams[b]
            ref = orcs[b].decode(s.q[pos[b]], s.k[:, pos[b]], s.v[:, pos[b]], s.leaving(pos[b]),
                                 attend=last)
            if last:
                check_output(got[b], ref, f"seq {b} position {pos[b]}")
            pos[b] += 1

    for i in range(T1):
        step(i == T1 - 1)
    cache.reset(0, 1)
    orcs[1] = make_oracle(geo)
    pos[1] = 0
    for i in range(T2):
        step(i == T2 - 1)
    for b in range(B):
        _cmp_kept(cache.state(0, b), orcs[b], f"seq {b} after the reset of seq 1")
    # reset + non-empty prefill: the prefill writes the blocks itself
    cache.reset(0, 2)
    s = streams[2]
    cache.prefill_compact(0, 2, to_dev_bf16(s.k[:, :P]), to_dev_bf16(s.v[:, :P]),
                          to_dev_f32(s.scores[:, :P]))
    orcs[2] = make_oracle(geo)
    orcs[2].prefill(s.k[:, :P], s.v[:, :P], s.scores[:, :P])
    pos[2] = P
    step(True)
    for b in range(B):
        _cmp_kept(cache.state(0, b), orcs[b], f"seq {b} after the refill of seq 2")
    # reset + empty prompt, then the state: empty
    cache.reset(0, 0)
    cache.prefill_compact(0, 0, to_dev_bf16(s.k[:, :0]), to_dev_bf16(s.v[:, :0]),
                          to_dev_f32(s.scores[:, :0]))
    st = cache.state(0, 0)
    assert st.n == -1 and all(int(c) == 0 for c in st.counts)
    cache.close()


def test_nan_score_sets_flag():
    geo = Geo(4, 1, 64, 2, 10, 4)
    cache = make_cache(geo)
    s = Stream(geo, 40, 5)
    sc = s.scores[:, :30].copy()
    sc[0, 7] = np.nan
    cache.prefill_compact(0, 0, to_dev_bf16(s.k[:, :30]), to_dev_bf16(s.v[:, :30]), to_dev_f32(sc))
    st = cache.state(0, 0)
    assert st.flags & abi.KVPOP_FLAG_NAN_SCORE
    cache.close()
    cache = make_cache(geo)
    out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    for n in range(12):
        sl = s.leaving(n)
        if n == 9:
            sl[:] = np.nan
        cache.decode_step(0, to_dev_bf16(s.q[n][None]), to_dev_bf16(s.k[:, n][None]),
                          to_dev_bf16(s.v[:, n][None]), to_dev_f32(sl[None]), out)
    assert cache.state(0, 0).flags & abi.KVPOP_FLAG_NAN_SCORE
    cache.close()
