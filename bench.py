"""Benchmark of the fixed-budget KV cache hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch of the
one-layer Qwen3-8B workload at 4x (32 query heads, 8 KV heads, head_dim 128,
budget 4,032 = 4 sink + 3,772 scored + 256 recent): reset, prefill
compaction of a 16,384-token prompt, then 1,024 decode steps (delayed
eviction + GQA decode attention).  Inputs are resident in HBM before timing.
A whole pass is captured once in a HIP graph and replayed; the decode and
prefill phases are also timed on their own (decode replayed from its own
graph, the two prefill launches direct), back to back.

Prints ONE JSON line.  value = decode steps per second of whole-pass time
(prefill included).  The roofline object covers the decode step (at batch 1
the attention kernel over 32 splits per KV head and the kernel that merges
the splits and updates the cache): algorithmic bytes per step / average
decode step time (HIP events on the replay stream).  cpu_baseline times the
CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode graph|eager]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/sec + achieved HBM GB/s, 4032-entry/head cache, Qwen3-8B layer shapes"
HBM_PEAK_GBPS = 8000.0
# one 32-bit VALU operation per lane per clock: 157.3 TFLOP/s of packed fp32
# FMA is 4 flops per lane-clock, so 39.3 T lane-operations per second
ALU_PEAK_GOPS = 157.3e3 / 4
PROFILE_PMC = os.path.join(ROOT, "profiles", "decode_kernel_qwen3_8b_layer_4x_traffic.json")
PROFILE_PMC_B64 = os.path.join(ROOT, "profiles", "decode_kernel_batched_serving_b64_traffic.json")


def decode_bytes_per_step(w, n_kept: int) -> int:
    """Algorithmic bytes of one decode step (one layer) at batch w.batch.

    Read K and V of every kept row, read q, write out, append the new K/V row.
    """
    D, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    per_seq = Hkv * n_kept * D * 2 * 2 + Hq * D * 2 + Hq * D * 2 + Hkv * D * 2 * 2
    return per_seq * w.batch


def prefill_bytes(w, P: int) -> int:
    """Algorithmic bytes of one prefill compaction: candidate scores read once,
    kept rows read and written, slot metadata (position 4 B, key 8 B) written."""
    s, k, W, D, Hkv = w.n_sink, w.n_scored, w.n_recent, w.head_dim, w.n_kv_heads
    C = max(0, P - W - s)
    kept = min(s, P) + min(k, C) + (P - max(min(P, max(s, P - W)), 0))
    return Hkv * (C * 4 + 2 * kept * D * 2 * 2 + kept * 12)


def _load_traffic(kernel_hash: str, path: str = PROFILE_PMC):
    """HBM traffic per decode step from the committed counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha1") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_step")


def _hold_gpu(ms: float):
    """Keep the current stream busy for about `ms` milliseconds (a spinning
    kernel), so that the host has queued what follows before the GPU gets
    there: the timed region then holds no host launch latency."""
    import torch
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 2.4e6))  # cycles at 2.4 GHz


def _strip_comments(src: str) -> str:
    """C++ source without comments and blank lines: what the compiler sees
    of it, so that an edited comment does not count as a changed kernel."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())


def _kernel_hash() -> str:
    import hashlib
    h = hashlib.sha1()
    for name in ("kvpop_decode.hip", "kvpop_device.h", "kvpop_internal.h"):
        with open(os.path.join(ROOT, "fixed_budget_learned_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()


def cpu_baseline(w, sample_steps: int):
    """Time the CPU oracle (as it stands) on the first ``sample_steps`` decode
    steps after a full prefill of the same workload."""
    import numpy as np
    from fixed_budget_learned_amd.inputs import TokenStream
    from oracle import KVpopOracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    P = w.prompt_len
    ts = TokenStream(w, 0, 0, P, sample_steps)
    kk, vv = ts.step_kv()
    sl = ts.step_leaving_scores()
    orc = KVpopOracle(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_scored, w.n_recent)
    t0 = time.perf_counter()
    orc.prefill(ts.prompt_k(), ts.prompt_v(), ts.prompt_scores())
    t1 = time.perf_counter()
    for i in range(sample_steps):
        orc.decode(ts.q[i], kk[i], vv[i], sl[i])
    t2 = time.perf_counter()
    return {
        "value": sample_steps / (t2 - t1),
        "unit": "decode steps/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{w.name}: prefill {P} tokens then the first {sample_steps} of "
                  f"{w.decode_steps} decode steps (all 8 KV heads, 32 query heads), fp64",
        "prefill_tokens_per_s": P / (t1 - t0),
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "host_cpu": _cpu_model(),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dense_vs_kvpop(contexts, steps: int, reps: int):
    """Decode time per step of the fixed-budget cache against a cache that
    never evicts (dense attention over all n tokens), at growing context.

    Both use the Qwen3-8B layer shape at batch 1 and the same kernels; the
    dense cache is the special case whose scored region holds every token.
    Inputs: seeded device-side N(0,1) K/V/q and scores.
    """
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.configs import QWEN3_8B_LAYER_4X as w
    D, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260706)
    rows = []
    for P in contexts:
        T = P + steps
        k = torch.randn((Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn((Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
        sc = torch.randn((Hkv, T), generator=gen, device="cuda")
        q = torch.randn((steps, 1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
        kn = k[:, P:].transpose(0, 1).contiguous().view(steps, 1, Hkv, D)
        vn = v[:, P:].transpose(0, 1).contiguous().view(steps, 1, Hkv, D)
        sl = sc[:, P - w.n_recent:T - w.n_recent].transpose(0, 1).contiguous().view(steps, 1, Hkv)
        pk, pv, ps = k[:, :P].contiguous(), v[:, :P].contiguous(), sc[:, :P].contiguous()
        out = torch.empty((steps, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
        res = {"context": P}
        for mode in ("kvpop", "dense"):
            n_scored = w.n_scored if mode == "kvpop" else T
            cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, n_scored, w.n_recent,
                                                   max_positions=T))
            budget = w.n_sink + n_scored + w.n_recent

            def pre():
                cache.reset(0, 0)
                cache.prefill_compact(0, 0, pk, pv, ps)

            def dec():
                for i in range(steps):
                    cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out[i])

            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                pre()
                dec()
            torch.cuda.synchronize()
            gp, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gp, stream=stream):
                pre()
            with torch.cuda.graph(gd, stream=stream):
                dec()
            ms = 0.0
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    gp.replay()
                    e0.record(stream)
                    gd.replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                if r > 0:
                    ms += e0.elapsed_time(e1)
            us = ms * 1e3 / (reps * steps)
            kept = min(budget, P + steps // 2)
            nbytes = Hkv * kept * D * 4 + Hq * D * 4 + Hkv * D * 4
            res[f"{mode}_us_per_step"] = us
            res[f"{mode}_GBps"] = nbytes / (us * 1e-6) / 1e9
            cache.close()
            del gp, gd
        res["dense_over_kvpop"] = res["dense_us_per_step"] / res["kvpop_us_per_step"]
        rows.append(res)
        del k, v, sc, q, kn, vn, sl, pk, pv, ps, out
        torch.cuda.empty_cache()
    return rows


def dynamic_backend(steps: int, reps: int, every: int = 256):
    """The Dynamic backend (grow into `every` rows of slack, prune after
    every `every`-th step) against the Static one on the one-layer Qwen3-8B
    4x workload: prefill 16,384, then `steps` decode steps, both captured in
    graphs; plus the prune kernel alone after `every` steps of growth.
    Inputs: seeded device-side N(0,1) K/V/q and scores."""
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.configs import QWEN3_8B_LAYER_4X as w
    D, Hq, Hkv, W, P = w.head_dim, w.n_q_heads, w.n_kv_heads, w.n_recent, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5000)
    T = P + steps
    k = torch.randn((Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    sc = torch.randn((Hkv, T), generator=gen, device="cuda")
    q = torch.randn((steps, 1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    kn = k[:, P:].transpose(0, 1).contiguous().view(steps, 1, Hkv, D)
    vn = v[:, P:].transpose(0, 1).contiguous().view(steps, 1, Hkv, D)
    sl = sc[:, P - W:T - W].transpose(0, 1).contiguous().view(steps, 1, Hkv)
    pk, pv, ps = k[:, :P].contiguous(), v[:, :P].contiguous(), sc[:, :P].contiguous()
    out = torch.empty((1, Hq, D), dtype=torch.bfloat16, device="cuda")
    res = {"workload": w.name, "prune_interval": every, "decode_steps": steps}
    stream = torch.cuda.Stream()
    for mode, interval in (("static", 0), ("dynamic", every)):
        cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, w.n_scored, W,
                                               max_positions=T, prune_interval=interval))

        def pre():
            cache.reset(0, 0)
            cache.prefill_compact(0, 0, pk, pv, ps)

        def dec():
            for i in range(steps):
                cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out)

        with torch.cuda.stream(stream):
            pre()
            dec()
        torch.cuda.synchronize()
        gp, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp, stream=stream):
            pre()
        with torch.cuda.graph(gd, stream=stream):
            dec()
        ms = 0.0
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                gp.replay()
                e0.record(stream)
                gd.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            if r > 0:
                ms += e0.elapsed_time(e1)
        res[f"{mode}_us_per_step"] = ms * 1e3 / (reps * steps)
        res[f"{mode}_steps_per_s"] = reps * steps / (ms / 1e3)
        st = cache.state(0, 0)
        res[f"{mode}_rows_after"] = int(max(st.counts))
        cache.close()
        del gp, gd
    res["dynamic_over_static"] = res["dynamic_us_per_step"] / res["static_us_per_step"]
    # the prune alone: grow `every` steps with no scheduled prune, then prune
    cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, w.n_scored, W,
                                           max_positions=T, prune_interval=4096))
    us = []
    for r in range(reps + 1):
        with torch.cuda.stream(stream):
            cache.reset(0, 0)
            cache.prefill_compact(0, 0, pk, pv, ps)
            for i in range(every):
                cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            cache.prune(0)
            e1.record(stream)
        torch.cuda.synchronize()
        if r > 0:
            us.append(e0.elapsed_time(e1) * 1e3)
    st = cache.state(0, 0)
    assert all(int(c) == w.budget for c in st.counts), "prune left more than the budget"
    cache.close()
    res["prune_us"] = sum(us) / len(us)
    res["prune_us_per_step_amortised"] = res["prune_us"] / every
    del k, v, sc, q, kn, vn, sl, pk, pv, ps
    torch.cuda.empty_cache()
    return res


def layered_config(w, steps: int, reps: int):
    """Decode steps/s and prefill tokens/s of a batch-1 workload over all its
    layers (each step and each prefill runs once per layer), with the
    fraction of the HBM roofline.  Seeded device-side N(0,1) K/V/q; scores
    drawn as the workload states.  Prefill inputs are generated one layer at
    a time (the 131k workload needs 19 GB of them in all).
    """
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.inputs import T_SCORES, draw_scores, rng_for
    L, Hq, Hkv, D = w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim
    P = w.prompt_len or 0
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2000 + w.wid)
    # the decode graph below is replayed reps times after one eager pass and
    # the cache keeps advancing on the device: P + steps * (reps + 1) positions
    cache = abi.KVpopCache(abi.make_config(L, 1, Hq, Hkv, D, w.n_sink, w.n_scored, w.n_recent,
                                           max_positions=P + steps * (reps + 2) + 1))
    stream = torch.cuda.Stream()
    pre_ms = pre_batch_ms = 0.0
    if P > 0:
        # every layer's prompt (19 GB for the 131k workload) resident at once
        ks, vs, scs = [], [], []
        for layer in range(L):
            ks.append(torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16))
            vs.append(torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16))
            scs.append(torch.from_numpy(draw_scores(rng_for(w.wid, layer, 0, T_SCORES),
                                                    w.score_dist, (Hkv, P))).to("cuda"))
        torch.cuda.synchronize()
        # one call per layer ...
        for layer in range(L):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                _hold_gpu(0.2)
                e0.record(stream)
                cache.prefill_compact(layer, 0, ks[layer], vs[layer], scs[layer])
                e1.record(stream)
            torch.cuda.synchronize()
            pre_ms += e0.elapsed_time(e1)
        # ... and every layer in one batched call, into a second cache
        cb = abi.KVpopCache(abi.make_config(L, 1, Hq, Hkv, D, w.n_sink, w.n_scored, w.n_recent,
                                            max_positions=P + 1))
        items = [(layer, 0, ks[layer], vs[layer], scs[layer]) for layer in range(L)]

        def reset_all():
            for layer in range(L):
                cb.reset(layer, 0)

        with torch.cuda.stream(stream):
            cb.prefill_compact_batch(items)  # warm-up
        torch.cuda.synchronize()
        # launched directly behind a spinning kernel: the host marshals the
        # items and enqueues the launches while the GPU spins, so neither the
        # marshalling nor a graph replay's own overhead (~11 us) is timed
        for r in range(reps + 1):
            reset_all()  # host state only: the sequences are empty again
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                _hold_gpu(1.0)
                e0.record(stream)
                cb.prefill_compact_batch(items)
                e1.record(stream)
            torch.cuda.synchronize()
            if r > 0:
                pre_batch_ms += e0.elapsed_time(e1) / reps
        st_a, st_b = cache.state(L - 1, 0), cb.state(L - 1, 0)
        assert all(a.tolist() == b.tolist() for a, b in zip(st_a.kept, st_b.kept)), \
            "batched prefill differs"
        cb.close()
        del ks, vs, scs, items
        torch.cuda.empty_cache()
    q = torch.randn((steps, L, 1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    kn = torch.randn((steps, L, 1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((steps, L, 1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    sl = torch.from_numpy(draw_scores(rng_for(w.wid, 0, 1, T_SCORES), w.score_dist,
                                      (steps, L, 1, Hkv))).to("cuda")
    out = torch.empty((L, 1, Hq, D), dtype=torch.bfloat16, device="cuda")

    def dec():
        for i in range(steps):
            for layer in range(L):
                cache.decode_step(layer, q[i, layer], kn[i, layer], vn[i, layer], sl[i, layer],
                                  out[layer])

    def dec_one_launch():
        for i in range(steps):
            cache.decode_step_layers(0, q[i], kn[i], vn[i], sl[i], out)

    def timed(fn):
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (reps * steps)

    us = timed(dec)
    us1 = timed(dec_one_launch) if L > 1 else None
    cache.close()
    # decode bytes per step: every layer reads its kept rows; a cache started
    # empty holds at least P + steps rows during the timed replays
    kept = min(w.budget, P + steps + 1)
    dbytes = L * decode_bytes_per_step(w, kept)
    res = {"workload": w.name, "layers": L, "batch": 1, "budget": w.budget, "prompt_len": P,
           "decode_us_per_step": us, "decode_steps_per_s": 1e6 / us,
           "decode_GBps": dbytes / (us * 1e-6) / 1e9,
           "decode_frac": dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
           "decode_launch": "one kvpop_decode_step launch per layer-step",
           "decode_bytes_per_step": dbytes, "decode_steps_timed": reps * steps}
    if us1 is not None:
        res["decode_one_launch"] = {
            "us_per_step": us1, "steps_per_s": 1e6 / us1,
            "GBps": dbytes / (us1 * 1e-6) / 1e9,
            "frac": dbytes / (us1 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "launch": "kvpop_decode_step_layers: every layer in one launch",
            "valid_for": "independent per-layer inputs only (these synthetic layers); a model "
                         "decodes layer by layer, since layer l+1's query depends on layer l's "
                         "output"}
    if P > 0:
        pbytes = L * prefill_bytes(w, P)
        res.update({"prefill_us_all_layers": pre_batch_ms * 1e3,
                    "prefill_tokens_per_s": P / (pre_batch_ms / 1e3),
                    "prefill_GBps": pbytes / (pre_batch_ms / 1e3) / 1e9,
                    "prefill_frac": pbytes / (pre_batch_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                    "prefill_bytes": pbytes,
                    "prefill_launch": "all layers in one kvpop_prefill_compact_batch call, launched "
                                      "directly behind a spinning kernel",
                    "prefill_us_one_call_per_layer": pre_ms * 1e3})
    return res


def memory_context():
    """Device bytes of the fixed-budget caches of the 36-layer workloads
    against a dense cache of the same model at 131,072 tokens, beside the
    pages' peak-VRAM figures (quoted as context, not as a target: they are
    whole-model measurements on unstated hardware)."""
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.configs import LONG_131K_8X, QWEN3_8B_36L_4X
    res = {}
    for w, positions in ((LONG_131K_8X, 131072 + 2048), (QWEN3_8B_36L_4X, 16384 + 4096)):
        cfg = abi.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink,
                              w.n_scored, w.n_recent, max_positions=positions)
        rows = w.n_layers * w.n_kv_heads * w.budget
        res[w.name] = {"budget_per_head": w.budget,
                       "kv_rows_bytes": rows * w.head_dim * 2 * 2,
                       "arena_bytes": abi.required_bytes(cfg),
                       "arena_note": "kvpop_cache_required_bytes: K/V rows, slot metadata and the "
                                     "prefill/decode workspaces, allocated once at creation"}
    w = LONG_131K_8X
    res["dense_cache_131k_bytes"] = w.n_layers * w.n_kv_heads * 131072 * w.head_dim * 2 * 2
    res["pages_context"] = {
        "dense_peak_vram_GB": 36, "kvpop_peak_vram_GB": 19,
        "what": "whole-model peak VRAM, Qwen3-8B at batch 1 decoding to 131k tokens; hardware "
                "not stated",
        "source": "English aiweekly article, third paragraph (also the French article, first and "
                  "third paragraphs)"}
    return res


def decode_cold(w, steps: int):
    """Decode step time of the one-layer workload when its cache is not
    resident in any cache level: a 1 GiB buffer is written between steps
    (more than the 256 MB last-level cache), then one decode step is timed
    alone with events around it."""
    import torch
    from fixed_budget_learned_amd import abi
    Hq, Hkv, D, P = w.n_q_heads, w.n_kv_heads, w.head_dim, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3000 + w.wid)
    cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, w.n_scored, w.n_recent,
                                           max_positions=P + steps + 1))
    k = torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16)
    sc = torch.randn((Hkv, P), generator=gen, device="cuda")
    cache.prefill_compact(0, 0, k, v, sc)
    q = torch.randn((steps, 1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    kn = torch.randn((steps, 1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((steps, 1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    sl = torch.randn((steps, 1, Hkv), generator=gen, device="cuda")
    out = torch.empty((1, Hq, D), dtype=torch.bfloat16, device="cuda")
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(steps):
        scratch.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    cache.close()
    ms.sort()
    us = ms[len(ms) // 2] * 1e3
    bpl = decode_bytes_per_step(w, w.budget)
    return {"decode_us_per_step_median": us, "GBps": bpl / (us * 1e-6) / 1e9,
            "frac": bpl / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "steps": steps,
            "note": "1 GiB written between steps; events around each single step "
                    "(includes its launch latency)"}


def prefix_thresholds_rate(w, reps: int):
    """Time kvpop_prefix_thresholds on one prompt of the workload (all KV
    heads): positions per second, and the bytes it must move (scores in,
    8-byte thresholds out) against the HBM roofline."""
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.inputs import T_SCORES, draw_scores, rng_for
    Hkv, P = w.n_kv_heads, w.prompt_len
    sc = torch.from_numpy(draw_scores(rng_for(w.wid, 0, 0, T_SCORES), w.score_dist,
                                      (Hkv, P))).to("cuda")
    thr = torch.empty((Hkv, P), dtype=torch.int64, device="cuda")
    cache = abi.KVpopCache(abi.make_config(1, 1, w.n_q_heads, Hkv, w.head_dim, w.n_sink,
                                           w.n_scored, w.n_recent, max_positions=P))
    cache.prefix_thresholds(sc, thr)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        cache.prefix_thresholds(sc, thr)
    e1.record()
    torch.cuda.synchronize()
    cache.close()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = Hkv * (P - w.n_sink - w.n_recent) * 4 + Hkv * P * 8
    # Compute side: a streaming top-k compares every candidate with the
    # current threshold and inserts each entrant into the sorted k kept keys
    # (ceil(log2 k) compares).  Entrants: k * (1 + ln(C / k)) for candidates
    # in random order (the expected number of prefix top-k changes).
    import math
    C, k = P - w.n_sink - w.n_recent, w.n_scored
    entrants = k * (1 + math.log(C / k)) if C > k else C
    compares = Hkv * (C + entrants * math.ceil(math.log2(max(k, 2))))
    gops = compares / (us * 1e-6) / 1e9
    return {"workload": w.name, "prompt_len": P, "us_per_call": us,
            "positions_per_s": P / (us * 1e-6),
            "roofline": {"bound": "alu", "achieved": gops, "peak": ALU_PEAK_GOPS,
                         "unit": "G compares/s", "frac": gops / ALU_PEAK_GOPS,
                         "work_per_call": compares,
                         "note": "latency-bound: per (segment, KV head) one workgroup sweeps "
                                 "its candidates in dependent chunks; neither compares, LDS nor "
                                 "HBM bytes bind it"},
            "hbm": {"GBps": nbytes / (us * 1e-6) / 1e9,
                    "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "bytes": nbytes}}


def future_target_rate(w, reps: int):
    """Time kvpop_future_attention_target over one prompt of the workload
    (both passes): the algorithmic flops are the two causal products
    (2 * D per (query, key) pair: every causal pair in the log-sum-exp pass,
    the pairs with query >= key + W in the column pass) per query head."""
    import torch
    from fixed_budget_learned_amd import abi
    Hq, Hkv, D, W, T = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_recent, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4000 + w.wid)
    q = torch.randn((Hq, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    work = torch.empty((2, Hq, T), dtype=torch.float32, device="cuda")
    y = torch.empty((Hkv, T), dtype=torch.float32, device="cuda")
    cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, w.n_scored, W,
                                           max_positions=T))
    # untimed warm-up, about 50 ms of calls: the first ~35 ms run up to 10 %
    # slower while the shader clock rises from idle
    for _ in range(20):
        cache.future_attention_target(q, k, work, y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        cache.future_attention_target(q, k, work, y)
    e1.record()
    torch.cuda.synchronize()
    cache.close()
    us = e0.elapsed_time(e1) * 1e3 / reps
    pairs = T * (T + 1) / 2 + max(0, T - W) * (T - W + 1) / 2
    flops = Hq * pairs * 2 * D
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": w.name, "tokens": T, "us_per_call": us, "TFLOPs": tf,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": tf / 2500.0, "flops_per_call": flops}}


def batched_serving(steps: int, reps: int, mode: str = "graph"):
    """Batched serving: 64 sequences of the Qwen3-8B layer shape with 4,032
    slots per KV head, prompts uniform in [4096, 32768] (seeded), scores
    lognormal quantised to 256 levels.  One decode launch serves all 64
    sequences.  The one-call-per-prompt prefill and the decode steps are
    captured as HIP graphs and replayed, the batched prefill call is launched
    directly (mode "eager": plain launches throughout); K/V/q are seeded
    device-side N(0,1).
    """
    import numpy as np
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.configs import BATCH64_SERVING as w
    from fixed_budget_learned_amd.inputs import T_SCORES, draw_scores, prompt_lengths, rng_for
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    lens = [int(x) for x in prompt_lengths(w)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + w.wid)
    pk, pv, ps = [], [], []
    for b, P in enumerate(lens):
        pk.append(torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16))
        pv.append(torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16))
        ps.append(torch.from_numpy(draw_scores(rng_for(w.wid, 0, b, T_SCORES), w.score_dist,
                                               (Hkv, P))).to("cuda"))
    q = torch.randn((steps, B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    kn = torch.randn((steps, B, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((steps, B, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    # leaving-token scores of the decode steps: a stream of its own (seq index B)
    sl = torch.from_numpy(draw_scores(rng_for(w.wid, 0, B, T_SCORES), w.score_dist,
                                      (steps, B, Hkv))).to("cuda")
    out = torch.empty((steps, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    cache = abi.KVpopCache(abi.make_config(1, B, Hq, Hkv, D, w.n_sink, w.n_scored, w.n_recent,
                                           max_positions=max(lens) + steps + 1))

    items = [(0, b, pk[b], pv[b], ps[b]) for b in range(B)]

    def reset():
        for b in range(B):
            cache.reset(0, b)

    def pre():  # every prompt of the batch in one call
        cache.prefill_compact_batch(items)

    def pre_each():  # one call per prompt, for comparison
        for b in range(B):
            cache.prefill_compact(0, b, pk[b], pv[b], ps[b])

    def dec():
        for i in range(steps):
            cache.decode_step(0, q[i], kn[i], vn[i], sl[i], out[i])

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        reset()
        pre()
        dec()
    torch.cuda.synchronize()
    if mode == "graph":
        # A reset only marks the sequences empty in the host state (it
        # launches nothing), which the prefill calls check when they are
        # captured; a replayed prefill rewrites every sequence's state, so
        # the replays need no reset between them.  The batched call is
        # launched directly behind a spinning kernel (the host marshals the
        # prompt list meanwhile), like the one-prompt prefill of the main line.
        ge, gd = (torch.cuda.CUDAGraph() for _ in range(2))
        reset()
        with torch.cuda.graph(ge, stream=stream):
            pre_each()
        reset()
        with torch.cuda.stream(stream):
            pre()
        with torch.cuda.graph(gd, stream=stream):
            dec()
        run_each, run_dec = ge.replay, gd.replay
    else:
        run_each, run_dec = pre_each, dec
    pre_ms = each_ms = dec_ms = 0.0
    for r in range(reps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        if mode != "graph":
            reset()
        with torch.cuda.stream(stream):
            _hold_gpu(1.0)
            e[0].record(stream)
            run_each()
            e[1].record(stream)
        reset()  # the batched call needs empty sequences
        with torch.cuda.stream(stream):
            _hold_gpu(1.0)
            e[2].record(stream)
            pre()
            e[3].record(stream)
            run_dec()
            e[4].record(stream)
        torch.cuda.synchronize()
        if r > 0:
            each_ms += e[0].elapsed_time(e[1])
            pre_ms += e[2].elapsed_time(e[3])
            dec_ms += e[3].elapsed_time(e[4])
    counts = cache.state(0, B - 1).counts
    assert all(int(c) == w.budget for c in counts), "batched caches not full"
    cache.close()
    us = dec_ms * 1e3 / (reps * steps)
    bpl = decode_bytes_per_step(w, w.budget)
    gbps = bpl / (us * 1e-6) / 1e9
    ptok = sum(lens)
    pbytes = sum(prefill_bytes(w, P) for P in lens)
    pre_s = pre_ms / 1e3 / reps
    return {
        "workload": w.name, "batch": B, "budget": w.budget,
        "prompt_tokens": ptok, "decode_steps_timed": steps * reps,
        "decode_us_per_step": us, "decode_steps_per_s": 1e6 / us,
        "decode_tokens_per_s": B * 1e6 / us,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "bytes_per_step": bpl,
                     "traffic": _load_traffic(_kernel_hash(), PROFILE_PMC_B64),
                     "kernel": "decode_kernel, one workgroup per KV head (head_dim 128, "
                               "4 query heads per KV head)"},
        "prefill_tokens_per_s": ptok / pre_s,
        "prefill_GBps": pbytes / pre_s / 1e9,
        "prefill_frac": pbytes / pre_s / 1e9 / HBM_PEAK_GBPS,
        "prefill_us": pre_s * 1e6,
        "prefill_launch": "all 64 prompts in one kvpop_prefill_compact_batch call, launched "
                          "directly behind a spinning kernel",
        "prefill_us_one_call_per_prompt": each_ms * 1e3 / reps,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--workload", default="qwen3_8b_layer_4x")
    ap.add_argument("--cpu-sample-steps", type=int, default=384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="decode steps per pass (default: the workload's); for short profiles")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batch-64 serving measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, 36-layer and 131k-token workloads and the cold-cache line")
    ap.add_argument("--batched-only", action="store_true",
                    help="run only the batch-64 serving measurement (for profiles)")
    ap.add_argument("--only", choices=("future", "thresholds", "dynamic", "long_context",
                                       "stack_16k", "cold"),
                    default=None,
                    help="run only this section (for profiles): future, thresholds, dynamic and "
                         "cold (decode with the cache evicted from every cache level between "
                         "steps) on the one-layer workload, long_context the 36-layer "
                         "131k-token one, stack_16k the 36-layer 16k-token one")
    ap.add_argument("--no-dense-sweep", action="store_true",
                    help="skip the fixed-budget vs dense decode comparison at 16k-131k context")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device-to-device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the cache path shards by sequence and KV head with no "
              "exchange, so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from fixed_budget_learned_amd import abi
    from fixed_budget_learned_amd.configs import BY_NAME
    from fixed_budget_learned_amd.inputs import TokenStream

    if args.copy_bytes:
        x = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda").uniform_()
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": x.numel() * 4, "copies": max(1, args.steps)}), flush=True)
        return

    if args.only:
        abi.load()
        from fixed_budget_learned_amd.configs import LONG_131K_8X, QWEN3_8B_36L_4X, QWEN3_8B_LAYER_4X
        if args.only == "future":
            r = future_target_rate(QWEN3_8B_LAYER_4X, max(1, args.steps))
        elif args.only == "thresholds":
            r = [prefix_thresholds_rate(QWEN3_8B_LAYER_4X, max(1, args.steps)),
                 prefix_thresholds_rate(LONG_131K_8X, max(1, args.steps))]
        elif args.only == "long_context":
            r = layered_config(LONG_131K_8X, args.decode_steps or 32, max(1, args.steps))
        elif args.only == "stack_16k":
            r = layered_config(QWEN3_8B_36L_4X, args.decode_steps or 32, max(1, args.steps))
        elif args.only == "cold":
            r = decode_cold(QWEN3_8B_LAYER_4X, args.decode_steps or 32)
        else:
            r = dynamic_backend(args.decode_steps or 1024, max(1, args.steps))
        print(json.dumps({args.only: r}), flush=True)
        return
    if args.batched_only:
        abi.load()
        print(json.dumps({"batched_serving": batched_serving(args.decode_steps or 64, args.steps,
                                                             args.mode)}), flush=True)
        return

    w = BY_NAME[args.workload]
    if w.batch != 1 or w.n_layers != 1 or w.prompt_len is None:
        print("bench.py drives one-layer, batch-1 workloads", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    abi.load()
    dev = torch.device("cuda:0")
    P, S = w.prompt_len, (args.decode_steps or w.decode_steps)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    ts = TokenStream(w, 0, 0, P, S)
    kk, vv = ts.step_kv()
    pk, pv = bf(ts.prompt_k()), bf(ts.prompt_v())
    ps = torch.from_numpy(ts.prompt_scores()).to(dev)
    qd, kd, vd = bf(ts.q), bf(kk), bf(vv)
    sd = torch.from_numpy(ts.step_leaving_scores()).to(dev)
    out = torch.empty((S, 1, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    cfg = abi.make_config(1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_scored,
                          w.n_recent)
    cache = abi.KVpopCache(cfg)
    qs = [qd[i:i + 1] for i in range(S)]
    ks = [kd[i:i + 1] for i in range(S)]
    vs = [vd[i:i + 1] for i in range(S)]
    ss = [sd[i:i + 1] for i in range(S)]
    os_ = [out[i] for i in range(S)]

    def prefill_phase():
        cache.reset(0, 0)
        cache.prefill_compact(0, 0, pk, pv, ps)

    def decode_phase():
        for i in range(S):
            cache.decode_step(0, qs[i], ks[i], vs[i], ss[i], os_[i])

    def whole_pass():
        prefill_phase()
        decode_phase()

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.mode == "graph":
        # One eager pass first (also warms the library), then a whole pass
        # (reset, prefill, S decode steps) is captured in one HIP graph and
        # replayed once per timed step: back-to-back replays of one graph
        # carry no host launches, and a kernel that follows another graph's
        # replay on the stream can start up to ~25 us late.  The decode phase
        # alone is captured too, for the per-step figure.
        with torch.cuda.stream(stream):
            whole_pass()
        torch.cuda.synchronize()
        g_pass, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pass, stream=stream):
            whole_pass()
        with torch.cuda.graph(g_dec, stream=stream):
            decode_phase()
        torch.cuda.synchronize()
        run_pass, run_dec = g_pass.replay, g_dec.replay
    else:
        run_pass, run_dec = whole_pass, decode_phase

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_pass()
    torch.cuda.synchronize()

    # ---- the timed region: K whole passes ------------------------------------
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        _hold_gpu(1.0)  # outside the timed region: the host runs ahead from here
        ev[0].record(stream)
        for k in range(args.steps):
            run_pass()
        ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev[0].elapsed_time(ev[1])
    st = cache.state(0, 0)
    assert st.n == P + S - 1 and all(int(c) == w.budget for c in st.counts), "unexpected final state"

    # ---- the phases on their own, K times each, back to back ----------------
    # decode: the cache keeps advancing (full, budget rows per head)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(stream):
        _hold_gpu(1.0)
        e[0].record(stream)
        for k in range(args.steps):
            run_dec()
        e[1].record(stream)
    # prefill: reset + prefill of the same prompt, launched directly (two
    # launches; the reset enqueues nothing)
        _hold_gpu(1.0)
        e[2].record(stream)
        for k in range(args.steps):
            prefill_phase()
        e[3].record(stream)
    torch.cuda.synchronize()
    dec_ms = e[0].elapsed_time(e[1])
    pre_ms = e[2].elapsed_time(e[3])
    st = cache.state(0, 0)
    assert st.n == P - 1 and all(int(c) == w.budget for c in st.counts), "unexpected final state"
    cache.close()

    dsteps = args.steps * S
    dec_step_s = dec_ms / 1e3 / dsteps
    n_kept = w.budget
    bpl = decode_bytes_per_step(w, n_kept)
    achieved = bpl / dec_step_s / 1e9
    khash = _kernel_hash()
    traffic = _load_traffic(khash)
    pbytes = prefill_bytes(w, P)
    result = {
        "metric": METRIC,
        "value": dsteps / (total_ms / 1e3),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "budget": w.budget,
                   "n_sink": w.n_sink, "n_scored": w.n_scored, "n_recent": w.n_recent,
                   "prompt_len": P, "decode_steps_per_pass": S,
                   "launch": ("each pass replayed from one HIP graph" if args.mode == "graph"
                              else "every launch direct")},
        "decode_only_steps_per_s": dsteps / (dec_ms / 1e3),
        "decode_us_per_step": dec_step_s * 1e6,
        "prefill_us": pre_ms * 1e3 / args.steps,
        "phases_timed": "decode: K replays of the decode phase's graph back to back; prefill: K "
                        "reset + prefill calls launched directly, back to back; value and "
                        "ms_per_step: K whole-pass replays",
        "prefill_tokens_per_s": P * args.steps / (pre_ms / 1e3),
        "prefill_GBps": pbytes * args.steps / (pre_ms / 1e3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "traffic_unit": "bytes per step (FETCH_SIZE and WRITE_SIZE, copy-calibrated)",
            "kernel": "decode step: decode_kernel, 32 splits per KV head; the last split of each "
                      "head merges the partials and writes the cache update in the same launch; "
                      "head_dim 128, 4 query heads per KV head",
            "bytes_per_step": bpl,
            "note": "one layer's working set (16.5 MB) fits in the 256 MB last-level cache, so "
                    "back-to-back steps can be served partly from cache",
        },
        "wall_s_timed": wall,
    }
    if not args.no_batched:
        result["batched_serving"] = batched_serving(64, 3, args.mode)
    if not args.no_configs:
        from fixed_budget_learned_amd.configs import (LONG_131K_8X, QWEN3_8B_36L_4X, TINY,
                                                      TP8_SHARE_4X)
        result["decode_cold_cache"] = decode_cold(w, 32)
        result["future_attention_target"] = future_target_rate(w, 5)
        result["prefix_thresholds"] = [prefix_thresholds_rate(w, 5),
                                       prefix_thresholds_rate(LONG_131K_8X, 3)]
        result["configs"] = [layered_config(TINY, 512, 2),
                             layered_config(QWEN3_8B_36L_4X, 32, 2),
                             layered_config(LONG_131K_8X, 32, 2),
                             layered_config(TP8_SHARE_4X, 256, 2)]
    result["memory"] = memory_context()
    if not args.no_dense_sweep:
        result["dense_vs_kvpop"] = dense_vs_kvpop((16384, 32768, 65536, 131072), 64, 3)
        result["dynamic_backend"] = dynamic_backend(1024, 3)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_steps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
