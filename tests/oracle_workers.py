"""CPU-side oracle runs for the full-size GPU parity tests, in worker
processes (the streaming oracle is plain Python and one sequence of the
batch-64 workload takes seconds).  Imports NumPy, the input generators and
the oracle only: the workers never touch the GPU.

Every function returns plain lists and arrays so that results pickle back
to the test process, which compares them with what the GPU produced.
"""
from __future__ import annotations

import multiprocessing as mp
import os

from fixed_budget_learned_amd.configs import BY_NAME
from fixed_budget_learned_amd.inputs import TokenStream
from oracle import KVpopOracle, kept_by_definition


def stream_oracle(w_name: str, layer: int, seq: int, P: int, steps: int, check_steps, out_steps):
    """Follow one (layer, sequence) of a workload with the streaming oracle:
    kept sets after the prefill (key -1) and after every step in
    check_steps, outputs (float64 [Hq][D]) after every step in out_steps."""
    w = BY_NAME[w_name]
    ts = TokenStream(w, layer, seq, P, steps)
    orc = KVpopOracle(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.n_scored, w.n_recent)
    orc.prefill(ts.prompt_k(), ts.prompt_v(), ts.prompt_scores())
    kept = {-1: [orc.kept(g) for g in range(w.n_kv_heads)]}
    outs = {}
    kk, vv = ts.step_kv()
    sl = ts.step_leaving_scores()
    check_steps, out_steps = set(check_steps), set(out_steps)
    last = max(check_steps | out_steps, default=-1)
    for i in range(last + 1):
        ref = orc.decode(ts.q[i], kk[i], vv[i], sl[i], attend=(i in out_steps))
        if ref is not None:
            outs[i] = ref
        if i in check_steps:
            kept[i] = [orc.kept(g) for g in range(w.n_kv_heads)]
    return kept, outs


def kept_at(w_name: str, layer: int, seq: int, P: int, steps: int, positions):
    """Kept sets of every KV head of one (layer, sequence) after each position
    in `positions`, from the definition written out (sinks, window, top-k of
    the candidates by key)."""
    w = BY_NAME[w_name]
    ts = TokenStream(w, layer, seq, P, steps)
    return {n: [kept_by_definition(ts.scores[g], n, w.n_sink, w.n_scored, w.n_recent)
                for g in range(w.n_kv_heads)] for n in positions}


def pool(n: int | None = None):
    """Worker pool started with 'spawn', so that no worker inherits the test
    process's GPU context; at most 16 workers (the CPU share of one GPU)."""
    n = n or min(16, len(os.sched_getaffinity(0)))
    return mp.get_context("spawn").Pool(n)
