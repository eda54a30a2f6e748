"""Synthetic workload geometries for the per-KV-head fixed-budget cache.

Each workload fixes the cache geometry (sinks, scored slots, recent window),
the attention shape and the length of the synthetic token stream.  The cache
geometry at 4x compression follows the "Qwen3-8B-KVpop-4x" model card (intro):
at most 4,032 entries per KV head, made of 4 sink tokens, 3,772 scored
long-range tokens and a 256-token recent window.  The 88 % compression
geometry keeps the same sinks and window and a budget of 2,048.

Nothing here computes anything the method does; these are plain constants.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    wid: int                     # integer id, also the seed component
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_sink: int
    n_scored: int
    n_recent: int
    prompt_len: Optional[int]                 # fixed prompt length, or None
    prompt_len_range: Optional[Tuple[int, int]]  # inclusive range when drawn
    decode_steps: int
    score_dist: str              # "uniform" | "normal" | "qlognormal256"

    @property
    def budget(self) -> int:
        return self.n_sink + self.n_scored + self.n_recent

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


TINY = Workload(
    wid=1, name="tiny_single_head", n_layers=1, batch=1, n_q_heads=1,
    n_kv_heads=1, head_dim=64, n_sink=4, n_scored=44, n_recent=16,
    prompt_len=0, prompt_len_range=None, decode_steps=512,
    score_dist="uniform")

QWEN3_8B_LAYER_4X = Workload(
    wid=2, name="qwen3_8b_layer_4x", n_layers=1, batch=1, n_q_heads=32,
    n_kv_heads=8, head_dim=128, n_sink=4, n_scored=3772, n_recent=256,
    prompt_len=16384, prompt_len_range=None, decode_steps=1024,
    score_dist="normal")

QWEN3_8B_36L_4X = Workload(
    wid=3, name="qwen3_8b_36layer_4x", n_layers=36, batch=1, n_q_heads=32,
    n_kv_heads=8, head_dim=128, n_sink=4, n_scored=3772, n_recent=256,
    prompt_len=16384, prompt_len_range=None, decode_steps=4096,
    score_dist="normal")

LONG_131K_8X = Workload(
    wid=4, name="long_context_131k_8x", n_layers=36, batch=1, n_q_heads=32,
    n_kv_heads=8, head_dim=128, n_sink=4, n_scored=1788, n_recent=256,
    prompt_len=131072, prompt_len_range=None, decode_steps=2048,
    score_dist="normal")

BATCH64_SERVING = Workload(
    wid=5, name="batched_serving_b64", n_layers=1, batch=64, n_q_heads=32,
    n_kv_heads=8, head_dim=128, n_sink=4, n_scored=3772, n_recent=256,
    prompt_len=None, prompt_len_range=(4096, 32768), decode_steps=512,
    score_dist="qlognormal256")

# One GPU's share of the one-layer 4x workload under tensor parallelism over
# the 8 KV heads: one KV head and its 4 query heads (a measured shape only).
TP8_SHARE_4X = Workload(
    wid=6, name="qwen3_8b_layer_4x_tp8_share", n_layers=1, batch=1, n_q_heads=4,
    n_kv_heads=1, head_dim=128, n_sink=4, n_scored=3772, n_recent=256,
    prompt_len=16384, prompt_len_range=None, decode_steps=1024,
    score_dist="normal")

WORKLOADS = {w.wid: w for w in (TINY, QWEN3_8B_LAYER_4X, QWEN3_8B_36L_4X,
                                LONG_131K_8X, BATCH64_SERVING)}
BY_NAME = {w.name: w for w in WORKLOADS.values()}
