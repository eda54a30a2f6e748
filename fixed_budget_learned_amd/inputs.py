"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module only draws random numbers and packs them; it holds none of the
cache method's arithmetic.  Every tensor is a pure function of
(workload id, layer, sequence, tensor id) through NumPy's PCG64 seeded with
SeedSequence([20260706, workload, layer, seq, tensor]).

Tensor ids: 0 prompt/stream K, 1 stream V, 2 scores, 3 q, 6 prompt lengths.
K/V/q are drawn as float32 N(0,1) and rounded to bfloat16 with
round-to-nearest-even; they are handed around as uint16 bit patterns.

Scores by distribution:
  uniform        float32 U(0,1)
  normal         float32 N(0,1)
  qlognormal256  x = exp(z), z ~ N(0,1); level = min(255, floor(32 x));
                 score = level / 32 (exact in float32; 256 levels, many ties)
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

SEED_ROOT = 20260706
T_K, T_V, T_SCORES, T_Q, T_PROMPT_LENS = 0, 1, 2, 3, 6


def rng_for(wid: int, layer: int, seq: int, tensor_id: int) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, int(wid), int(layer), int(seq), int(tensor_id)])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits_rne(rng.standard_normal(shape, dtype=np.float32))


def draw_scores(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        return rng.random(shape, dtype=np.float32)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "qlognormal256":
        z = rng.standard_normal(shape, dtype=np.float64)
        level = np.minimum(255.0, np.floor(32.0 * np.exp(z)))
        return (level / 32.0).astype(np.float32)
    raise ValueError(f"unknown score distribution {dist!r}")


def prompt_lengths(w: Workload) -> np.ndarray:
    """Prompt length of every sequence of the workload (int64 [batch])."""
    if w.prompt_len is not None:
        return np.full(w.batch, w.prompt_len, dtype=np.int64)
    lo, hi = w.prompt_len_range
    return rng_for(w.wid, 0, 0, T_PROMPT_LENS).integers(lo, hi, size=w.batch, endpoint=True)


class TokenStream:
    """All per-position inputs of one (layer, sequence) stream.

    k, v    uint16 [Hkv][T][D]  bf16 K/V of positions 0..T-1
    scores  float32 [Hkv][T]    per-(KV head, position) score
    q       uint16 [steps][Hq][D] query of each decode step
    The first ``prompt_len`` positions form the prompt; decode step i
    (0-based) processes position prompt_len + i.
    """

    def __init__(self, w: Workload, layer: int, seq: int, prompt_len: int, steps: int):
        self.w, self.layer, self.seq = w, layer, seq
        self.prompt_len, self.steps = int(prompt_len), int(steps)
        T = self.prompt_len + self.steps
        self.T = T
        Hkv, Hq, D = w.n_kv_heads, w.n_q_heads, w.head_dim
        self.k = normal_bf16(rng_for(w.wid, layer, seq, T_K), (Hkv, T, D))
        self.v = normal_bf16(rng_for(w.wid, layer, seq, T_V), (Hkv, T, D))
        self.scores = draw_scores(rng_for(w.wid, layer, seq, T_SCORES), w.score_dist, (Hkv, T))
        self.q = normal_bf16(rng_for(w.wid, layer, seq, T_Q), (self.steps, Hq, D))

    # --- slices in the layouts the cache calls take -------------------------
    def prompt_k(self):
        return np.ascontiguousarray(self.k[:, :self.prompt_len])

    def prompt_v(self):
        return np.ascontiguousarray(self.v[:, :self.prompt_len])

    def prompt_scores(self):
        return np.ascontiguousarray(self.scores[:, :self.prompt_len])

    def step_kv(self):
        """k_new/v_new of every decode step: uint16 [steps][Hkv][D] each."""
        P = self.prompt_len
        k = np.ascontiguousarray(self.k[:, P:].transpose(1, 0, 2))
        v = np.ascontiguousarray(self.v[:, P:].transpose(1, 0, 2))
        return k, v

    def step_leaving_scores(self):
        """Score handed to decode step i: that of position (P + i) - W.

        float32 [steps][Hkv]; zero where that position is negative (the call
        ignores the value whenever no scored token leaves the window).
        """
        W = self.w.n_recent
        out = np.zeros((self.steps, self.w.n_kv_heads), dtype=np.float32)
        for i in range(self.steps):
            t = self.prompt_len + i - W
            if t >= 0:
                out[i] = self.scores[:, t]
        return out
