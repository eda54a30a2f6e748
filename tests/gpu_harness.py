"""Helpers for the GPU parity tests: drive the HIP path through the C ABI and
the oracle on the same seeded host arrays, and compare.

Acceptance bars (written once, used everywhere):
  kept sets        bit-exact (sorted positions of every KV head)
  attention output per (layer, sequence, step) tensor [Hq][D]:
                   max |gpu - oracle| <= 2e-2  and
                   ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2

Regression bar, beside it.  The kernels take bf16 inputs, compute the
softmax and P.V in fp32 and round the result to bf16 once, so every output
element is the exact (fp64) value rounded to bf16, up to fp32 round-off
that can flip a rounding decision: |gpu - oracle| <= one bf16 ulp of the
oracle value (2^(floor(log2|x|) - 7)) + 1e-6.  Measured on the one-layer 4x
workload the GPU's relative L2 error equals that of rounding the exact
output to bf16 (1.66e-3); one missing or duplicated kept row moves an
element by about p * |v - out|, several ulps there, and fails this bar.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

from fixed_budget_learned_amd import abi
from oracle import KVpopOracle, bf16_to_f64

ATOL_MAX = 2e-2
RTOL_L2 = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def to_dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_to_f64(bits)


REG_ABS = 1e-6


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits); 2^-133 at 0."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def check_output(gpu: np.ndarray, ref: np.ndarray, what: str):
    d = np.abs(gpu - ref)
    mx = float(d.max()) if d.size else 0.0
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert mx <= ATOL_MAX, f"{what}: max |err| {mx:.3e} > {ATOL_MAX}"
    assert rel <= RTOL_L2, f"{what}: relative L2 err {rel:.3e} > {RTOL_L2}"
    ulps = d / bf16_ulp(ref)
    bad = d > bf16_ulp(ref) + REG_ABS
    if bad.any():
        i = int(np.argmax(np.where(bad, ulps, 0)))
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond one bf16 ulp of the oracle "
                             f"(worst {float(ulps.flat[i]):.2f} ulp: gpu {float(gpu.flat[i]):.6e} "
                             f"oracle {float(ref.flat[i]):.6e})")
    return mx, rel


def check_kept(cache: abi.KVpopCache, layer: int, seq: int, orc: KVpopOracle, what: str):
    st = cache.state(layer, seq)
    assert st.n == orc.n, f"{what}: position {st.n} != {orc.n}"
    assert st.flags == 0, f"{what}: flags {st.flags}"
    for g in range(orc.Hkv):
        want = orc.kept(g)
        got = st.kept[g].tolist()
        if got != want:
            missing = sorted(set(want) - set(got))[:10]
            extra = sorted(set(got) - set(want))[:10]
            raise AssertionError(f"{what}: head {g} kept set differs "
                                 f"(|got|={len(got)}, |want|={len(want)}, missing {missing}, extra {extra})")


@dataclass
class Geo:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_sink: int
    n_scored: int
    n_recent: int


def make_cache(geo: Geo, n_layers=1, batch=1, decode_splits=0, max_positions=1 << 30,
               prune_interval=0, decode_finish=0):
    cfg = abi.make_config(n_layers, batch, geo.n_q_heads, geo.n_kv_heads, geo.head_dim,
                          geo.n_sink, geo.n_scored, geo.n_recent,
                          max_positions=max_positions, decode_splits=decode_splits,
                          prune_interval=prune_interval, decode_finish=decode_finish)
    return abi.KVpopCache(cfg)


def make_oracle(geo: Geo, dynamic: bool = False) -> KVpopOracle:
    return KVpopOracle(geo.n_q_heads, geo.n_kv_heads, geo.head_dim, geo.n_sink,
                       geo.n_scored, geo.n_recent, dynamic=dynamic)


class Stream:
    """Synthetic per-position inputs of one sequence (host arrays)."""

    def __init__(self, geo: Geo, T: int, seed: int, score_kind: str = "uniform"):
        rng = np.random.default_rng(seed)
        from fixed_budget_learned_amd.inputs import bf16_bits_rne
        H, Hq, D = geo.n_kv_heads, geo.n_q_heads, geo.head_dim
        self.k = bf16_bits_rne(rng.standard_normal((H, T, D), dtype=np.float32))
        self.v = bf16_bits_rne(rng.standard_normal((H, T, D), dtype=np.float32))
        self.q = bf16_bits_rne(rng.standard_normal((T, Hq, D), dtype=np.float32))
        if score_kind == "uniform":
            self.scores = rng.random((H, T), dtype=np.float32)
        elif score_kind == "normal":
            self.scores = rng.standard_normal((H, T), dtype=np.float32)
        elif score_kind == "ties":
            self.scores = rng.integers(0, 4, size=(H, T)).astype(np.float32)
        elif score_kind == "signed_zero_ties":
            self.scores = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(H, T))
        elif score_kind == "increasing":
            self.scores = np.tile(np.arange(T, dtype=np.float32), (H, 1))
        elif score_kind == "decreasing":
            self.scores = np.tile(-np.arange(T, dtype=np.float32), (H, 1))
        elif score_kind == "inf":
            self.scores = rng.choice(np.array([-np.inf, np.inf, 0.5, -3.0], np.float32), size=(H, T))
        else:
            raise ValueError(score_kind)
        self.W = geo.n_recent

    def leaving(self, n: int) -> np.ndarray:
        t = n - self.W
        H = self.scores.shape[0]
        return self.scores[:, t].copy() if t >= 0 else np.zeros(H, np.float32)
