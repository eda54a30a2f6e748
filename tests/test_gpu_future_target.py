"""Parity of the future-attention target kernels (through the C ABI) with the
oracle.  Both sides read the same bf16 q and k; the GPU multiplies them on
bf16 MFMA with fp32 accumulation and takes exponentials and logarithms in
fp32, so each y[g][j] (a sum of at most G * T probabilities) is held to
|err| <= 1e-3 * (1 + |y|).
"""
import math

import numpy as np
import pytest
import torch

from gpu_harness import Geo, log, make_cache, to_dev_bf16
from fixed_budget_learned_amd import abi
from fixed_budget_learned_amd.inputs import bf16_bits_rne
from oracle import future_attention_target

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


def _run(Hq, Hkv, D, W, T, q, k, with_work=False):
    geo = Geo(Hq, Hkv, D, 4, 16, W)
    cache = make_cache(geo, max_positions=max(T, 1))
    work = torch.full((2, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((Hkv, T), float("nan"), dtype=torch.float32, device="cuda")
    cache.future_attention_target(to_dev_bf16(q), to_dev_bf16(k), work, y)
    got = y.cpu().numpy().astype(np.float64)
    cache.close()
    if with_work:
        return got, work.cpu().numpy().astype(np.float64)
    return got


CASES = [
    # Hq, Hkv, D, W, T, scale of the random q/k
    (4, 2, 64, 5, 300, 1.0),
    (8, 2, 128, 16, 1000, 1.0),
    (4, 4, 128, 1, 777, 2.0),
    (8, 1, 64, 3, 129, 3.0),
    (2, 1, 128, 64, 64, 1.0),
    (32, 8, 128, 256, 2048, 1.0),
]


@pytest.mark.parametrize("Hq,Hkv,D,W,T,sd", CASES,
                         ids=[f"hq{c[0]}_hkv{c[1]}_d{c[2]}_w{c[3]}_t{c[4]}" for c in CASES])
def test_future_target_matches_oracle(Hq, Hkv, D, W, T, sd):
    rng = np.random.default_rng(Hq * 1000 + T)
    q = bf16_bits_rne((sd * rng.standard_normal((Hq, T, D))).astype(np.float32))
    k = bf16_bits_rne(rng.standard_normal((Hkv, T, D)).astype(np.float32))
    log(f"future target Hq={Hq} Hkv={Hkv} D={D} W={W} T={T}")
    got = _run(Hq, Hkv, D, W, T, q, k)
    want = future_attention_target(q, k, W, 1.0 / math.sqrt(D))
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    assert np.all(err <= 1e-3 * (1.0 + np.abs(want))), \
        f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


def test_per_head_shares_and_lse():
    """work[1][h] is head h's own target (the oracle on that head alone), and
    work[0][h][i] the log2 of the causal softmax denominator of query i."""
    Hq, Hkv, D, W, T = 8, 2, 64, 9, 400
    rng = np.random.default_rng(21)
    q = bf16_bits_rne((1.5 * rng.standard_normal((Hq, T, D))).astype(np.float32))
    k = bf16_bits_rne(rng.standard_normal((Hkv, T, D)).astype(np.float32))
    y, work = _run(Hq, Hkv, D, W, T, q, k, with_work=True)
    scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    for h in range(Hq):
        want = future_attention_target(q[h:h + 1], k[h // G:h // G + 1], W, scale)[0]
        assert np.all(np.abs(work[1][h] - want) <= 1e-3 * (1.0 + np.abs(want))), h
    # lse of a few queries of head 3, from the definition in fp64
    qf = q.astype(np.uint32) << 16
    kf = k.astype(np.uint32) << 16
    qf = qf.view(np.float32).astype(np.float64)
    kf = kf.view(np.float32).astype(np.float64)
    for i in (0, 1, 63, 64, 200, T - 1):
        s = scale * (kf[0, :i + 1] @ qf[3, i])
        want = (s.max() + np.log(np.exp(s - s.max()).sum())) / math.log(2.0)
        assert abs(work[0][3][i] - want) <= 1e-3 * (1.0 + abs(want)), i
    assert np.allclose(y, work[1].reshape(Hkv, G, T).sum(axis=1), rtol=1e-6, atol=1e-6)


def test_uniform_attention_harmonic_sums_on_gpu():
    """q = 0: y[j] = G * (H_T - H_{j+W}), computed on the GPU."""
    Hq, Hkv, D, W, T = 8, 2, 128, 7, 500
    rng = np.random.default_rng(9)
    q = np.zeros((Hq, T, D), np.uint16)
    k = bf16_bits_rne(rng.standard_normal((Hkv, T, D)).astype(np.float32))
    got = _run(Hq, Hkv, D, W, T, q, k)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    G = Hq // Hkv
    want = np.array([G * (H[T] - H[j + W]) if j + W < T else 0.0 for j in range(T)])
    for g in range(Hkv):
        assert np.abs(got[g] - want).max() <= 1e-3 * (1 + want.max())


def test_window_past_the_end_gives_zero():
    Hq, Hkv, D, T = 4, 2, 64, 100
    rng = np.random.default_rng(10)
    q = bf16_bits_rne(rng.standard_normal((Hq, T, D)).astype(np.float32))
    k = bf16_bits_rne(rng.standard_normal((Hkv, T, D)).astype(np.float32))
    assert np.all(_run(Hq, Hkv, D, T, T, q, k) == 0.0)
