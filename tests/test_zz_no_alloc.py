"""The no-allocation future-target entry point against the one that takes a
workspace argument: same kernels, so the targets must agree bit for bit, on
two calls in a row (the second with a smaller input, so the static
workspace holds the first call's contents when the second starts), and a
size beyond the static workspace is rejected before anything runs."""
import numpy as np
import pytest
import torch

from gpu_harness import Geo, log, make_cache, to_dev_bf16
from fixed_budget_learned_amd import abi
from fixed_budget_learned_amd.inputs import bf16_bits_rne

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    abi.load()
    torch.cuda.init()


def _qk(rng, Hq, Hkv, T, D):
    q = bf16_bits_rne(rng.standard_normal((Hq, T, D)).astype(np.float32))
    k = bf16_bits_rne(rng.standard_normal((Hkv, T, D)).astype(np.float32))
    return to_dev_bf16(q), to_dev_bf16(k)


@pytest.mark.parametrize("Hq,Hkv,D,W,T1,T2", [(32, 8, 128, 256, 4096, 1000),
                                              (8, 2, 64, 16, 700, 129)])
def test_noalloc_matches_workspace_entry_point(Hq, Hkv, D, W, T1, T2):
    log(f"no-alloc future target Hq={Hq} Hkv={Hkv} D={D} W={W} T={T1} then {T2}")
    cache = make_cache(Geo(Hq, Hkv, D, 4, 16, W), max_positions=T1)
    rng = np.random.default_rng(Hq + T1)
    for T in (T1, T2):
        q, k = _qk(rng, Hq, Hkv, T, D)
        work = torch.full((2, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
        y_ref = torch.full((Hkv, T), float("nan"), dtype=torch.float32, device="cuda")
        y_new = torch.full((Hkv, T), float("nan"), dtype=torch.float32, device="cuda")
        cache.future_attention_target(q, k, work, y_ref)
        cache.future_attention_target_noalloc(q, k, y_new)
        torch.cuda.synchronize()
        assert torch.isfinite(y_new).all()
        assert torch.equal(y_new, y_ref), f"T={T}: targets differ"
    cache.close()


def test_noalloc_rejects_sizes_beyond_the_static_workspace():
    Hq, Hkv, D = 32, 8, 128
    T = (32 << 20) // (2 * Hq * 4) + 1          # one token past 32 MiB of workspace
    cache = make_cache(Geo(Hq, Hkv, D, 4, 16, 256), max_positions=T)
    q = torch.zeros((Hq, T, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((Hkv, T, D), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((Hkv, T), dtype=torch.float32, device="cuda")
    with pytest.raises(abi.KVpopError) as e:
        cache.future_attention_target_noalloc(q, k, y)
    assert e.value.code == abi.KVPOP_ERANGE
    # the largest size that fits is accepted
    T = (32 << 20) // (2 * Hq * 4)
    cache.future_attention_target_noalloc(q[:, :T].contiguous(), k[:, :T].contiguous(),
                                          y[:, :T].contiguous())
    torch.cuda.synchronize()
    cache.close()
