"""C-ABI contract checks that need no GPU.

The library must load, export every function include/kvpop.h declares, and
reject bad arguments before touching the HIP runtime.  Where a check reaches
the runtime on a host without a GPU it must report KVPOP_EHIP, not crash.
"""
import ctypes
import os
import re

import pytest

from fixed_budget_learned_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpop.h")


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVPOP_API\s+[\w\s\*]+?\b(kvpop_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return abi.load()


def test_header_declares_the_boundary():
    names = _header_functions()
    for want in ("kvpop_cache_create", "kvpop_prefill_compact", "kvpop_decode_step",
                 "kvpop_cache_state"):
        assert want in names
    assert set(names) == set(abi.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_error_codes_match_header():
    text = open(HEADER).read()
    for name, val in (("KVPOP_OK", abi.KVPOP_OK), ("KVPOP_EINVAL", abi.KVPOP_EINVAL),
                      ("KVPOP_ENOMEM", abi.KVPOP_ENOMEM), ("KVPOP_EHIP", abi.KVPOP_EHIP),
                      ("KVPOP_ESTATE", abi.KVPOP_ESTATE), ("KVPOP_ERANGE", abi.KVPOP_ERANGE)):
        m = re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % name, text)
        assert m and int(m.group(1)) == val, name


def test_strerror_strings(lib):
    seen = set()
    for code in (0, -1, -2, -3, -4, -5, 7):
        s = abi.strerror(code)
        assert isinstance(s, str) and s
        seen.add(s)
    assert len(seen) == 7


def _cfg(**kw):
    base = dict(n_layers=1, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                n_sink=4, n_scored=3772, n_recent=256)
    base.update(kw)
    return abi.make_config(**base)


def test_required_bytes_layout(lib):
    c = _cfg()
    nb = abi.required_bytes(c)
    kv = 2 * 8 * 4032 * 128 * 2
    assert nb >= kv + 8 * 4032 * (8 + 4) + 8 * 256 * 4
    assert nb % 256 == 0
    # K/V storage grows linearly with layers and sequences
    assert abi.required_bytes(_cfg(n_layers=36)) - nb >= 35 * (kv + 8 * 4032 * 12)
    # the Dynamic backend holds prune_interval more rows per head
    grow = abi.required_bytes(_cfg(prune_interval=256)) - nb
    assert grow >= 8 * 256 * (2 * 128 * 2 + 12)
    assert abi.required_bytes(_cfg(prune_interval=4096)) > 0


@pytest.mark.parametrize("bad", [
    dict(n_q_heads=30), dict(n_q_heads=48, n_kv_heads=4), dict(head_dim=96),
    dict(n_recent=0), dict(n_sink=-1), dict(n_scored=-2), dict(n_layers=0),
    dict(batch=0), dict(max_positions=0), dict(decode_splits=257),
    dict(softmax_scale=float("nan")), dict(n_kv_heads=0),
    dict(prune_interval=-1), dict(prune_interval=4097),
    dict(decode_finish=-1), dict(decode_finish=3),
])
def test_invalid_configs_rejected(lib, bad):
    c = _cfg(**bad)
    assert abi.required_bytes(c) == 0
    h = ctypes.c_void_p(123)
    assert lib.kvpop_cache_create(ctypes.byref(c), None, 0, ctypes.byref(h)) == abi.KVPOP_EINVAL
    assert h.value is None


def test_create_null_arguments(lib):
    c = _cfg()
    assert lib.kvpop_cache_create(None, None, 0, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_cache_create(ctypes.byref(c), None, 0, None) == abi.KVPOP_EINVAL


def test_misaligned_and_small_arena_rejected(lib):
    c = _cfg()
    h = ctypes.c_void_p()
    assert lib.kvpop_cache_create(ctypes.byref(c), 0x1001, 1 << 40, ctypes.byref(h)) == abi.KVPOP_EINVAL
    assert lib.kvpop_cache_create(ctypes.byref(c), 0x1000, 1024, ctypes.byref(h)) == abi.KVPOP_ENOMEM


def test_null_cache_handle_everywhere(lib):
    st = abi.State()
    assert lib.kvpop_prefill_compact(None, 0, 0, 4, 1, 1, 1, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_decode_step(None, 0, 1, 1, 1, 1, 1, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_cache_state(None, 0, 0, ctypes.byref(st), None, None, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_cache_reset(None, 0, 0, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_prefix_thresholds(None, 4, 1, 1, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_future_attention_target(None, 4, 1, 1, 1, 1, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_cache_prune(None, 0, None) == abi.KVPOP_EINVAL
    assert lib.kvpop_prefill_compact_batch(None, 1, None, None) == abi.KVPOP_EINVAL
    lib.kvpop_cache_destroy(None)


def test_create_without_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    c = _cfg(n_scored=44, n_recent=16, n_q_heads=1, n_kv_heads=1, head_dim=64)
    h = ctypes.c_void_p()
    assert lib.kvpop_cache_create(ctypes.byref(c), None, 0, ctypes.byref(h)) == abi.KVPOP_EHIP
    assert h.value is None


def test_noalloc_entry_point_validates_before_the_runtime(lib):
    """The no-allocation future target rejects a NULL cache before touching
    the HIP runtime (the size limit needs a cache and is checked on the GPU)."""
    vp = ctypes.c_void_p
    assert lib.kvpop_future_attention_target_noalloc(None, 16, vp(1), vp(1), vp(1), None) == \
        abi.KVPOP_EINVAL
