"""ctypes binding of ``libkvpop.so`` (declared in include/kvpop.h).

Argument marshalling only: every step of the cache path runs in the HIP
kernels behind the C ABI.  Tensors are PyTorch tensors on the GPU (PyTorch
provides the device memory and streams); this module checks their dtype,
shape, device and contiguity, then passes raw pointers.  A missing library
raises ``KVpopLibraryMissing``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvpop.so")

KVPOP_OK, KVPOP_EINVAL, KVPOP_ENOMEM, KVPOP_EHIP, KVPOP_ESTATE, KVPOP_ERANGE = 0, -1, -2, -3, -4, -5
KVPOP_FLAG_NAN_SCORE = 1

EXPORTED = ("kvpop_cache_required_bytes", "kvpop_cache_create", "kvpop_cache_destroy",
            "kvpop_cache_reset", "kvpop_prefill_compact", "kvpop_decode_step",
            "kvpop_cache_state", "kvpop_strerror",
            "kvpop_prefix_thresholds", "kvpop_future_attention_target", "kvpop_cache_prune",
            "kvpop_prefill_compact_batch", "kvpop_future_attention_target_noalloc",
            "kvpop_decode_step_layers")


class KVpopLibraryMissing(RuntimeError):
    pass


class KVpopError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_scored", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("max_positions", ctypes.c_int32), ("decode_splits", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("prune_interval", ctypes.c_int32),
                ("decode_finish", ctypes.c_int32)]


class PrefillItem(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("seq", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("scores", ctypes.c_void_p)]


class State(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (built by fixed_budget_learned_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KVpopLibraryMissing(
            f"{LIB_PATH} is missing; build it with `python -m fixed_budget_learned_amd.build`")
    # torch ships its own HIP runtime.  Loaded first, it is the one the
    # library binds to; loaded after the library, a second runtime comes up
    # whose device memory and streams the library cannot use (cache creation
    # then fails with a HIP error).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kvpop_cache_required_bytes.argtypes = [ctypes.POINTER(Config)]
    lib.kvpop_cache_required_bytes.restype = sz
    lib.kvpop_cache_create.argtypes = [ctypes.POINTER(Config), vp, sz, ctypes.POINTER(vp)]
    lib.kvpop_cache_create.restype = ctypes.c_int
    lib.kvpop_cache_destroy.argtypes = [vp]
    lib.kvpop_cache_destroy.restype = None
    lib.kvpop_cache_reset.argtypes = [vp, i32, i32, vp]
    lib.kvpop_cache_reset.restype = ctypes.c_int
    lib.kvpop_prefill_compact.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    lib.kvpop_prefill_compact.restype = ctypes.c_int
    lib.kvpop_decode_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.kvpop_decode_step.restype = ctypes.c_int
    lib.kvpop_cache_state.argtypes = [vp, i32, i32, ctypes.POINTER(State), vp, vp, vp]
    lib.kvpop_cache_state.restype = ctypes.c_int
    lib.kvpop_prefix_thresholds.argtypes = [vp, i32, vp, vp, vp]
    lib.kvpop_prefix_thresholds.restype = ctypes.c_int
    lib.kvpop_future_attention_target.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    lib.kvpop_future_attention_target.restype = ctypes.c_int
    lib.kvpop_decode_step_layers.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.kvpop_decode_step_layers.restype = ctypes.c_int
    lib.kvpop_future_attention_target_noalloc.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.kvpop_future_attention_target_noalloc.restype = ctypes.c_int
    lib.kvpop_prefill_compact_batch.argtypes = [vp, i32, ctypes.POINTER(PrefillItem), vp]
    lib.kvpop_prefill_compact_batch.restype = ctypes.c_int
    lib.kvpop_cache_prune.argtypes = [vp, i32, vp]
    lib.kvpop_cache_prune.restype = ctypes.c_int
    lib.kvpop_strerror.argtypes = [ctypes.c_int]
    lib.kvpop_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().kvpop_strerror(int(code)).decode()


def make_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, n_sink, n_scored, n_recent,
                max_positions=1 << 30, decode_splits=0, softmax_scale=0.0,
                prune_interval=0, decode_finish=0) -> Config:
    """prune_interval 0: Static backend; P >= 1: Dynamic backend pruned after
    every P-th decode step of a layer.  decode_finish 0: the library chooses
    how split heads are merged; 1: in the same launch; 2: in a second launch
    (see the header)."""
    return Config(int(n_layers), int(batch), int(n_q_heads), int(n_kv_heads), int(head_dim),
                  int(n_sink), int(n_scored), int(n_recent), int(max_positions),
                  int(decode_splits), float(softmax_scale), int(prune_interval),
                  int(decode_finish))


def required_bytes(cfg: Config) -> int:
    return int(load().kvpop_cache_required_bytes(ctypes.byref(cfg)))


@dataclass
class HeadState:
    n: int
    flags: int
    counts: np.ndarray          # [Hkv]
    kept: List[np.ndarray]      # per KV head, ascending positions


def _check(code: int, what: str):
    if code != KVPOP_OK:
        raise KVpopError(code, what)


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t, dtype, shape, name: str) -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return int(t.data_ptr())


class KVpopCache:
    """A fixed-budget cache on the current GPU (one handle of the C ABI)."""

    def __init__(self, cfg: Config, arena=None):
        lib = load()
        self.cfg = cfg
        self.budget = cfg.n_sink + cfg.n_scored + cfg.n_recent
        self.capacity = self.budget + cfg.prune_interval   # rows per KV head
        self._arena = arena
        h = ctypes.c_void_p()
        ptr, nbytes = None, 0
        if arena is not None:
            ptr, nbytes = int(arena.data_ptr()), arena.numel() * arena.element_size()
        _check(lib.kvpop_cache_create(ctypes.byref(cfg), ptr, nbytes, ctypes.byref(h)),
               "kvpop_cache_create")
        self._h = h

    @property
    def handle(self) -> int:
        return self._h.value

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load().kvpop_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, layer: int, seq: int, stream=None):
        _check(load().kvpop_cache_reset(self._h, layer, seq, _stream_ptr(stream)),
               "kvpop_cache_reset")

    def prefill_compact(self, layer: int, seq: int, k, v, scores, stream=None):
        import torch
        c = self.cfg
        P = int(k.shape[1]) if k is not None and k.dim() == 3 else 0
        kp = _dev_ptr(k, torch.bfloat16, (c.n_kv_heads, P, c.head_dim), "k")
        vp = _dev_ptr(v, torch.bfloat16, (c.n_kv_heads, P, c.head_dim), "v")
        sp = _dev_ptr(scores, torch.float32, (c.n_kv_heads, P), "scores")
        _check(load().kvpop_prefill_compact(self._h, layer, seq, P, kp, vp, sp,
                                            _stream_ptr(stream)), "kvpop_prefill_compact")

    def prefill_compact_batch(self, items, stream=None):
        """Compact several prompts at once: items is a sequence of
        (layer, seq, k, v, scores) with the tensors of prefill_compact."""
        import torch
        c = self.cfg
        arr = (PrefillItem * max(1, len(items)))()
        for i, (layer, seq, k, v, scores) in enumerate(items):
            P = int(k.shape[1]) if k is not None and k.dim() == 3 else 0
            arr[i].layer, arr[i].seq, arr[i].n_tokens, arr[i].pad = int(layer), int(seq), P, 0
            arr[i].k = _dev_ptr(k, torch.bfloat16, (c.n_kv_heads, P, c.head_dim), "k")
            arr[i].v = _dev_ptr(v, torch.bfloat16, (c.n_kv_heads, P, c.head_dim), "v")
            arr[i].scores = _dev_ptr(scores, torch.float32, (c.n_kv_heads, P), "scores")
        _check(load().kvpop_prefill_compact_batch(self._h, len(items), arr, _stream_ptr(stream)),
               "kvpop_prefill_compact_batch")

    def decode_step(self, layer: int, q, k_new, v_new, score_leaving, out, stream=None):
        import torch
        c = self.cfg
        B = c.batch
        qp = _dev_ptr(q, torch.bfloat16, (B, c.n_q_heads, c.head_dim), "q")
        kp = _dev_ptr(k_new, torch.bfloat16, (B, c.n_kv_heads, c.head_dim), "k_new")
        vp = _dev_ptr(v_new, torch.bfloat16, (B, c.n_kv_heads, c.head_dim), "v_new")
        sp = _dev_ptr(score_leaving, torch.float32, (B, c.n_kv_heads), "score_leaving")
        op = _dev_ptr(out, torch.bfloat16, (B, c.n_q_heads, c.head_dim), "out")
        _check(load().kvpop_decode_step(self._h, layer, qp, kp, vp, sp, op, _stream_ptr(stream)),
               "kvpop_decode_step")

    def decode_step_layers(self, layer0: int, q, k_new, v_new, score_leaving, out, stream=None):
        """One decode step of layers layer0 .. layer0 + n - 1 in one launch (n
        = q.shape[0]); every tensor of decode_step with a leading layer
        dimension.  Only for layers whose inputs are independent of each
        other's outputs (see the header)."""
        import torch
        c = self.cfg
        B = c.batch
        n = int(q.shape[0]) if q is not None and q.dim() == 4 else 0
        qp = _dev_ptr(q, torch.bfloat16, (n, B, c.n_q_heads, c.head_dim), "q")
        kp = _dev_ptr(k_new, torch.bfloat16, (n, B, c.n_kv_heads, c.head_dim), "k_new")
        vp = _dev_ptr(v_new, torch.bfloat16, (n, B, c.n_kv_heads, c.head_dim), "v_new")
        sp = _dev_ptr(score_leaving, torch.float32, (n, B, c.n_kv_heads), "score_leaving")
        op = _dev_ptr(out, torch.bfloat16, (n, B, c.n_q_heads, c.head_dim), "out")
        _check(load().kvpop_decode_step_layers(self._h, layer0, n, qp, kp, vp, sp, op,
                                               _stream_ptr(stream)), "kvpop_decode_step_layers")

    def prune(self, layer: int, stream=None):
        """Dynamic backend: prune every head of `layer` back to the budget now."""
        _check(load().kvpop_cache_prune(self._h, layer, _stream_ptr(stream)), "kvpop_cache_prune")

    def prefix_thresholds(self, scores, thr, stream=None):
        """Threshold key of every prompt position per KV head (see the
        header): scores float32 [Hkv][P] in, thr int64 [Hkv][P] out (the
        uint64 keys' bits)."""
        import torch
        c = self.cfg
        P = int(scores.shape[1]) if scores is not None and scores.dim() == 2 else 0
        sp = _dev_ptr(scores, torch.float32, (c.n_kv_heads, P), "scores")
        tp = _dev_ptr(thr, torch.int64, (c.n_kv_heads, P), "thr")
        _check(load().kvpop_prefix_thresholds(self._h, P, sp, tp, _stream_ptr(stream)),
               "kvpop_prefix_thresholds")

    def future_attention_target(self, q, k, work, y, stream=None):
        """Future-attention target (see the header): q bf16 [Hq][T][D],
        k bf16 [Hkv][T][D], work float32 [2][Hq][T] workspace (work[0]
        receives the log2-domain log-sum-exps, work[1] each query head's
        share), y float32 [Hkv][T] out."""
        import torch
        c = self.cfg
        T = int(q.shape[1]) if q is not None and q.dim() == 3 else 0
        qp = _dev_ptr(q, torch.bfloat16, (c.n_q_heads, T, c.head_dim), "q")
        kp = _dev_ptr(k, torch.bfloat16, (c.n_kv_heads, T, c.head_dim), "k")
        wp = _dev_ptr(work, torch.float32, (2, c.n_q_heads, T), "work")
        yp = _dev_ptr(y, torch.float32, (c.n_kv_heads, T), "y")
        _check(load().kvpop_future_attention_target(self._h, T, qp, kp, wp, yp,
                                                    _stream_ptr(stream)),
               "kvpop_future_attention_target")

    def future_attention_target_noalloc(self, q, k, y, stream=None):
        """The future-attention target with the library's static workspace
        instead of a caller-provided one (see the header): q bf16 [Hq][T][D],
        k bf16 [Hkv][T][D], y float32 [Hkv][T] out."""
        import torch
        c = self.cfg
        T = int(q.shape[1]) if q is not None and q.dim() == 3 else 0
        qp = _dev_ptr(q, torch.bfloat16, (c.n_q_heads, T, c.head_dim), "q")
        kp = _dev_ptr(k, torch.bfloat16, (c.n_kv_heads, T, c.head_dim), "k")
        yp = _dev_ptr(y, torch.float32, (c.n_kv_heads, T), "y")
        _check(load().kvpop_future_attention_target_noalloc(self._h, T, qp, kp, yp,
                                                            _stream_ptr(stream)),
               "kvpop_future_attention_target_noalloc")

    def state(self, layer: int, seq: int, stream=None) -> HeadState:
        c = self.cfg
        st = State()
        counts = np.zeros(c.n_kv_heads, dtype=np.int32)
        kept = np.zeros((c.n_kv_heads, self.capacity), dtype=np.int32)
        _check(load().kvpop_cache_state(self._h, layer, seq, ctypes.byref(st),
                                        counts.ctypes.data, kept.ctypes.data,
                                        _stream_ptr(stream)), "kvpop_cache_state")
        return HeadState(st.n, st.flags, counts,
                         [kept[g, :counts[g]].copy() for g in range(c.n_kv_heads)])
