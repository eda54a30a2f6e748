"""KVpop per-KV-head fixed-budget sparse KV cache for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library (``libkvpop.so``, hand-written HIP
kernels) declared in ``include/kvpop.h``; ``fixed_budget_learned_amd.abi`` is
its thin ctypes binding.  Importing this package loads nothing.
"""
