"""Device-clock timeline of one batch-1 decode step (the one-layer Qwen3-8B
workload at 4x: 32 query heads, 8 KV heads, D 128, budget 4,032, after a
16,384-token prefill), from the timeline build of the library:

    python -m fixed_budget_learned_amd.build --timeline    # here, once
    python -m fixed_budget_learned_amd.timeline            # on the GPU

Thread 0 of every workgroup stamps s_memrealtime (100 MHz) at eight points of
the step.  Each sample runs BURST steps back to back (queued behind a
spinning kernel, as a decode loop runs them) and keeps the stamps of the last
one, timed from its first workgroup's start; earlier steps' stamps left in
the buffer (a finisher of an earlier step) predate it and are dropped.  The
table gives the median and maximum over workgroups and samples.
"""
from __future__ import annotations

import ctypes
import os
import sys

POINTS = [
    "workgroup start",
    "chunk loop done (wave 0)",
    "in-workgroup reduction and barrier",
    "partial state stored (issued)",
    "stores acknowledged",
    "ticket returned",
    "finisher: split factors and barrier",
    "finisher done, stores acknowledged",
]


BURST = 8


def main(samples: int = 64) -> None:
    import numpy as np
    import torch
    from fixed_budget_learned_amd import abi, build
    from fixed_budget_learned_amd.configs import QWEN3_8B_LAYER_4X as w

    if not os.path.exists(build.TIMELINE_LIB_PATH):
        sys.exit(f"{build.TIMELINE_LIB_PATH} is missing: run "
                 "`python -m fixed_budget_learned_amd.build --timeline` first")
    abi.LIB_PATH = build.TIMELINE_LIB_PATH
    lib = abi.load()
    lib.kvpop_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    Hq, Hkv, D, P = w.n_q_heads, w.n_kv_heads, w.head_dim, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    cache = abi.KVpopCache(abi.make_config(1, 1, Hq, Hkv, D, w.n_sink, w.n_scored, w.n_recent))
    cache.prefill_compact(0, 0,
                          torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16),
                          torch.randn((Hkv, P, D), generator=gen, device="cuda").to(torch.bfloat16),
                          torch.randn((Hkv, P), generator=gen, device="cuda"))
    q = torch.randn((1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    kn = torch.randn((1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((1, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((1, Hq, D), dtype=torch.bfloat16, device="cuda")
    sl = torch.randn((BURST, 1, Hkv), generator=gen, device="cuda")
    nwg = 256
    host = np.zeros((nwg, 8), np.uint64)
    rows = []
    for i in range(samples + 2):
        if lib.kvpop_timeline_clear() != 0:
            raise RuntimeError("kvpop_timeline_clear failed")
        torch.cuda.synchronize()
        torch.cuda._sleep(2_400_000)  # about 1 ms: the burst is queued before it runs
        for b in range(BURST):
            cache.decode_step(0, q, kn, vn, sl[b], out)
        torch.cuda.synchronize()
        if lib.kvpop_timeline_read(host.ctypes.data, nwg) != 0:
            raise RuntimeError("kvpop_timeline_read failed")
        if i >= 2:  # the first samples warm the code and the caches
            rows.append(host.astype(np.int64).copy())
    cache.close()
    print(f"| point | median us | max us | stamps |")
    print("|---|---|---|---|")
    for j, name in enumerate(POINTS):
        vals = []
        for a in rows:
            t0 = a[:, 0][a[:, 0] > 0].min()
            v = a[:, j][a[:, j] >= t0]
            vals.extend(((v - t0) * 0.01).tolist())  # 100 MHz ticks -> us
        if vals:
            print(f"| {name} | {np.median(vals):.2f} | {max(vals):.2f} | {len(vals)} |")
    print(f"\n{samples} samples of the last of {BURST} back-to-back steps, {nwg} workgroups "
          "each (32 splits x 8 KV heads); the finisher rows come from one workgroup per head.")


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 64)
