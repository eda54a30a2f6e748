"""The binding loaded before anything imports torch (ctypes load first, torch
second) still shares torch's HIP runtime: a cache can be created and a step
run.  Run in a fresh interpreter, since the test process has torch loaded."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
from fixed_budget_learned_amd import abi
abi.load()                      # before this script imports torch
import torch
cache = abi.KVpopCache(abi.make_config(1, 1, 4, 1, 64, 1, 8, 4))
q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
kv = torch.zeros((1, 1, 64), dtype=torch.bfloat16, device="cuda")
sc = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
cache.decode_step(0, q, kv, kv, sc, out)
torch.cuda.synchronize()
cache.close()
print("ok")
"""


@pytest.mark.gpu
def test_library_loaded_before_torch():
    print("case: abi.load() before import torch, fresh interpreter", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
