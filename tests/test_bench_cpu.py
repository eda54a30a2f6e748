"""Host-side pieces of bench.py: the kernel-source hash that ties the stored
HBM counters to the decode kernel, and the one-GPU contract."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = """// header comment
template <int D> __global__ void k(float* p) {  // trailing comment
  /* block
     comment */ p[threadIdx.x] = 1.f;

}
"""


def test_comment_edits_keep_the_hash_input():
    edited = SRC.replace("// header comment", "// another header").replace("block", "blk")
    assert bench._strip_comments(edited) == bench._strip_comments(SRC)
    assert "comment" not in bench._strip_comments(SRC)
    assert "p[threadIdx.x] = 1.f;" in bench._strip_comments(SRC)


def test_code_edits_change_the_hash_input():
    changed = SRC.replace("1.f", "2.f")
    assert bench._strip_comments(changed) != bench._strip_comments(SRC)


def test_kernel_hash_is_stable():
    assert bench._kernel_hash() == bench._kernel_hash()
    assert len(bench._kernel_hash()) == 40


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
