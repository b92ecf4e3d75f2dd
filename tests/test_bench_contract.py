"""The benchmark's fixed figures and its command-line contract (CPU only).

The roofline fractions bench.py reports divide algorithmic bytes or flops by
measured time; these tests pin those per-unit figures to the values derived
from the shapes (state read and write, the token inputs and outputs, the
chunkwise products), and check that a request for more than one GPU is
refused before any device is touched.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_sequence_head():
    # fp32 state read and written (2 * 128 * 128 * 4), bf16 q, k, v (3 * 128 * 2),
    # fp32 per-channel gate (128 * 4), beta (4), bf16 output (128 * 2)
    assert bench.decode_bytes(1, 1, 128) == 131072 + 768 + 512 + 4 + 256 == 132612
    assert abs(bench.decode_bytes(256, 32, 128) / 1e9 - 1.0864) < 1e-4


def test_prefill_bytes_and_flops():
    # per token-head: q, k, v, o in bf16 (4 * 256), g fp32 (512), beta (4)
    assert bench.prefill_bytes(1, 1, 1, 128) - 2 * 128 * 128 * 4 == 1540
    assert abs(bench.prefill_bytes(1, 16, 4096, 128) / 1e6 - 103.0) < 0.05
    per = bench.prefill_flops(1, 1, 1, 128, 64)
    assert abs(per - (6 * 128 * 128 + 63 * 128 + 65 * 4 * 128 + 64 * 64 / 3)) < 1e-6
    assert round(per) == 141013
    assert abs(bench.prefill_flops(1, 16, 4096, 128, 64) / 1e9 - 9.24) < 0.01


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
