"""The benchmark's byte accounting reproduces the memory figures the paper
prints for the context projection (paper §7.3, "KV Injection Mechanism and
Memory Overhead": D = 2048, BF16), and bench.py refuses more than one GPU."""
import os
import subprocess
import sys

import bench
from synth.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fc_memory_matches_the_paper():
    w, x_in, x_out = bench.fc_memory(2048, 2048, 5, 2)
    assert w == 5 * 2048 * 2048 * 2 and abs(w / 1e6 - 42) < 0.5         # "about 42 MB"
    assert abs(x_in / 1e6 - 42) < 2.5 and abs(x_out / 1e6 - 8.4) < 0.5  # "about 40 MB and 8 MB"
    assert bench.fc_memory(2048, 16, 5, 2)[1] < 400_000                  # block 16: "below 400 KB"


def test_draft_bytes_of_the_batch1_workload():
    s = CONFIGS[2]
    b = bench.algorithmic_bytes(s, [2048], 8, 1, 16)
    # layers 5 x 386 MB + LM head 1245 MB + 42 MB of context K/V
    assert abs(b["draft"] / 1e9 - 3.216) < 0.01
    assert abs(b["lm_head"] / 1e9 - 1.2447) < 0.001
    assert abs(b["kv_read"] / 1e6 - 41.9) < 0.1


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
