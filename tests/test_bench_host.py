"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes it divides by are the ones derived by hand from the workload shapes,
and a request for more than one GPU ends with a message."""

import subprocess
import sys
import os

import bench
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_256k():
    spec = WORKLOADS["qwen7b_ctx256k_l28"]
    ab = bench.algorithmic_bytes(spec, 262144, 1639, 2)
    H, g, d, e = 4, 7, 128, 2
    assert ab["desc"] == H * 16384 * 2 * d * e == 33554432  # min and max row per block and KV head
    assert ab["kv"] == H * 1639 * 16 * 2 * d * e == 53706752  # K and V rows of the selected blocks (full tail)
    assert ab["q"] == H * g * d * e and ab["out"] == H * g * d * 4
    assert ab["total"] == 87282688
    assert ab["kv"] + ab["q"] + ab["out"] == 53728256  # the sparse decode call's bytes


def test_algorithmic_bytes_partial_tail():
    spec = WORKLOADS["qwen7b_ctx32k_b1"]
    ab = bench.algorithmic_bytes(spec, 16 * 100 + 3, 11, 2)
    # ten full selected blocks plus the tail block's three valid rows
    assert ab["kv"] == 4 * (10 * 16 + 3) * 2 * 128 * 2
    assert ab["desc"] == 4 * 101 * 2 * 128 * 2


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_tables_read_fresh_data():
    """The sweep and workload tables cycle through enough layer caches that
    one replay touches more than 1 GiB, four times the last-level cache."""
    base = WORKLOADS["qwen7b_ctx256k_l28"]
    for L in (16384, 65536, 262144):
        nl = bench.layers_for_fresh_reads(base, [L])
        n = max(16, -(-((L + 15) // 16) // 10))
        assert nl * bench.algorithmic_bytes(base, L, n, 2)["total"] >= 1 << 30
        assert 2 <= nl <= 256
