"""Host-side parts of bench.py: the selected-pair count behind the attention roofline figure
(against the oracle's selection mask), and the single-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_selected_pairs_counts_the_oracle_mask():
    rng = np.random.default_rng(3)
    for B, T, K in ((1, 64, 16), (2, 130, 40), (1, 257, 300)):
        topk = synth.random_topk(int(rng.integers(1 << 30)), B, T, K).copy()
        flat = topk.reshape(-1)
        n = flat.size
        flat[rng.integers(0, n, n // 10)] = flat[rng.integers(0, n, n // 10)]   # duplicates
        flat[rng.integers(0, n, n // 20)] = -1
        flat[rng.integers(0, n, n // 20)] = rng.integers(T, T + 9, n // 20)     # past the end
        want = int(oracle.selection_mask(topk, T).sum())
        assert bench.selected_pairs(topk) == want


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
