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


def test_executed_mfma_work_matches_the_counted_instructions():
    """The schedule formula behind executed_mfma_flop_per_launch against the MFMA instruction
    count rocprofv3 recorded for the headline launch (profiles/sparse_attn_traffic.txt): the
    headline selection flags every causal key tile."""
    topk = synth.make("headline", ("topk",))["topk"]
    tiles = bench.flagged_tiles(topk)
    assert tiles.sum() == 2 * bench.causal_tiles(4096)
    flop = bench.executed_mfma_flop(tiles)
    assert flop / (2 * 32 * 32 * 16) == 45350912
    rec = open(os.path.join(ROOT, "profiles", "sparse_attn_traffic.txt")).read()
    counted = float(rec.split("per dispatch: SQ_INSTS_MFMA ")[1].split(",")[0])
    assert abs(flop / (2 * 32 * 32 * 16) - counted) <= 5e-5 * counted
    # tiny shapes: one query tile, 8 waves, n scored key tiles
    assert bench.executed_mfma_flop(np.array([[1]])) == 128 * 8 * (24 + 40) * 32768
    assert bench.executed_mfma_flop(np.array([[2]])) == 128 * 8 * (24 + 80) * 32768


def test_flagged_tiles_against_the_oracle_mask():
    """flagged_tiles counts the 64-key tiles holding an allowed pair of each 256-query tile, as
    read off the oracle's dense allowed set; an item without any allowed key counts one tile."""
    rng = np.random.default_rng(5)
    for B, T, K in ((1, 64, 16), (2, 300, 40), (1, 700, 64)):
        topk = synth.random_topk(int(rng.integers(1 << 30)), B, T, K).copy()
        topk[:, 256:512:3] = -1
        if T > 512:
            topk[0, 512:] = np.minimum(topk[0, 512:], 100)     # keys of the first two tiles only
        allowed = oracle.selection_mask(topk, T)
        want = np.zeros((B, (T + 255) // 256), np.int64)
        for b in range(B):
            for qt in range(want.shape[1]):
                blk = allowed[b, 256 * qt:256 * qt + 256]
                want[b, qt] = max(1, sum(blk[:, 64 * k:64 * k + 64].any() for k in range((T + 63) // 64)))
        assert np.array_equal(bench.flagged_tiles(topk), want)
    assert bench.flagged_tiles(np.full((1, 10, 4), -1, np.int32)).tolist() == [[1]]
    assert bench.causal_tiles(64) == 1 and bench.causal_tiles(65) == 2 and bench.causal_tiles(300) == 4 + 5


def test_attention_clock_falls_back_to_the_counter_record():
    """An amdsmi engine-clock sample outside the plausible range under load (an idle or
    per-partition reading) is replaced by the clock from the kernel's counter record, which
    matches the current kernel source."""
    rec = bench.attn_counter_record("gfx_clock_mhz")
    assert rec is not None and 1000 <= rec <= 2600
    assert bench.attention_clock(1950.0) == (1950.0, bench.attention_clock(1950.0)[1])
    assert "amdsmi" in bench.attention_clock(1950.0)[1]
    for bad in (None, 660.0, 9000.0):
        clk, src = bench.attention_clock(bad)
        assert clk == rec and "counters" in src
