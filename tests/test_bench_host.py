"""Host-side checks of bench.py's work accounting (no GPU): the executed-pair
and executed-block counts against plain loops on small random selections, and
the refusal of more than one GPU."""

import subprocess
import sys

import numpy as np

import bench


def _loops(offN, offM, idx, rows, tile):
    P_N, s = idx.shape
    pairs = q_blocks = 0
    for p in range(P_N):
        t = offN[p + 1] - offN[p]
        keys = sum(offM[q + 1] - offM[q] for q in idx[p])
        pairs += t * keys
        q_blocks += ((t + rows - 1) // rows) * rows * ((keys + tile - 1) // tile) * tile
    kv_blocks = 0
    for q in range(len(offM) - 1):
        src = offM[q + 1] - offM[q]
        stream = sum(offN[p + 1] - offN[p] for p in range(P_N) if q in idx[p])
        kv_blocks += ((src + rows - 1) // rows) * rows * ((stream + tile - 1) // tile) * tile
    return pairs, q_blocks, kv_blocks


def test_executed_pair_and_block_counts():
    rng = np.random.default_rng(7)
    for P_N, P_M, s in ((5, 7, 3), (9, 4, 4), (1, 1, 1)):
        offN = np.concatenate([[0], np.cumsum(rng.integers(0, 300, P_N))]).astype(np.int32)
        offM = np.concatenate([[0], np.cumsum(rng.integers(0, 300, P_M))]).astype(np.int32)
        idx = np.stack([rng.permutation(P_M)[:s] for _ in range(P_N)]).astype(np.int32)
        pairs, qb, kvb = _loops(offN, offM, idx, 128, 64)
        assert bench.executed_pairs(offN, offM, idx) == pairs
        d, k = 128, 200
        flop, qb2, kvb2 = bench.executed_block_flops(offN, offM, idx, d, k)
        assert (qb2, kvb2) == (qb, kvb)
        assert flop == 2.0 * qb * (2 * d + k) + 2.0 * kvb * (2 * d + 2 * k)
        assert bench.algorithmic_flops(pairs, d, k) == 2.0 * pairs * (4 * d + 3 * k)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_step_stats_percentiles():
    # nearest-rank percentiles and the median of per-step times, against a
    # hand count: 10 values 1..10 -> p10 = 1, p90 = 9, median 5.5, mean 5.5
    st = bench.step_stats([7.0, 3.0, 10.0, 1.0, 5.0, 9.0, 2.0, 8.0, 4.0, 6.0])
    assert st == {"median": 5.5, "mean": 5.5, "p10": 1.0, "p90": 9.0, "n": 10}
    st = bench.step_stats([2.0, 1.0, 3.0])
    assert st["median"] == 2.0 and st["p10"] == 1.0 and st["p90"] == 3.0
