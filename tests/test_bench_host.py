"""Host-side pieces of bench.py (no GPU): its useful-pair count N agrees with
the oracle's, and it refuses more than one GPU."""
import subprocess
import sys

import numpy as np

import bench
import oracle
import workloads
from test_oracle_pins import _weird_idx


def test_useful_pairs_matches_oracle_dense():
    rng = np.random.default_rng(4)
    idx = _weird_idx(rng, 2, 3, 97, 8, 5)
    w = workloads.make_dense(2, 6, 3, 97, 16, 5, 8, "f32", block_idx=idx)
    n = bench.useful_pairs(w.block_idx, 2, 8, bench.row_groups(w))
    assert n == oracle.count_pairs(idx, 6, 8)


def test_useful_pairs_matches_oracle_packed():
    w = workloads.make_thd([30, 0, 64, 7], 8, 2, 16, 4, 8, "f32", "own_first_random", seed=2)
    n = bench.useful_pairs(w.block_idx, 4, 8, bench.row_groups(w))
    assert n == oracle.count_pairs_thd(w.block_idx, w.cu_seqlens, 8, 8)


def test_workload_pair_counts():
    """Exact N of the small workloads (fp32 T 256, bf16 T 1024, NSA lists T
    8192), and of the dense causal 4 x 4096 workload as a closed form."""
    for name in ("f32_T256", "bf16_T1024", "select_T8192"):
        w = workloads.make_workload(name)
        G = w.Hq // w.Hkv
        n = bench.useful_pairs(w.block_idx, G, w.block_size, bench.row_groups(w))
        assert n == oracle.count_pairs(w.block_idx, w.Hq, w.block_size)
    w = workloads.make_workload("causal_B4_T4096")
    n = bench.useful_pairs(w.block_idx, 4, 64, bench.row_groups(w))
    assert n == 4 * 32 * 4096 * 4097 // 2


def test_refuses_several_gpus():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_window_pair_counts_brute_force():
    """With a sliding window the useful pairs are the selected keys j with
    t - W < j <= t, counted row by row here."""
    import numpy as np

    w = workloads.make_dense(1, 4, 2, 150, 32, 5, 16, "f32", seed=3)
    G, bs = 2, 16
    for W in (1, 9, 40, 500):
        n = bench.useful_pairs(w.block_idx, G, bs, ((w.block_idx[0, h], 150) for h in range(2)), W)
        brute = 0
        for h in range(2):
            for t in range(150):
                sel = {u for u in w.block_idx[0, h, t].tolist() if 0 <= u < 10 and u * bs <= t}
                brute += sum(1 for u in sel for j in range(u * bs, min((u + 1) * bs, t + 1))
                             if j > t - W)
        assert n == brute * G, (W, n, brute * G)
