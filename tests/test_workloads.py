"""Properties of the seeded input generators (CPU)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000, dtype=np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]  # exact ties and an exact value
    ours = workloads.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref)


def _check_rows(idx, T, bs, S, first_block):
    NB = -(-T // bs)
    for t in range(T):
        i = t // bs
        for h in range(idx.shape[0]):
            row = idx[h, t]
            valid = row[row >= 0]
            assert len(set(valid.tolist())) == len(valid)  # distinct
            assert i in valid                               # own block listed
            assert np.all(valid <= i) and np.all(valid < NB)
            n_expect = min(S, i + 1)
            assert len(valid) == n_expect
            assert np.all(row[n_expect:] == -1)             # -1 exactly past the valid count
            if first_block and i > 0:
                assert 0 in valid


def test_own_random_recipe():
    rng = np.random.default_rng(1)
    idx = workloads.block_idx_own_random(rng, 2, 200, 16, 4)
    _check_rows(idx, 200, 16, 4, False)


def test_own_first_random_recipe():
    rng = np.random.default_rng(2)
    idx = workloads.block_idx_own_first_random(rng, 2, 640, 32, 6)
    _check_rows(idx, 640, 32, 6, True)


def test_dense_recipe():
    idx = workloads.block_idx_dense(1, 300, 64, 5)
    _check_rows(idx, 300, 64, 5, True)


def test_workloads_reproducible_and_shaped():
    a = workloads.make_workload("f32_T256", seed=0)
    b = workloads.make_workload("f32_T256", seed=0)
    c = workloads.make_workload("f32_T256", seed=1)
    for x, y in ((a.q, b.q), (a.block_idx, b.block_idx), (a.dO, b.dO)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (1, 2, 256, 32) and a.block_idx.shape == (1, 1, 256, 4)
    assert a.q.dtype == np.float32
    w1 = workloads.make_workload("bf16_T1024")
    assert w1.q.shape == (2, 6, 1024, 64) and w1.block_idx.shape == (2, 2, 1024, 8)
    np.testing.assert_array_equal(workloads.round_to_bf16(w1.q), w1.q)


def test_thd_workload_lengths():
    w = workloads.make_workload("packed_8seq", seed=0)
    lens = np.diff(w.cu_seqlens)
    assert len(lens) == 8 and np.all(lens % 64 == 0)
    assert np.all((lens >= 128) & (lens <= 4096))
    assert w.q.shape == (w.cu_seqlens[-1], 32, 128) and w.block_idx.shape == (8, w.cu_seqlens[-1], 16)
    for z in range(8):
        a, b = w.cu_seqlens[z], w.cu_seqlens[z + 1]
        _check_rows(w.block_idx[:, a:b], b - a, 64, 16, True)
