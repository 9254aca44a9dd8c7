"""GPU parity for bf16 with 16-key blocks (page 1's gate runs its config
matrix over block sizes; 16 is the smallest the workloads use).  The
matrix-core kernels contract 32 keys at a time, so a 16-key block is walked
as a 32-key job with its upper half masked, and dK/dV runs on a 32-key tile
whose upper 16 keys are neither computed into the block nor written.  Every
output element is compared with the float64 oracle (6e-2 max-abs)."""
import numpy as np
import pytest

import workloads
from _harness import run_gpu
from test_gpu_parity import _full_parity, _weird_block_idx
from test_gpu_window import _check as window_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", [
    dict(name="bs16-G2-D32", B=1, Hq=2, Hkv=1, T=256, D=32, S=4),   # the f32 T 256 shape
    dict(name="bs16-G4-D128-ragged", B=2, Hq=8, Hkv=2, T=333, D=128, S=6),
    dict(name="bs16-G16-D64", B=1, Hq=16, Hkv=1, T=250, D=64, S=5),
    dict(name="bs16-G3-D64-S>NB", B=1, Hq=6, Hkv=2, T=90, D=64, S=9),
])
def test_block16_irregular_lists(case):
    rng = np.random.default_rng(71)
    c = dict(case)
    name = c.pop("name")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], 16, c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], 16, "bf16",
                             seed=72, name=name, block_idx=idx)
    _full_parity(w)


def test_block16_split_lists():
    """Lists longer than one dK/dV work item (fp32 partials and the ordered
    reduce on the 32-key slot layout)."""
    w = workloads.make_dense(1, 8, 2, 2048, 64, 8, 16, "bf16", "own_first_random", seed=73,
                             name="bs16-split")
    _full_parity(w)


def test_block16_whole_prefix_pairs():
    """Every row lists its whole causal prefix: dK/dV runs on pairs of
    16-key blocks (an odd block count leaves the last pair half empty)."""
    B, Hq, Hkv, T, D, bs = 2, 8, 2, 200, 128, 16
    NB = -(-T // bs)
    idx = np.broadcast_to(workloads.block_idx_dense(Hkv, T, bs, NB)[None], (B, Hkv, T, NB)).copy()
    w = workloads.make_dense(B, Hq, Hkv, T, D, NB, bs, "bf16", seed=74, name="bs16-prefix",
                             block_idx=idx)
    _full_parity(w)


def test_block16_packed_and_window():
    """Packed sequences (one empty), then the same with sliding windows of 5
    and 40 keys (inside one block, across blocks)."""
    w = workloads.make_thd([130, 0, 47, 260], 8, 2, 64, 6, 16, "bf16", "own_first_random",
                           seed=75, name="bs16-packed")
    _full_parity(w)
    for W in (5, 40):
        window_check(w, W)


def test_block16_block_boundaries_bitwise():
    """Keys of block u + 1 never leak into block u's 32-key job: changing K/V
    of a block nobody lists leaves every output bitwise unchanged, and that
    block's dk/dv are exactly zero."""
    B, Hq, Hkv, T, D, bs, S = 1, 4, 1, 128, 64, 16, 3
    idx = np.full((B, Hkv, T, S), -1, np.int32)
    idx[0, 0, :, 0] = np.arange(T) // bs            # own block
    idx[0, 0, 64:, 1] = 2                            # tokens 64.. list block 2 (keys 32..47)
    # block 3 (keys 48..63) is listed only by its own tokens 48..63
    w = workloads.make_dense(B, Hq, Hkv, T, D, S, bs, "bf16", seed=76, block_idx=idx,
                             name="bs16-sentinel")
    base = run_gpu(w)
    idx2 = idx.copy()
    idx2[0, 0, 48:64, 0] = -1                        # now nobody lists block 3
    w2 = workloads.make_dense(B, Hq, Hkv, T, D, S, bs, "bf16", seed=76, block_idx=idx2,
                              name="bs16-sentinel2")
    a = run_gpu(w2)
    w2.k[0, 0, 48:64] += 1.5
    w2.v[0, 0, 48:64] -= 2.0
    b = run_gpu(w2)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[name], b[name]), name
    assert np.all(a["dk"][0, 0, 48:64] == 0.0) and np.all(a["dv"][0, 0, 48:64] == 0.0)
    # tokens outside 48..63 are unaffected by dropping block 3's own listing
    for name in ("o", "lse", "dq"):
        keep = np.r_[0:48, 64:T]
        assert np.array_equal(base[name][0, :, keep], a[name][0, :, keep]), name
