"""Seeded synthetic inputs for NSA selection attention (numpy only).

This module holds no arithmetic of the method: it only draws tensors and
block lists.  Both the oracle side and the HIP side take their inputs from
here, so a test can feed the same seeded draw to each.

What the draws follow:
  * page 1 of the reference text, "test_kernel_backward.py" (run_one): the
    tensor layout q, dO [B, Hq, T, D]; k, v [B, Hkv, T, D]; standard normal
    values; one seed; the draw order q, k, v, block_idx, dO.
  * the five workload shapes and block-list recipes of the benchmark
    definition (own block + random distinct earlier blocks, -1 padded; own
    block + first block + random earlier; dense causal; packed
    variable-length sequences).

Randomness: numpy PCG64 via ``numpy.random.default_rng(seed)``.  Values are
float32 normal draws; bfloat16 workloads round them to bfloat16 (round to
nearest even) and keep them as float32 arrays holding bf16-exact values.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "round_to_bf16",
    "block_idx_own_random",
    "block_idx_own_first_random",
    "block_idx_dense",
    "make_dense",
    "make_thd",
    "make_workload",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16, returned as float32 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _random_subsets(rng: np.random.Generator, n_rows: int, lo: int, hi: int, m: int) -> np.ndarray:
    """n_rows independent uniformly random m-subsets of [lo, hi), random order."""
    if m <= 0 or hi <= lo:
        return np.zeros((n_rows, 0), dtype=np.int32)
    keys = rng.random((n_rows, hi - lo))
    order = np.argsort(keys, axis=1, kind="stable")[:, :m]
    return (order + lo).astype(np.int32)


def block_idx_own_random(rng, n_heads: int, T: int, bs: int, S: int) -> np.ndarray:
    """[n_heads, T, S]: own block t//bs, then min(S-1, i) distinct random
    blocks from [0, i), then -1 padding."""
    out = np.full((n_heads, T, S), -1, dtype=np.int32)
    NB = -(-T // bs)
    for i in range(NB):
        t0, t1 = i * bs, min((i + 1) * bs, T)
        n = n_heads * (t1 - t0)
        m = min(S - 1, i)
        rows = np.full((n, S), -1, dtype=np.int32)
        rows[:, 0] = i
        rows[:, 1:1 + m] = _random_subsets(rng, n, 0, i, m)
        out[:, t0:t1, :] = rows.reshape(n_heads, t1 - t0, S)
    return out


def block_idx_own_first_random(rng, n_heads: int, T: int, bs: int, S: int) -> np.ndarray:
    """[n_heads, T, S]: own block i; for i > 0 also block 0 and min(S-2, i-1)
    distinct random blocks from [1, i); then -1 padding."""
    out = np.full((n_heads, T, S), -1, dtype=np.int32)
    NB = -(-T // bs)
    for i in range(NB):
        t0, t1 = i * bs, min((i + 1) * bs, T)
        n = n_heads * (t1 - t0)
        rows = np.full((n, S), -1, dtype=np.int32)
        rows[:, 0] = i
        if i > 0 and S > 1:
            rows[:, 1] = 0
            m = min(S - 2, i - 1)
            rows[:, 2:2 + m] = _random_subsets(rng, n, 1, i, m)
        out[:, t0:t1, :] = rows.reshape(n_heads, t1 - t0, S)
    return out


def block_idx_dense(n_heads: int, T: int, bs: int, S: int) -> np.ndarray:
    """[n_heads, T, S]: every block 0..i (i = t//bs), then -1 padding."""
    out = np.full((n_heads, T, S), -1, dtype=np.int32)
    t = np.arange(T)
    i = t // bs
    s = np.arange(S)
    row = np.where(s[None, :] <= i[:, None], s[None, :], -1).astype(np.int32)
    out[:] = row[None]
    return out


RECIPES = ("own_random", "own_first_random", "dense")


def _block_idx(rng, recipe: str, n_heads: int, T: int, bs: int, S: int) -> np.ndarray:
    if recipe == "own_random":
        return block_idx_own_random(rng, n_heads, T, bs, S)
    if recipe == "own_first_random":
        return block_idx_own_first_random(rng, n_heads, T, bs, S)
    if recipe == "dense":
        return block_idx_dense(n_heads, T, bs, S)
    raise ValueError(f"unknown block_idx recipe {recipe!r}")


@dataclasses.dataclass
class Workload:
    """One seeded draw.  Dense: q/dO [B,Hq,T,D], k/v [B,Hkv,Tk,D] (Tk >= T;
    the queries are the last T key positions), block_idx [B,Hkv,T,S].  Packed (cu_seqlens set): q/dO [Ttot,Hq,D],
    k/v [Ttot,Hkv,D], block_idx [Hkv,Ttot,S] with sequence-local indices."""
    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    S: int
    block_size: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_idx: np.ndarray
    dO: np.ndarray
    cu_seqlens: Optional[np.ndarray] = None
    max_seqlen: int = 0

    @property
    def scale(self) -> float:
        return float(self.D) ** -0.5

    @property
    def packed(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def n_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.packed else self.B


def _normal(rng, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def make_dense(B, Hq, Hkv, T, D, S, block_size, dtype="bf16", recipe="own_random",
               seed=0, name="dense", block_idx=None, Tk=None) -> Workload:
    """Dense [B,H,T,D] draw in the order q, k, v, block_idx, dO.  With Tk > T
    the keys are [B,Hkv,Tk,D] and the block lists are the recipe's lists of
    the last T of Tk positions."""
    rng = np.random.default_rng(seed)
    Tk = T if Tk is None else int(Tk)
    q = _normal(rng, (B, Hq, T, D), dtype)
    k = _normal(rng, (B, Hkv, Tk, D), dtype)
    v = _normal(rng, (B, Hkv, Tk, D), dtype)
    if block_idx is None:
        idx = np.stack([_block_idx(rng, recipe, Hkv, Tk, block_size, S)[:, Tk - T:]
                        for _ in range(B)])
        idx = np.ascontiguousarray(idx)
    else:
        idx = np.ascontiguousarray(block_idx, dtype=np.int32)
    dO = _normal(rng, (B, Hq, T, D), dtype)
    return Workload(name, dtype, B, Hq, Hkv, T, D, S, block_size, q, k, v, idx, dO)


def make_thd(lengths: List[int], Hq, Hkv, D, S, block_size, dtype="bf16",
             recipe="own_first_random", seed=0, name="thd", rng=None) -> Workload:
    """Packed draw: sequences concatenated along tokens; block lists are
    sequence-local.  Draw order q, k, v, block_idx (per sequence), dO."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    Ttot = int(cu[-1])
    q = _normal(rng, (Ttot, Hq, D), dtype)
    k = _normal(rng, (Ttot, Hkv, D), dtype)
    v = _normal(rng, (Ttot, Hkv, D), dtype)
    idx = np.full((Hkv, Ttot, S), -1, dtype=np.int32)
    for z, L in enumerate(lengths):
        idx[:, cu[z]:cu[z + 1], :] = _block_idx(rng, recipe, Hkv, L, block_size, S)
    dO = _normal(rng, (Ttot, Hq, D), dtype)
    return Workload(name, dtype, 1, Hq, Hkv, Ttot, D, S, block_size, q, k, v, idx, dO,
                    cu_seqlens=cu, max_seqlen=max(lengths) if lengths else 0)


# The five benchmark workloads, named by what they are: shape description.
WORKLOADS = {
    "f32_T256": "B1 Hq2 Hkv1 D32 T256 bs16 S4 f32, own block + random earlier",
    "bf16_T1024": "B2 Hq6 Hkv2 D64 T1024 bs32 S8 bf16, own block + random earlier",
    "select_T8192": "B1 Hq32 Hkv2 D128 T8192 bs64 S16 bf16, own + first + random earlier",
    "causal_B4_T4096": "B4 Hq32 Hkv8 D128 T4096 bs64 S64 bf16, dense causal",
    "packed_8seq": "THD 8 seqs len 64*U{2..64} Hq32 Hkv8 D128 bs64 S16 bf16, own + first + random",
}


def make_workload(name: str, seed: int = 0) -> Workload:
    if name == "f32_T256":
        return make_dense(1, 2, 1, 256, 32, 4, 16, "f32", "own_random", seed, name)
    if name == "bf16_T1024":
        return make_dense(2, 6, 2, 1024, 64, 8, 32, "bf16", "own_random", seed, name)
    if name == "select_T8192":
        return make_dense(1, 32, 2, 8192, 128, 16, 64, "bf16", "own_first_random", seed, name)
    if name == "causal_B4_T4096":
        return make_dense(4, 32, 8, 4096, 128, 64, 64, "bf16", "dense", seed, name)
    if name == "packed_8seq":
        rng = np.random.default_rng(seed)
        lengths = (64 * rng.integers(2, 65, size=8)).tolist()
        return make_thd(lengths, 32, 8, 128, 16, 64, "bf16", "own_first_random",
                        name=name, rng=rng)
    raise ValueError(f"unknown workload {name!r}")
