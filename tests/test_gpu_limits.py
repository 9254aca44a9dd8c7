"""GPU parity at the edges of what the library accepts: the longest sequence
whose block count still fits the forward / dQ kernels' LDS, and the largest
number of (batch entry, KV head) groups (8192), on both dK/dV paths.  The
limits are found from the library's own host-side validation (no GPU call)
and checked to be the limits (one more block or group is refused); outputs
are then compared with the oracle on sampled rows and key blocks, plus the
sum invariants over every key."""
import numpy as np
import pytest

import workloads
from block_sparse_attention_nsa_amd import _lib
from _harness import run_gpu, say, to_dev
from test_gpu_parity import _invariants, _sampled_parity

pytestmark = pytest.mark.gpu


def _problem(**kw):
    p = _lib.Problem()
    base = dict(layout=0, B=1, T=256, Hq=2, Hkv=1, D=128, S=8, block_size=64, n_seqs=0,
                max_seqlen=0, dtype=1, scale=128 ** -0.5, window=0)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def _accepted(**kw) -> bool:
    n = _lib.load().nsa_sel_bwd_workspace_bytes(_problem(**kw))
    return n > 0 and _lib.last_error() == ""


def _own_first_random(rng, T, bs, S):
    """[Hkv=1, T, S] lists: own block i, block 0, and S - 2 random blocks of
    [1, i) (repeats possible: a block listed twice counts once on both sides),
    -1 where i is too small to have them."""
    i = np.arange(T) // bs
    idx = np.full((T, S), -1, dtype=np.int64)
    idx[:, 0] = i
    idx[:, 1] = np.where(i > 0, 0, -1)
    r = 1 + np.floor(rng.random((T, S - 2)) * np.maximum(i - 1, 1)[:, None]).astype(np.int64)
    idx[:, 2:] = np.where((i > 1)[:, None], r, -1)
    return idx.astype(np.int32)[None, None]


def test_longest_sequence():
    """T at the forward / dQ LDS limit (bf16, D 128, block 64), ragged tail:
    block masks and union of 3268 blocks per workgroup, a 418k-row list for
    block 0 split into many fp32 partials (block 0 is among the key blocks
    compared with the oracle)."""
    lo, hi = 64, 1 << 22
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if _accepted(T=mid):
            lo = mid
        else:
            hi = mid
    NB = -(-lo // 64)
    assert not _accepted(T=NB * 64 + 1) and "LDS" in _lib.last_error()
    T = lo - 5
    rng = np.random.default_rng(21)
    idx = _own_first_random(rng, T, 64, 8)
    w = workloads.make_dense(1, 2, 1, T, 128, 8, 64, "bf16", seed=22, name=f"longest-T{T}",
                             block_idx=idx)
    say(f"[{w.name}] NB={NB} (limit), B=1 Hq=2 Hkv=1 D=128 S=8")
    d = to_dev(w)
    out = run_gpu(w, d)
    for key in out:
        assert np.isfinite(out[key][~np.isinf(out[key])]).all(), key
    _sampled_parity(w, out, np.random.default_rng(23), blocks=[(0, 0, 0), (0, 0, 1), (0, 0, NB // 2), (0, 0, NB - 1)])
    _invariants(w, out, d)


@pytest.mark.parametrize("lists", ["own_random", "whole_prefix"])
def test_most_groups(lists):
    """8192 (batch entry, KV head) groups: per-group prefixes and the dK/dV
    plan over all of them (the last scan workgroup's pass), with lists that
    take the per-block dK/dV path and with whole causal prefixes (the paired
    path, 8192 pair items)."""
    B, Hq, Hkv, T, D, bs = 4096, 4, 2, 40, 64, 32
    assert _accepted(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, S=2, block_size=bs)
    assert not _accepted(B=B + 1, Hq=Hq, Hkv=Hkv, T=T, D=D, S=2, block_size=bs)
    assert "exceeds 8192" in _lib.last_error()
    if lists == "whole_prefix":
        t = np.arange(T)
        row = np.where(np.arange(2)[None, :] <= (t // bs)[:, None], np.arange(2)[None, :], -1)
        idx = np.broadcast_to(row, (B, Hkv, T, 2)).astype(np.int32).copy()
        w = workloads.make_dense(B, Hq, Hkv, T, D, 2, bs, "bf16", seed=24, name="groups-prefix",
                                 block_idx=idx)
    else:
        w = workloads.make_dense(B, Hq, Hkv, T, D, 2, bs, "bf16", "own_random", seed=25,
                                 name="groups-random")
    say(f"[{w.name}] ZH={B * Hkv} B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} bs={bs}")
    d = to_dev(w)
    out = run_gpu(w, d)
    _sampled_parity(w, out, np.random.default_rng(26),
                    blocks=[(0, 0, 0), (B - 1, Hkv - 1, 1), (B // 2, 1, 0), (B - 1, 0, 0)])
    _invariants(w, out, d)
