"""GPU parity for dense problems with more keys than queries (Tk > T): the
queries are the last T key positions, query t attends keys j <= t + Tk - T
of its listed blocks (bottom-right causal alignment, one of the backward
flavours page 3 of the reference text lists).  Every output element against
the float64 oracle at page 1's gates, on the bf16 kernels (query walks with
counters and with a barrier per job, the dS hand-off and the recomputing
dQ, 16- to 128-key blocks), the f32 kernels, a sliding window, a single
decoding query, and the inversion bit-exact."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads
from _harness import TOL, assert_close, say, to_dev
from test_gpu_parity import _full_parity, _weird_block_idx
from test_gpu_window import _check as window_check

pytestmark = pytest.mark.gpu


def _br(name, B, Hq, Hkv, T, Tk, D, S, bs, dtype="bf16", recipe="own_first_random", weird=False,
        seed=91):
    idx = None
    if weird:
        rng = np.random.default_rng(seed + 100)
        full = _weird_block_idx(rng, B, Hkv, Tk, bs, S)
        idx = np.ascontiguousarray(full[:, :, Tk - T:])
    return workloads.make_dense(B, Hq, Hkv, T, D, S, bs, dtype, recipe, seed=seed, name=name,
                                block_idx=idx, Tk=Tk)


@pytest.mark.parametrize("case", [
    dict(name="br-G1-D64-bs64", B=2, Hq=2, Hkv=2, T=100, Tk=333, D=64, S=5, bs=64, weird=True),
    dict(name="br-G4-D128-bs32", B=1, Hq=8, Hkv=2, T=77, Tk=300, D=128, S=6, bs=32, weird=True),
    dict(name="br-G16-D128-bs64-handoff", B=1, Hq=32, Hkv=2, T=256, Tk=1000, D=128, S=8, bs=64),
    dict(name="br-G3-D64-bs128", B=1, Hq=6, Hkv=2, T=130, Tk=520, D=64, S=3, bs=128, weird=True),
    dict(name="br-G8-D32-bs16", B=1, Hq=16, Hkv=2, T=64, Tk=200, D=32, S=7, bs=16),
    dict(name="br-T-equals-Tk", B=1, Hq=8, Hkv=2, T=200, Tk=200, D=64, S=4, bs=32, weird=True),
])
def test_bottom_right_bf16(case):
    c = dict(case)
    w = _br(c.pop("name"), **c)
    _full_parity(w)


def test_bottom_right_decoding_query():
    """One query at the end of 1024 keys (16 heads per KV head, 8 blocks of 16:
    the hand-off path) and of 999 keys (4 heads, lists that can cover the
    whole prefix: the recomputing dQ)."""
    for Hq, Tk, S, handoff in ((32, 1024, 8, True), (8, 999, 16, False)):
        w = _br(f"br-decode-{Hq}", 2, Hq, 2, 1, Tk, 128, S, 64, seed=92)
        d = to_dev(w)
        p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale)
        assert nsa.ds_handoff(p) == handoff
        _full_parity(w)


def test_bottom_right_dense_lists():
    """Every query lists every block up to its position (selections that
    cover whole prefixes: the query walk with a barrier per job; blocks are
    not paired when queries and keys do not align)."""
    B, Hq, Hkv, T, Tk, D, bs = 1, 8, 2, 150, 400, 128, 64
    NB = -(-Tk // bs)
    full = workloads.block_idx_dense(Hkv, Tk, bs, NB)
    idx = np.ascontiguousarray(np.broadcast_to(full[None, :, Tk - T:], (B, Hkv, T, NB)))
    w = workloads.make_dense(B, Hq, Hkv, T, D, NB, bs, "bf16", seed=93, name="br-dense",
                             block_idx=idx, Tk=Tk)
    _full_parity(w)


def test_bottom_right_f32():
    w = _br("br-f32", 2, 4, 2, 50, 130, 32, 4, 16, dtype="f32", weird=True, seed=94)
    _full_parity(w)


def test_bottom_right_window():
    w = _br("br-window", 1, 8, 2, 120, 400, 64, 6, 32, weird=True, seed=95)
    for W in (17, 90):
        window_check(w, W)


@pytest.mark.parametrize("window", [0, 40])
def test_bottom_right_inversion_bit_exact(window):
    B, Hkv, T, Tk, bs, S = 2, 2, 90, 260, 32, 5
    w = _br("br-invert", B, 4, Hkv, T, Tk, 64, S, bs, weird=True, seed=96)
    d = to_dev(w)
    offsets, tokens = nsa.nsa_sel_invert(d["q"], d["k"], d["idx"], bs, window=window)
    torch.cuda.synchronize()
    offsets, tokens = offsets.cpu().numpy(), tokens.cpu().numpy()
    NB = -(-Tk // bs)
    Smin = min(S, NB)
    counts, ref = oracle.invert(w.block_idx, bs, window, Tk=Tk)
    pos = 0
    for z in range(B):
        for hkv in range(Hkv):
            off = offsets[z, hkv]
            base = Smin * (z * Hkv + hkv) * T
            for u in range(NB):
                c = int(counts[z, hkv, u])
                assert off[u + 1] - off[u] == c, (z, hkv, u)
                np.testing.assert_array_equal(tokens[base + off[u]: base + off[u + 1]], ref[pos:pos + c])
                pos += c
    say(f"[br-invert] window {window}: {pos} entries bit-exact")
