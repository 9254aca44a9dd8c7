"""GPU parity of the sliding-window mask (problem.window = W > 0: keys
t - W < j <= t on top of the block selection) against the float64 oracle,
page 1's max-abs gates (2e-3 fp32, 6e-2 bf16)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads
from _harness import TOL, assert_close, say, to_dev
from test_gpu_parity import _weird_block_idx

pytestmark = pytest.mark.gpu


def _run(w, W, d=None):
    d = d or to_dev(w)
    ms = w.max_seqlen if w.packed else None
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, d["cu"], ms,
                             window=W)
    dq, dk, dv = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                                 w.scale, d["cu"], ms, window=W)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    return dict(o=f(o), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv))


def _oracle(w, W):
    if w.packed:
        o, lse = oracle.fwd_thd(w.q, w.k, w.v, w.block_idx, w.cu_seqlens, w.block_size, w.scale,
                                window=W)
        dq, dk, dv, _, _ = oracle.bwd_thd(w.q, w.k, w.v, w.dO, w.block_idx, w.cu_seqlens,
                                          w.block_size, w.scale, window=W)
    else:
        o, lse = oracle.fwd(w.q, w.k, w.v, w.block_idx, w.block_size, w.scale, window=W)
        dq, dk, dv, _, _ = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, w.block_size, w.scale,
                                      window=W)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def _check(w, W):
    say(f"[{w.name}] window {W}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"bs={w.block_size} S={w.S} packed={w.packed}")
    got, ref = _run(w, W), _oracle(w, W)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, got[name], ref[name], TOL[w.dtype])


@pytest.mark.parametrize("case", [
    dict(name="win-G4-D128-bs64", B=1, Hq=8, Hkv=2, T=333, D=128, S=5, bs=64, W=(1, 37, 150)),
    dict(name="win-G16-D64-bs32", B=1, Hq=16, Hkv=1, T=200, D=64, S=4, bs=32, W=(20,)),
    dict(name="win-prefix-G2-D128-bs64", B=1, Hq=4, Hkv=2, T=300, D=128, S=5, bs=64, W=(70,)),
])
def test_bf16_window_irregular_lists(case):
    """bf16 with irregular lists (the last case can cover whole prefixes:
    the barrier walk in forward and dQ), windows narrower than a block, about
    half a block and wider than two blocks."""
    rng = np.random.default_rng(51)
    c = dict(case)
    name, Ws = c.pop("name"), c.pop("W")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], c["bs"], c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=52, name=name, block_idx=idx)
    for W in Ws:
        _check(w, W)


def test_f32_window_packed():
    w = workloads.make_thd([60, 0, 130, 9], 4, 2, 32, 3, 16, "f32", "own_random", seed=53,
                           name="win-f32-packed")
    for W in (5, 40):
        _check(w, W)


def test_window_wider_than_sequence_is_bitwise_no_window():
    """W >= T takes the windowed kernels but masks nothing: the same bits as
    the no-window kernels (NSA lists, then whole-prefix lists)."""
    for recipe in ("own_first_random", "dense"):
        w = workloads.make_dense(1, 8, 2, 256, 64, 4 if recipe != "dense" else 8, 32, "bf16",
                                 recipe=recipe, seed=54, name=f"win-wide-{recipe}")
        d = to_dev(w)
        a, b = _run(w, 0, d), _run(w, w.T, d)
        for n in a:
            assert np.array_equal(a[n], b[n]), (recipe, n)


def test_window_with_sink():
    """A sliding window and attention-sink logits together (bf16, irregular
    lists): o, lse, dq, dk, dv and dsink against the oracle."""
    import math
    rng = np.random.default_rng(55)
    B, Hq, Hkv, T, D, S, bs, W = 1, 8, 2, 260, 64, 5, 32, 45
    idx = _weird_block_idx(rng, B, Hkv, T, bs, S)
    w = workloads.make_dense(B, Hq, Hkv, T, D, S, bs, "bf16", seed=56, name="win-sink",
                             block_idx=idx)
    sink_np = rng.normal(0.5, 1.5, size=Hq).astype(np.float32)
    d = to_dev(w)
    sink = torch.from_numpy(sink_np).cuda()
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], bs, w.scale, sink=sink, window=W)
    dq, dk, dv, ds = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], bs, w.scale,
                                     sink=sink, window=W)
    torch.cuda.synchronize()
    sk = sink_np.astype(np.float64)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.block_idx, bs, w.scale, sink=sk, window=W)
    rdq, rdk, rdv, lse64, delta64 = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, bs, w.scale,
                                               sink=sk, window=W)
    rds = oracle.dsink(sk, lse64, delta64, head_axis=1)
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    tol = TOL["bf16"]
    for name, a, b in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk),
                       ("dv", dv, rdv)):
        assert_close(name, f(a), b, tol)
    assert_close("dsink", f(ds), rds, tol * math.sqrt(T))
