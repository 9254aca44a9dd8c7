"""GPU parity on strided tensors: the library takes per-tensor (batch entry,
head, token) strides (page 3's backward honours the output strides its
caller declares).  Each case runs the same seeded draw once contiguous and
once through strided views -- inputs as [B, T, H, D] buffers viewed as
[B, H, T, D], outputs written into slices of wider buffers -- and checks
that o, lse, dq, dk, dv are bitwise the same (the arithmetic does not depend
on the layout), that the strided results match the float64 oracle, and that
no element outside the output views was written."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import workloads
from _harness import TOL, assert_close, oracle_full, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 7.0  # bf16- and fp32-exact, never produced by these problems' outputs


def _wide(shape, dtype, dev, pad_last=True):
    """A sentinel-filled buffer whose last dimension is twice D; the view
    [..., :D] is a strided tensor with a contiguous last dimension."""
    shp = tuple(shape[:-1]) + (2 * shape[-1] if pad_last else shape[-1],)
    return torch.full(shp, SENTINEL, dtype=dtype, device=dev)


def _run_strided(w):
    dev = torch.device("cuda")
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    D = w.D
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    if w.packed:
        # [T, H, D] views of [T, H, 2D] buffers: head stride 2 D, token stride 2 H D
        def inp(x):
            buf = _wide(x.shape, dt, dev)
            buf[..., :D] = up(x)
            return buf[..., :D]
        q, k, v, dO = (inp(x) for x in (w.q, w.k, w.v, w.dO))
        o_buf = _wide(w.q.shape, dt, dev)
        dq_buf = _wide(w.q.shape, dt, dev)
        dk_buf = _wide(w.k.shape, dt, dev)
        dv_buf = torch.full((w.k.shape[1], w.k.shape[0], D), SENTINEL, dtype=dt, device=dev)
        o, dq, dk = o_buf[..., :D], dq_buf[..., :D], dk_buf[..., :D]
        dv = dv_buf.transpose(0, 1)                      # [T, Hkv, D] view of [Hkv, T, D]
        cu = torch.from_numpy(w.cu_seqlens).to(dev)
        ms = w.max_seqlen
    else:
        # [B, T, H, D] buffers viewed as [B, H, T, D]
        bthd = lambda x: up(np.ascontiguousarray(np.asarray(x).transpose(0, 2, 1, 3))).transpose(1, 2)
        q, k, v, dO = (bthd(x) for x in (w.q, w.k, w.v, w.dO))
        o_buf = torch.full((w.B, w.T, w.Hq, D), SENTINEL, dtype=dt, device=dev)
        o = o_buf.transpose(1, 2)
        dq_buf = _wide(w.q.shape, dt, dev)
        dk_buf = torch.full((w.B, w.T, w.Hkv, 2 * D), SENTINEL, dtype=dt, device=dev)
        dv_buf = _wide(w.k.shape, dt, dev)
        dq = dq_buf[..., :D]
        dk = dk_buf[..., D:].transpose(1, 2)
        dv = dv_buf[..., D:]
        cu, ms = None, None
    # (a one-head tensor viewed through a size-1 transpose is still contiguous)
    for t in (q, dO, o, dq, dk, dv):
        assert not t.is_contiguous()
    idx = torch.from_numpy(np.ascontiguousarray(w.block_idx, dtype=np.int32)).to(dev)
    o_, lse = nsa.nsa_sel_fwd(q, k, v, idx, w.block_size, w.scale, cu, ms, out=o)
    assert o_ is o
    nsa.nsa_sel_bwd(q, k, v, o, lse, dO, idx, w.block_size, w.scale, cu, ms, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    got = dict(o=f(o), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv))
    # nothing outside the views was written
    for name, buf, view in (("o", o_buf, o), ("dq", dq_buf, dq), ("dk", dk_buf, dk),
                            ("dv", dv_buf, dv)):
        mask = torch.ones_like(buf, dtype=torch.bool)
        mask_view = mask.as_strided(view.shape, view.stride(), view.storage_offset() - buf.storage_offset())
        mask_view.fill_(False)
        outside = buf[mask]
        assert outside.numel() == 0 or bool((outside == SENTINEL).all()), f"{name}: wrote outside its view"
    return got


def _check(w):
    say(f"[{w.name}] strided views: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"bs={w.block_size} packed={w.packed}")
    base = run_gpu(w)
    got = _run_strided(w)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(got[name], base[name]), f"{name} differs from the contiguous run"
    ref = oracle_full(w)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, got[name], ref[name], TOL[w.dtype])


@pytest.mark.parametrize("case", [
    dict(name="str-G4-D128-bs64", B=2, Hq=8, Hkv=2, T=333, D=128, S=5, bs=64, dtype="bf16"),
    dict(name="str-G16-D64-bs32", B=1, Hq=16, Hkv=1, T=200, D=64, S=4, bs=32, dtype="bf16"),
    dict(name="str-G2-D32-f32", B=2, Hq=4, Hkv=2, T=150, D=32, S=4, bs=16, dtype="f32"),
])
def test_dense_strided_views(case):
    c = dict(case)
    name, dtype = c.pop("name"), c.pop("dtype")
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], dtype,
                             "own_first_random", seed=51, name=name)
    _check(w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_strided_views(dtype):
    w = workloads.make_thd([100, 0, 257, 64], 8, 2, 64 if dtype == "bf16" else 32, 6, 32, dtype,
                           "own_first_random", seed=52, name=f"str-packed-{dtype}")
    _check(w)


def test_whole_prefix_strided():
    """Dense causal lists (the paired dK/dV path and the barrier walks) on
    strided views."""
    B, Hq, Hkv, T, D, bs = 2, 8, 2, 256, 128, 64
    NB = T // bs
    idx = np.broadcast_to(workloads.block_idx_dense(Hkv, T, bs, NB)[None], (B, Hkv, T, NB)).copy()
    w = workloads.make_dense(B, Hq, Hkv, T, D, NB, bs, "bf16", seed=53, name="str-prefix",
                             block_idx=idx)
    _check(w)


def test_kv_shared_across_batch_with_zero_stride():
    """k and v given once and expanded over the batch (batch stride 0): the
    same results as the contiguous repeated tensors."""
    B, Hq, Hkv, T, D, bs, S = 3, 8, 2, 200, 64, 32, 4
    w = workloads.make_dense(B, Hq, Hkv, T, D, S, bs, "bf16", "own_random", seed=54, name="kv0")
    w.k[:] = w.k[0:1]
    w.v[:] = w.v[0:1]
    base = run_gpu(w)
    d = to_dev(w)
    k0 = d["k"][0:1].expand(B, -1, -1, -1)
    v0 = d["v"][0:1].expand(B, -1, -1, -1)
    assert k0.stride(0) == 0
    o, lse = nsa.nsa_sel_fwd(d["q"], k0, v0, d["idx"], bs, w.scale)
    dq, dk, dv = nsa.nsa_sel_bwd(d["q"], k0, v0, o, lse, d["dO"], d["idx"], bs, w.scale)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    for name, a in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(f(a), base[name]), name
