"""GPU parity of the attention-sink extension (nsa_sel_fwd_sink,
nsa_sel_bwd with the sink-inclusive lse, nsa_sel_bwd_dsink) against the
float64 oracle on the same seeded inputs.

o, lse, dq, dk, dv use page 1's max-abs gates (2e-3 fp32, 6e-2 bf16).
The pages fix no gate for dsink[h], a sum of one term P_sink * Delta per row
of head h: each head is gated by the bound the GPU's own arithmetic implies
(_harness.dsink_bound: Delta from the o the GPU produced, P_sink from its lse,
fp32 rounding of both and of the sum), with 25 % slack."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads
from _harness import TOL, assert_close, dsink_bound, say, to_dev
from test_gpu_parity import _weird_block_idx

pytestmark = pytest.mark.gpu


def _sink_vals(rng, Hq, loc=0.5):
    return rng.normal(loc, 1.5, size=Hq).astype(np.float32)


def _run(w, d, sink_np):
    sink = torch.from_numpy(sink_np).to(d["q"].device)
    ms = w.max_seqlen if w.packed else None
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, d["cu"], ms,
                             sink=sink)
    dq, dk, dv, dsink = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"],
                                        w.block_size, w.scale, d["cu"], ms, sink=sink)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    return dict(o=f(o), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv), dsink=f(dsink))


def _oracle(w, sink_np):
    sk = sink_np.astype(np.float64)
    if w.packed:
        dq, dk, dv, lse, delta = oracle.bwd_thd(w.q, w.k, w.v, w.dO, w.block_idx, w.cu_seqlens,
                                                w.block_size, w.scale, sink=sk)
        o, lse_f = oracle.fwd_thd(w.q, w.k, w.v, w.block_idx, w.cu_seqlens, w.block_size, w.scale,
                                  sink=sk)
        # rows of no sequence (none here) would be left at 0; every token belongs to one
        ds = oracle.dsink(sk, lse, delta, head_axis=0)
    else:
        dq, dk, dv, lse, delta = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, w.block_size,
                                            w.scale, sink=sk)
        o, lse_f = oracle.fwd(w.q, w.k, w.v, w.block_idx, w.block_size, w.scale, sink=sk)
        ds = oracle.dsink(sk, lse, delta, head_axis=1)
    return dict(o=o, lse=lse_f, dq=dq, dk=dk, dv=dv, dsink=ds, lse_b=lse, delta=delta)


def _check(w, sink_np):
    tol = TOL[w.dtype]
    say(f"[{w.name}] sink parity: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"bs={w.block_size} packed={w.packed}")
    got = _run(w, to_dev(w), sink_np)
    ref = _oracle(w, sink_np)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, got[name], ref[name], tol)
    bound = dsink_bound(w, got, ref, sink_np, ref["lse_b"], ref["delta"])
    err = np.abs(got["dsink"] - ref["dsink"])
    say(f"  dsink: max|err| = {err.max():.3e}, per-head bound {bound.min():.3e}..{bound.max():.3e}, "
        f"max|dsink| = {np.abs(ref['dsink']).max():.3g}")
    assert np.all(err <= 1.25 * bound + 1e-6), (err, bound)
    return got, ref


@pytest.mark.parametrize("case", [
    dict(name="sink-G4-D128-bs64", B=1, Hq=8, Hkv=2, T=333, D=128, S=5, bs=64),
    dict(name="sink-G16-D64-bs32", B=1, Hq=16, Hkv=1, T=200, D=64, S=4, bs=32),
])
def test_bf16_sink_irregular_lists(case):
    """bf16, lists with -1 anywhere, repeats, out-of-range and future blocks
    and empty rows (their lse is the sink, o and dq zero)."""
    rng = np.random.default_rng(31)
    c = dict(case)
    name = c.pop("name")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], c["bs"], c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=32, name=name, block_idx=idx)
    sink = _sink_vals(rng, c["Hq"])
    got, _ = _check(w, sink)
    empty = np.all((idx < 0) | (idx >= -(-c["T"] // c["bs"])), axis=-1)  # [B, Hkv, T]
    G = c["Hq"] // c["Hkv"]
    rows = np.repeat(empty, G, axis=1)
    assert rows.any()
    lse_empty = np.broadcast_to(sink.astype(np.float64)[None, :, None], rows.shape)[rows]
    np.testing.assert_allclose(got["lse"][rows], lse_empty, rtol=0, atol=1e-5)
    assert not got["o"][rows].any() and not got["dq"][rows].any()


def test_f32_sink_packed_and_dominant_sink():
    """fp32 packed sequences (one empty) with small and with dominant sink
    logits (o near 0, lse near the sink)."""
    rng = np.random.default_rng(33)
    w = workloads.make_thd([50, 0, 90, 17], 4, 2, 32, 3, 16, "f32", "own_random", seed=34,
                           name="sink-f32-packed")
    _check(w, _sink_vals(rng, 4))
    _check(w, _sink_vals(rng, 4, loc=12.0))


def test_sink_autograd_and_determinism():
    """selection_attn with a sink tensor that requires grad: gradients reach
    it and equal nsa_sel_bwd's dsink; two runs agree bit for bit."""
    rng = np.random.default_rng(35)
    w = workloads.make_workload("bf16_T1024")
    d = to_dev(w)
    sink_np = _sink_vals(rng, w.Hq)
    a = _run(w, d, sink_np)
    b = _run(w, d, sink_np)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    q, k, v = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    sink = torch.from_numpy(sink_np).cuda().requires_grad_(True)
    o = nsa.selection_attn(q, k, v, d["idx"], w.block_size, w.scale, sink=sink)
    o.backward(d["dO"])
    torch.cuda.synchronize()
    assert np.array_equal(sink.grad.cpu().numpy().astype(np.float64), a["dsink"])
    assert np.array_equal(o.detach().float().cpu().numpy().astype(np.float64), a["o"])
