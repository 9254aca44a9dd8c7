"""GPU check of the stand-alone Delta launch (nsa_sel_delta; the backward's
prepare_delta stage runs the same kernel): Delta[row] = sum_d dO[row, d]
o[row, d], the row term of page 1's backward gradients, laid out like lse.

Every row is compared with the float64 sum of the same bf16 inputs.  A
bf16 x bf16 product is exact in fp32, so the only rounding is in the D - 1
additions, whatever their order: |err| <= (D - 1) 2^-24 sum_d |dO o| to first
order; the gate takes twice that.  Row counts leave ragged last blocks (the
kernel takes 4 groups of 256 / (D / 8) rows per block); D = 32, 64 and 128,
dense and packed (with an empty sequence).  The bitwise agreement of this
launch with the Delta that the one-call backward computes is covered by the
two-stream schedule test, which compares whole backward results."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import workloads
from _harness import say, to_dev

pytestmark = pytest.mark.gpu


def _bf16(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda().to(torch.bfloat16)


def _check(name, got, o, dO, row_axis_last):
    o64 = o.float().cpu().numpy().astype(np.float64)
    d64 = dO.float().cpu().numpy().astype(np.float64)
    prod = o64 * d64
    ref, mag = prod.sum(-1), np.abs(prod).sum(-1)
    if not row_axis_last:  # packed: [Ttot, Hq] -> lse layout [Hq, Ttot]
        ref, mag = ref.T, mag.T
    g = got.cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape
    assert np.isfinite(g).all()
    D = o.shape[-1]
    bound = 2.0 * (D - 1) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(g - ref)
    say(f"[{name}] rows={ref.size} D={D}: max|err| = {err.max():.3e}, "
        f"max err/bound = {(err / bound).max():.3f}")
    assert np.all(err <= bound), (err / bound).max()


@pytest.mark.parametrize("case", [
    dict(name="delta-D32", B=1, Hq=4, Hkv=1, T=257, D=32, S=3, bs=32),
    dict(name="delta-D64", B=2, Hq=6, Hkv=2, T=333, D=64, S=4, bs=32),
    dict(name="delta-D128", B=1, Hq=32, Hkv=2, T=1000, D=128, S=5, bs=64),
])
def test_delta_dense(case):
    c = dict(case)
    name = c.pop("name")
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=91, name=name)
    d = to_dev(w)
    rng = np.random.default_rng(92)
    o, dO = _bf16(rng, d["q"].shape), _bf16(rng, d["q"].shape)
    got = nsa.nsa_sel_delta(o, dO, w.block_size, d["idx"], d["k"], w.scale)
    torch.cuda.synchronize()
    _check(name, got, o, dO, row_axis_last=True)


def test_delta_packed():
    w = workloads.make_thd([300, 0, 65, 513], 8, 2, 128, 4, 64, "bf16", "own_first_random",
                           seed=93, name="delta-packed")
    d = to_dev(w)
    rng = np.random.default_rng(94)
    o, dO = _bf16(rng, d["q"].shape), _bf16(rng, d["q"].shape)
    got = nsa.nsa_sel_delta(o, dO, w.block_size, d["idx"], d["k"], w.scale, d["cu"], w.max_seqlen)
    torch.cuda.synchronize()
    _check("delta-packed", got, o, dO, row_axis_last=False)
