"""CPU checks of the derived dsink gate (tests/_harness.dsink_bound): it covers
an emulation of the GPU's roundings (bf16 o, fp32 lse, fp32 Delta, fp32
P_sink and an fp32 sum) and it rejects a 10 % error, which the earlier
element-gate-times-sqrt(rows) gate let through."""
import numpy as np

import oracle
import workloads
from _harness import dsink_bound


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def test_dsink_bound_covers_emulated_rounding_and_is_tight():
    w = workloads.make_dense(1, 8, 2, 300, 64, 5, 32, "bf16", seed=3, name="tol")
    rng = np.random.default_rng(4)
    sink = rng.normal(0.5, 1.5, size=w.Hq).astype(np.float32)
    sk = sink.astype(np.float64)
    o_r, lse_fwd = oracle.fwd(w.q, w.k, w.v, w.block_idx, w.block_size, w.scale, sink=sk)
    _, _, _, lse_r, dl_r = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, w.block_size, w.scale,
                                      sink=sk)
    ds_r = oracle.dsink(sk, lse_r, dl_r, head_axis=1)
    # the GPU's roundings: o to bf16, lse to fp32, Delta and P in fp32, a
    # serial fp32 sum per head
    o_g = workloads.round_to_bf16(_f32(o_r)).astype(np.float64)
    lse_g = _f32(lse_fwd).astype(np.float64)
    dl_g = np.sum(_f32(w.dO) * _f32(o_g), axis=-1, dtype=np.float32)
    p_g = np.exp(_f32(sk)[None, :, None] - _f32(lse_g)).astype(np.float32)
    terms = (p_g * dl_g).astype(np.float32)                      # [B, Hq, T]
    ds_g = np.zeros(w.Hq, np.float32)
    for t in range(w.T):
        ds_g = (ds_g + terms[0, :, t]).astype(np.float32)
    ds_g = -ds_g.astype(np.float64)
    got = {"o": o_g, "lse": lse_g}
    ref = {"o": o_r}
    bound = dsink_bound(w, got, ref, sink, lse_r, dl_r)
    err = np.abs(ds_g - ds_r)
    assert np.all(err <= bound), (err, bound)
    assert np.all(bound > 0)
    # far tighter than the old gate (6e-2 * sqrt(rows)) and than a 10 % error
    assert np.all(bound < 0.1 * 6e-2 * np.sqrt(w.T))
    big = np.abs(ds_r) > 1.0
    assert big.any()
    assert np.all(0.1 * np.abs(ds_r[big]) > 1.25 * bound[big] + 1e-6)
