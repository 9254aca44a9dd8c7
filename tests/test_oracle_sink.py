"""Pins of the oracle's attention-sink extension (CPU only).

Page 3 of the reference text names a dSink step in the backward's kernel
chain without defining it.  The reading taken: a per-head logit sink[h] (no
scale) joins every row's softmax denominator and carries no value, so
lse = log(sum_j exp(s_j) + exp(sink[h])), o = sum_j exp(s_j - lse) v_j, and
the backward's dq/dk/dv keep their formulas with that lse.  These tests pin
it to central finite differences, to a dense formulation with the sink as an
extra score column differentiated by torch autograd, to the no-sink oracle
(sink = -inf), and to closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import test_oracle_pins as pins


def _sink(rng, Hq):
    return rng.normal(0.5, 1.5, size=Hq)


@pytest.mark.parametrize("c", pins.TINY)
def test_sink_finite_differences(c):
    """Analytic dq, dk, dv and dsink equal central differences of
    L = <o(q, k, v, sink), dO>."""
    q, k, v, idx, dO = pins._case(**c)
    bs, Hq = c["bs"], c["Hq"]
    sink = _sink(np.random.default_rng(c["seed"] + 100), Hq)
    dq, dk, dv, lse, delta = oracle.bwd(q, k, v, dO, idx, bs, sink=sink)
    dsk = oracle.dsink(sink, lse, delta, head_axis=1)

    def loss(q, k, v, sink):
        o, _ = oracle.fwd(q, k, v, idx, bs, sink=sink)
        return float(np.sum(o * dO))

    h = 1e-6
    args = {"q": q, "k": k, "v": v, "sink": sink}
    for name, g in (("q", dq), ("k", dk), ("v", dv), ("sink", dsk)):
        x = args[name]
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            fd[i] = (loss(**{**args, name: xp}) - loss(**{**args, name: xm})) / (2 * h)
        err = np.abs(fd - g)
        assert np.all(err <= 1e-7 * (1 + np.abs(g))), (name, err.max())
        assert np.abs(g).max() > 1e-3


def _dense_with_sink_torch(q, k, v, idx, bs, scale, sink):
    """Dense masked scores plus one extra column per row holding the head's
    sink logit (value zero): library logsumexp and autograd."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NB = -(-T // bs)
    idx_t = torch.as_tensor(idx).long()
    valid = (idx_t >= 0) & (idx_t < NB)
    listed = torch.zeros(B, Hkv, T, NB + 1, dtype=torch.bool)
    listed.scatter_(-1, torch.where(valid, idx_t, NB), True)
    key_block = torch.arange(T) // bs
    causal = torch.arange(T)[None, :] <= torch.arange(T)[:, None]
    mask = (listed[..., :NB][..., key_block] & causal).repeat_interleave(G, dim=1)
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = (scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())).masked_fill(~mask, -math.inf)
    col = sink.view(1, Hq, 1, 1).expand(B, Hq, T, 1)
    lse = torch.logsumexp(torch.cat([s, col], dim=-1), dim=-1)
    p = torch.exp(s - lse[..., None])
    return torch.matmul(p, vv), lse


@pytest.mark.parametrize("seed,B,Hq,Hkv,T,D,bs,S", [
    (21, 2, 4, 2, 40, 8, 4, 5),
    (22, 1, 6, 2, 33, 6, 8, 3),
])
def test_sink_dense_autograd(seed, B, Hq, Hkv, T, D, bs, S):
    """o, lse, dq, dk, dv and dsink equal the dense formulation with the sink
    as an extra score column, differentiated by torch autograd (float64)."""
    q, k, v, idx, dO = pins._case(seed, B, Hq, Hkv, T, D, bs, S)
    sink = _sink(np.random.default_rng(seed), Hq)
    o, lse_f = oracle.fwd(q, k, v, idx, bs, sink=sink)
    dq, dk, dv, lse, delta = oracle.bwd(q, k, v, dO, idx, bs, sink=sink)
    dsk = oracle.dsink(sink, lse, delta, head_axis=1)
    qt, kt, vt, st = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                      for x in (q, k, v, sink))
    o_t, lse_t = _dense_with_sink_torch(qt, kt, vt, idx, bs, D ** -0.5, st)
    o_t.backward(torch.tensor(dO))
    for a, b in ((o, o_t), (lse_f, lse_t), (lse, lse_t), (dq, qt.grad), (dk, kt.grad),
                 (dv, vt.grad), (dsk, st.grad)):
        np.testing.assert_allclose(a, b.detach().numpy(), atol=1e-12, rtol=0)


def test_sink_minus_inf_is_no_sink():
    """A sink of -inf changes nothing, bit for bit."""
    q, k, v, idx, dO = pins._case(**pins.TINY[0])
    bs, Hq = pins.TINY[0]["bs"], pins.TINY[0]["Hq"]
    none = oracle.bwd(q, k, v, dO, idx, bs)
    off = oracle.bwd(q, k, v, dO, idx, bs, sink=np.full(Hq, -np.inf))
    for a, b in zip(none, off):
        assert np.array_equal(a, b)


def test_sink_closed_forms_and_empty_rows():
    """One token (one key): o = v0 * logistic(s0 - sink), lse = log(e^s0 +
    e^sink).  A row with no key: lse = sink, o = dq = 0, no dsink share."""
    rng = np.random.default_rng(5)
    D = 3
    q, k, v, dO = (rng.standard_normal((1, 1, 1, D)) for _ in range(4))
    idx = np.zeros((1, 1, 1, 1), np.int32)
    sink = np.array([0.7])
    o, lse = oracle.fwd(q, k, v, idx, 1, sink=sink)
    s0 = float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(D)
    p0 = 1.0 / (1.0 + math.exp(sink[0] - s0))
    np.testing.assert_allclose(o[0, 0, 0], p0 * v[0, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(math.exp(s0) + math.exp(sink[0])), rtol=1e-14)
    # empty rows: every entry padding
    q, k, v, dO = (rng.standard_normal((1, 2, 5, D)) for _ in range(4))
    k, v = k[:, :1], v[:, :1]
    idx = np.full((1, 1, 5, 2), -1, np.int32)
    sink = np.array([0.3, -1.2])
    dq, dk, dv, lse, delta = oracle.bwd(q, k, v, dO, idx, 2, sink=sink)
    o, _ = oracle.fwd(q, k, v, idx, 2, sink=sink)
    assert np.array_equal(lse, np.broadcast_to(sink[None, :, None], lse.shape))
    assert not o.any() and not dq.any() and not dk.any() and not dv.any()
    assert not oracle.dsink(sink, lse, delta, head_axis=1).any()
