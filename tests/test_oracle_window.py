"""Pins of the oracle's sliding-window mask (CPU only).

The pages list sliding-window masks among the backward's flavours and say
nothing more; the reading taken: a width W >= 1 keeps only the keys j with
t - W < j <= t on top of the block selection (W = 0: no window).  Pinned to
central finite differences, a dense masked formulation under torch
autograd, torch SDPA with an explicit window mask when every block is
selected, the no-window limit and a closed form (W = 1).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import test_oracle_pins as pins

WTINY = [dict(c, W=w) for c, w in zip(pins.TINY, (3, 2, 5))]


@pytest.mark.parametrize("c", WTINY)
def test_window_finite_differences(c):
    """Analytic dq, dk, dv equal central differences of <o, dO> with a window."""
    c = dict(c)
    W = c.pop("W")
    q, k, v, idx, dO = pins._case(**c)
    bs = c["bs"]
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs, window=W)

    def loss(q, k, v):
        o, _ = oracle.fwd(q, k, v, idx, bs, window=W)
        return float(np.sum(o * dO))

    h = 1e-6
    args = {"q": q, "k": k, "v": v}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
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


def _dense_window_torch(q, k, v, idx, bs, scale, W):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NB = -(-T // bs)
    idx_t = torch.as_tensor(idx).long()
    valid = (idx_t >= 0) & (idx_t < NB)
    listed = torch.zeros(B, Hkv, T, NB + 1, dtype=torch.bool)
    listed.scatter_(-1, torch.where(valid, idx_t, NB), True)
    key_block = torch.arange(T) // bs
    tq, tk = torch.arange(T)[:, None], torch.arange(T)[None, :]
    band = (tk <= tq) & (tk > tq - W)
    mask = (listed[..., :NB][..., key_block] & band).repeat_interleave(G, dim=1)
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = (scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())).masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    lse_safe = torch.where(torch.isinf(lse), torch.zeros_like(lse), lse)
    return torch.matmul(torch.exp(s - lse_safe[..., None]), vv), lse


@pytest.mark.parametrize("seed,B,Hq,Hkv,T,D,bs,S,W", [
    (41, 2, 4, 2, 40, 8, 4, 5, 7),
    (42, 1, 6, 2, 33, 6, 8, 3, 12),
])
def test_window_dense_autograd(seed, B, Hq, Hkv, T, D, bs, S, W):
    """o, lse, dq, dk, dv equal a dense masked softmax with the window band,
    differentiated by torch autograd in float64."""
    q, k, v, idx, dO = pins._case(seed, B, Hq, Hkv, T, D, bs, S)
    o, lse_f = oracle.fwd(q, k, v, idx, bs, window=W)
    dq, dk, dv, lse, _ = oracle.bwd(q, k, v, dO, idx, bs, window=W)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o_t, lse_t = _dense_window_torch(qt, kt, vt, idx, bs, D ** -0.5, W)
    o_t.backward(torch.tensor(dO))
    fin = ~np.isinf(lse_f)
    assert np.array_equal(np.isinf(lse_f), np.isinf(lse_t.detach().numpy()))
    np.testing.assert_allclose(lse_f[fin], lse_t.detach().numpy()[fin], atol=1e-12, rtol=0)
    for a, b in ((o, o_t), (dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(a, b.detach().numpy(), atol=1e-12, rtol=0)


def test_window_full_selection_is_windowed_sdpa():
    """Every block listed + window W equals torch SDPA with the band mask."""
    rng = np.random.default_rng(43)
    B, Hq, T, D, bs, W = 1, 2, 48, 8, 8, 10
    q, k, v, dO = (rng.standard_normal((B, Hq, T, D)) for _ in range(4))
    NB = T // bs
    idx = np.broadcast_to(np.arange(NB, dtype=np.int32), (B, Hq, T, NB)).copy()
    o, _ = oracle.fwd(q, k, v, idx, bs, window=W)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs, window=W)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tq, tk = torch.arange(T)[:, None], torch.arange(T)[None, :]
    band = (tk <= tq) & (tk > tq - W)
    ot = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=band)
    ot.backward(torch.tensor(dO))
    for a, b in ((o, ot), (dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(a, b.detach().numpy(), atol=1e-12, rtol=0)


def test_window_limits():
    """W >= T changes nothing (bit for bit); W = 1 leaves only the diagonal
    key: o = v_t, lse = scale <q_t, k_t>, dq = 0 (when the own block is listed)."""
    c = dict(pins.TINY[0])
    q, k, v, idx, dO = pins._case(**c)
    bs, T = c["bs"], c["T"]
    for a, b in zip(oracle.bwd(q, k, v, dO, idx, bs), oracle.bwd(q, k, v, dO, idx, bs, window=T)):
        assert np.array_equal(a, b)
    own = np.zeros_like(idx)
    own[...] = -1
    own[..., 0] = (np.arange(T) // bs)[None, None, :]
    o, lse = oracle.fwd(q, k, v, own, bs, window=1)
    dq, _, _, _, _ = oracle.bwd(q, k, v, dO, own, bs, window=1)
    G = q.shape[1] // k.shape[1]
    kk, vv = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    np.testing.assert_allclose(o, vv, rtol=1e-14)
    np.testing.assert_allclose(lse, np.sum(q * kk, axis=-1) / math.sqrt(q.shape[-1]), rtol=1e-13)
    assert np.abs(dq).max() == 0.0


def test_window_inversion_brute_force():
    """With a window, block u's list holds the tokens that list u and can see
    at least one of its keys (some j of u with t - W < j <= t), ascending,
    once each: plain Python against the oracle's inversion."""
    rng = np.random.default_rng(44)
    B, Hkv, T, bs, S, W = 2, 2, 50, 4, 6, 9
    idx = pins._weird_idx(rng, B, Hkv, T, bs, S)
    NB = -(-T // bs)
    counts, tokens = oracle.invert(idx, bs, window=W)
    pos = 0
    for b in range(B):
        for h in range(Hkv):
            for u in range(NB):
                lst = [t for t in range(T)
                       if u in set(int(x) for x in idx[b, h, t])
                       and any(t - W < j <= t for j in range(u * bs, min((u + 1) * bs, T)))]
                assert counts[b, h, u] == len(lst)
                assert tokens[pos:pos + len(lst)].tolist() == lst
                pos += len(lst)
    assert pos == len(tokens)
