"""Pins of the oracle's bottom-right causal alignment.

Page 3 of the reference text (the cudnn-frontend SM80 backward pull request)
lists a bottom-right causal flavour of the backward and nothing more.  The
reading taken: a dense problem may have Tk >= T keys per (batch entry, KV
head), the T queries being the last T positions of the key range, so query
t sits at key position p = t + Tk - T, attends keys j <= p (and, with a
window W, j > p - W) of its listed blocks, and block numbers count blocks
of the Tk keys.

Tied to something other than the new code path:
  * the square call: the bottom-right problem is the last T rows of a
    Tk x Tk problem, and its dk / dv are the square problem's with dO zeroed
    on the first Tk - T rows (those rows then have dS = 0 and P dO = 0);
  * a dense T x Tk masked softmax in torch float64 with autograd;
  * central finite differences;
  * a single decoding row (T = 1) written out in numpy;
  * the inversion and the pair count by brute force.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import _weird_idx


def _br_case(seed, B, Hq, Hkv, T, Tk, D, bs, S):
    """Square draw of Tk rows; the bottom-right problem takes its last T query
    rows (q, dO, block_idx) and all Tk keys."""
    rng = np.random.default_rng(seed)
    q_sq = rng.standard_normal((B, Hq, Tk, D))
    k = rng.standard_normal((B, Hkv, Tk, D))
    v = rng.standard_normal((B, Hkv, Tk, D))
    idx_sq = _weird_idx(rng, B, Hkv, Tk, bs, S)
    dO_sq = rng.standard_normal((B, Hq, Tk, D))
    off = Tk - T
    return (q_sq, k, v, idx_sq, dO_sq,
            np.ascontiguousarray(q_sq[:, :, off:]), np.ascontiguousarray(idx_sq[:, :, off:]),
            np.ascontiguousarray(dO_sq[:, :, off:]))


BR_CASES = [
    (31, 1, 4, 2, 13, 40, 6, 8, 4),    # Tk - T not a multiple of bs
    (32, 2, 3, 1, 1, 37, 4, 4, 6),     # one query: decoding
    (33, 1, 2, 2, 24, 24, 5, 4, 3),    # Tk = T
    (34, 1, 6, 3, 20, 52, 4, 16, 3),   # G = 2, a few large blocks
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,T,Tk,D,bs,S", BR_CASES)
@pytest.mark.parametrize("window", [0, 9])
def test_bottom_right_is_the_tail_of_the_square_problem(seed, B, Hq, Hkv, T, Tk, D, bs, S, window):
    q_sq, k, v, idx_sq, dO_sq, q, idx, dO = _br_case(seed, B, Hq, Hkv, T, Tk, D, bs, S)
    off = Tk - T
    o_sq, lse_sq = oracle.fwd(q_sq, k, v, idx_sq, bs, window=window)
    o, lse = oracle.fwd(q, k, v, idx, bs, window=window)
    np.testing.assert_allclose(o, o_sq[:, :, off:], atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(lse), np.isinf(lse_sq[:, :, off:]))
    fin = ~np.isinf(lse)
    np.testing.assert_allclose(lse[fin], lse_sq[:, :, off:][fin], atol=1e-12, rtol=0)
    dO_tail = dO_sq.copy()
    dO_tail[:, :, :off] = 0.0
    dq_sq, dk_sq, dv_sq, _, _ = oracle.bwd(q_sq, k, v, dO_tail, idx_sq, bs, window=window)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs, window=window)
    np.testing.assert_allclose(dq, dq_sq[:, :, off:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, dk_sq, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, dv_sq, atol=1e-12, rtol=0)
    assert np.abs(dk).max() > 1e-3 and np.abs(dq).max() > 1e-3  # not vacuous


def _dense_br_torch(q, k, v, idx, bs, scale, window=0):
    """T x Tk scores, a selection mask built with scatter, the bottom-right
    causal limit j <= t + Tk - T, library softmax; autograd for gradients."""
    B, Hq, T, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    NB = -(-Tk // bs)
    idx_t = torch.as_tensor(idx).long()
    valid = (idx_t >= 0) & (idx_t < NB)
    listed = torch.zeros(B, Hkv, T, NB + 1, dtype=torch.bool)
    listed.scatter_(-1, torch.where(valid, idx_t, NB), True)
    key_block = torch.arange(Tk) // bs
    pos = torch.arange(T)[:, None] + (Tk - T)
    keys = torch.arange(Tk)[None, :]
    allowed = keys <= pos
    if window:
        allowed = allowed & (keys > pos - window)
    mask = listed[..., :NB][..., key_block] & allowed
    mask = mask.repeat_interleave(G, dim=1)
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())
    s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    lse_safe = torch.where(torch.isinf(lse), torch.zeros_like(lse), lse)
    p = torch.exp(s - lse_safe[..., None])
    return torch.matmul(p, vv), lse


@pytest.mark.parametrize("seed,B,Hq,Hkv,T,Tk,D,bs,S", BR_CASES)
def test_bottom_right_dense_autograd(seed, B, Hq, Hkv, T, Tk, D, bs, S):
    _, k, v, _, _, q, idx, dO = _br_case(seed, B, Hq, Hkv, T, Tk, D, bs, S)
    scale = D ** -0.5
    o, lse = oracle.fwd(q, k, v, idx, bs)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o_t, lse_t = _dense_br_torch(qt, kt, vt, idx, bs, scale)
    o_t.backward(torch.tensor(dO))
    np.testing.assert_allclose(o, o_t.detach().numpy(), atol=1e-12, rtol=0)
    lt = lse_t.detach().numpy()
    assert np.array_equal(np.isinf(lse), np.isinf(lt))
    np.testing.assert_allclose(lse[~np.isinf(lse)], lt[~np.isinf(lt)], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12, rtol=0)


def test_bottom_right_finite_differences():
    _, k, v, _, _, q, idx, dO = _br_case(35, 1, 2, 1, 4, 11, 3, 3, 3)
    bs = 3
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs)

    def loss(q, k, v):
        o, _ = oracle.fwd(q, k, v, idx, bs)
        return float(np.sum(o * dO))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            a_p, a_m = {"q": q, "k": k, "v": v}, {"q": q, "k": k, "v": v}
            a_p[name], a_m[name] = xp, xm
            fd[i] = (loss(**a_p) - loss(**a_m)) / (2 * h)
        assert np.all(np.abs(fd - g) <= 1e-7 * (1 + np.abs(g))), name
        assert np.abs(g).max() > 1e-3


def test_single_decoding_row_written_out():
    """T = 1: the query sits at the last key position and sees every key of
    each block it lists (the last block may be partial)."""
    rng = np.random.default_rng(36)
    Tk, D, bs = 45, 5, 8
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, Tk, D))
    v = rng.standard_normal((1, 1, Tk, D))
    idx = np.array([[[[5, 1, -1, 1, 9]]]], dtype=np.int32)  # 9 >= NB = 6: skipped
    o, lse = oracle.fwd(q, k, v, idx, bs)
    keys = [j for j in range(Tk) if j // bs in (1, 5)]
    s = (D ** -0.5) * (k[0, 0, keys] @ q[0, 0, 0])
    ref_lse = np.log(np.sum(np.exp(s)))
    p = np.exp(s - ref_lse)
    np.testing.assert_allclose(lse[0, 0, 0], ref_lse, atol=1e-12, rtol=0)
    np.testing.assert_allclose(o[0, 0, 0], p @ v[0, 0, keys], atol=1e-12, rtol=0)


@pytest.mark.parametrize("window", [0, 7])
def test_bottom_right_inversion_and_pair_count(window):
    B, Hq, Hkv, T, Tk, bs, S = 2, 4, 2, 19, 50, 6, 5
    _, _, _, _, _, _, idx, _ = _br_case(37, B, Hq, Hkv, T, Tk, 2, bs, S)
    off = Tk - T
    NB = -(-Tk // bs)
    counts, tokens = oracle.invert(idx, bs, window, Tk=Tk)
    ref_counts = np.zeros((B, Hkv, NB), dtype=np.int32)
    ref_tokens = []
    for b in range(B):
        for h in range(Hkv):
            for u in range(NB):
                for t in range(T):
                    p = t + off
                    if u * bs <= p and u in set(idx[b, h, t].tolist()) and \
                            (window == 0 or (u + 1) * bs - 1 > p - window):
                        ref_counts[b, h, u] += 1
                        ref_tokens.append(t)
    assert np.array_equal(counts, ref_counts)
    assert np.array_equal(tokens, np.array(ref_tokens, dtype=np.int32))
    n = 0
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                lst = {u for u in idx[b, h, t].tolist() if 0 <= u < NB}
                n += G * sum(1 for j in range(Tk) if j // bs in lst and j <= t + off)
    assert oracle.count_pairs(idx, Hq, bs, Tk=Tk) == n
