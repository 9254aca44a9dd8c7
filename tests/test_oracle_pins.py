"""Pins of the float64 oracle against things other than itself.

Method source: page 1 of the reference text ("test_kernel_backward.py",
module docstring and run_one): NSA selection attention, G = Hq/Hkv query heads
sharing one KV head and one block list, backward = exact gradient of the
forward.  Each test below ties the oracle to an independent fact:

  * central finite differences of <o, dO>            -> the whole backward
  * dense masked softmax in torch float64 + autograd  -> forward and backward
  * all-blocks selection == causal SDPA (float64)     -> forward, backward, scale
  * own-block-only selection == per-block causal SDPA -> block geometry
  * GQA == sum over the G heads of the MHA expansion  -> head grouping
  * closed forms (first token, two keys in one dim)   -> lse, scale, softmax
  * invariants (rows sum to 1, sum_j dS = 0, Delta = <dO, o>)
  * sentinels: perturbing keys a row must not see leaves it unchanged, and
    perturbing keys it must see changes it           -> selection semantics
  * brute-force Python inversion                      -> block -> token lists
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _weird_idx(rng, B, Hkv, T, bs, S):
    """Own block + random earlier blocks, then sprinkled with the cases the
    pages leave open: -1 in any slot, other negatives, duplicates, indices
    >= NB, future blocks, and one row with nothing listed."""
    NB = -(-T // bs)
    idx = np.stack([workloads.block_idx_own_random(rng, Hkv, T, bs, S) for _ in range(B)])
    flat = idx.reshape(-1, S)
    n = flat.shape[0]
    for r in rng.choice(n, size=max(1, n // 4), replace=False):
        s = rng.integers(0, S)
        kind = rng.integers(0, 5)
        if kind == 0:
            flat[r, s] = -1
        elif kind == 1:
            flat[r, s] = -7
        elif kind == 2:
            flat[r, s] = flat[r, 0]  # duplicate of the own block
        elif kind == 3:
            flat[r, s] = NB + rng.integers(0, 3)  # out of range
        else:
            flat[r, s] = rng.integers(0, NB)  # possibly a future block
    flat[rng.integers(0, n)] = -1  # an empty row
    return flat.reshape(idx.shape)


def _case(seed, B, Hq, Hkv, T, D, bs, S):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    idx = _weird_idx(rng, B, Hkv, T, bs, S)
    dO = rng.standard_normal((B, Hq, T, D))
    return q, k, v, idx, dO


TINY = [
    dict(seed=1, B=1, Hq=2, Hkv=1, T=10, D=4, bs=3, S=3),   # G=2, T % bs != 0
    dict(seed=2, B=2, Hq=3, Hkv=1, T=8, D=3, bs=2, S=2),    # G=3, B=2
    dict(seed=3, B=1, Hq=2, Hkv=2, T=9, D=5, bs=4, S=3),    # G=1
]


@pytest.mark.parametrize("c", TINY)
def test_finite_differences(c):
    """O1: analytic grads equal central differences of L = <o(q,k,v), dO>."""
    q, k, v, idx, dO = _case(**c)
    bs = c["bs"]
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
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[i] = (loss(**args_p) - loss(**args_m)) / (2 * h)
        err = np.abs(fd - g)
        assert np.all(err <= 1e-7 * (1 + np.abs(g))), (name, err.max())
        assert np.abs(g).max() > 1e-3  # the check is not vacuous


def _dense_masked_torch(q, k, v, idx, bs, scale):
    """Independent formulation: a dense T x T score matrix, a selection mask
    built with scatter (so repeated listings collapse), library softmax, and
    torch autograd for the gradients."""
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
    mask = listed[..., :NB][..., key_block] & causal
    mask = mask.repeat_interleave(G, dim=1)
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())
    s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    lse_safe = torch.where(torch.isinf(lse), torch.zeros_like(lse), lse)
    p = torch.exp(s - lse_safe[..., None])
    o = torch.matmul(p, vv)
    return o, lse


@pytest.mark.parametrize("seed,B,Hq,Hkv,T,D,bs,S", [
    (11, 2, 4, 2, 40, 8, 4, 5),
    (12, 1, 6, 2, 33, 6, 8, 3),
    (13, 1, 3, 3, 24, 4, 2, 6),
])
def test_dense_masked_autograd(seed, B, Hq, Hkv, T, D, bs, S):
    """O2: the oracle's explicit forward/backward equal a dense masked softmax
    differentiated by torch autograd, in float64."""
    q, k, v, idx, dO = _case(seed, B, Hq, Hkv, T, D, bs, S)
    scale = D ** -0.5
    o_ref_np, lse_ref_np = oracle.fwd(q, k, v, idx, bs)
    dq, dk, dv, lse, delta = oracle.bwd(q, k, v, dO, idx, bs)

    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o_t, lse_t = _dense_masked_torch(qt, kt, vt, idx, bs, scale)
    o_t.backward(torch.tensor(dO))
    np.testing.assert_allclose(o_ref_np, o_t.detach().numpy(), atol=1e-12, rtol=0)
    both_inf = np.isinf(lse_ref_np) & np.isinf(lse_t.detach().numpy())
    assert np.array_equal(np.isinf(lse_ref_np), np.isinf(lse_t.detach().numpy()))
    np.testing.assert_allclose(lse_ref_np[~both_inf], lse_t.detach().numpy()[~both_inf],
                               atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref_np)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12, rtol=0)


def _sdpa_causal_gqa(q, k, v, dO):
    """torch SDPA (is_causal, math path, float64 CPU) with the G-fold head
    expansion; grads of k/v summed back over each group."""
    G = q.shape[1] // k.shape[1]
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1),
                                       is_causal=True)
    o.backward(torch.tensor(dO))
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("B,Hq,Hkv,T,D,bs", [(2, 4, 1, 48, 16, 8), (1, 6, 2, 35, 8, 16)])
def test_full_selection_is_causal_sdpa(B, Hq, Hkv, T, D, bs):
    """O3: listing every block 0..t//bs reproduces dense causal attention
    (fwd and bwd), with scale 1/sqrt(D)."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    dO = rng.standard_normal((B, Hq, T, D))
    NB = -(-T // bs)
    idx = np.stack([workloads.block_idx_dense(Hkv, T, bs, NB) for _ in range(B)])
    o, _ = oracle.fwd(q, k, v, idx, bs)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    o_r, dq_r, dk_r, dv_r = _sdpa_causal_gqa(q, k, v, dO)
    for a, b in ((o, o_r), (dq, dq_r), (dk, dk_r), (dv, dv_r)):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_own_block_only_is_blockwise_causal():
    """O8b: S=1 own-block-only selection equals causal attention run on each
    block of tokens alone."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, T, D, bs = 1, 4, 2, 40, 8, 8
    q, k, v, dO = (rng.standard_normal((B, h, T, D)) for h in (Hq, Hkv, Hkv, Hq))
    idx = (np.arange(T) // bs).astype(np.int32)[None, None, :, None].repeat(Hkv, 1)
    o, _ = oracle.fwd(q, k, v, idx, bs)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    for u in range(T // bs):
        sl = slice(u * bs, (u + 1) * bs)
        o_r, dq_r, dk_r, dv_r = _sdpa_causal_gqa(q[:, :, sl], k[:, :, sl], v[:, :, sl],
                                                 dO[:, :, sl])
        np.testing.assert_allclose(o[:, :, sl], o_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dq[:, :, sl], dq_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk[:, :, sl], dk_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv[:, :, sl], dv_r, atol=1e-12, rtol=0)


def test_gqa_equals_sum_over_heads():
    """O4: with G heads per KV head, dk/dv equal the sum over the group's
    heads of the MHA problem whose K/V and block lists are repeated per head;
    o and dq are unchanged by the expansion."""
    q, k, v, idx, dO = _case(21, 2, 6, 2, 30, 5, 4, 4)
    G = 3
    bs = 4
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    o, lse = oracle.fwd(q, k, v, idx, bs)
    ke, ve, ie = (np.repeat(x, G, axis=1) for x in (k, v, idx))
    dq_e, dk_e, dv_e, _, _ = oracle.bwd(q, ke, ve, dO, ie, bs)
    o_e, lse_e = oracle.fwd(q, ke, ve, ie, bs)
    np.testing.assert_allclose(o, o_e, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dq, dq_e, atol=1e-13, rtol=0)
    B, Hkv, T, D = k.shape
    np.testing.assert_allclose(dk, dk_e.reshape(B, Hkv, G, T, D).sum(2), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, dv_e.reshape(B, Hkv, G, T, D).sum(2), atol=1e-12, rtol=0)


def test_rows_sum_to_one_and_invariants():
    """O5/O6: with v = 1 every non-empty row outputs 1 (P sums to 1); with a
    one-hot v column each P_j lies in [0, 1]; sum_j dk = 0 per (b, hkv);
    sum_j dv = sum of dO over non-empty rows; Delta = <dO, o>."""
    q, k, v, idx, dO = _case(31, 2, 4, 2, 36, 6, 4, 4)
    bs = 4
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o1, lse = oracle.fwd(q, k, np.ones_like(v), idx, bs)
    empty = np.isinf(lse)
    assert empty.any() and not empty.all()
    np.testing.assert_allclose(o1[~empty], 1.0, atol=1e-14)
    assert np.all(o1[empty] == 0.0)
    vh = np.zeros_like(v)
    vh[..., 0] = 1.0
    vh[..., 1] = np.arange(T)[None, None, :]
    oh, _ = oracle.fwd(q, k, vh, idx, bs)
    assert np.all(oh[..., 0] >= -1e-15) and np.all(oh[..., 0] <= 1 + 1e-14)
    # o[...,1] is the expected key position, which cannot exceed t (causality).
    assert np.all(oh[..., 1] <= np.arange(T)[None, None, :] + 1e-9)

    o, _ = oracle.fwd(q, k, v, idx, bs)
    dq, dk, dv, lse2, delta = oracle.bwd(q, k, v, dO, idx, bs)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    nonempty = (~empty).astype(np.float64)[..., None]
    dv_expect = (dO * nonempty).reshape(B, Hkv, G, T, D).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), dv_expect, atol=1e-11)
    np.testing.assert_allclose(delta, np.sum(dO * o, axis=-1), atol=1e-12)
    assert np.all(dq[empty] == 0.0)


def test_closed_forms():
    """O8: the first token sees only key 0 (o = v0, lse = scale<q,k0>, dq = 0);
    a D=1, two-key row is a logistic function of the score gap."""
    q, k, v, idx, dO = _case(41, 1, 2, 1, 12, 4, 4, 3)
    idx[:, :, 0, :] = -1
    idx[:, :, 0, 0] = 0
    bs, D = 4, 4
    o, lse = oracle.fwd(q, k, v, idx, bs)
    dq, _, _, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    for h in range(2):
        np.testing.assert_allclose(o[0, h, 0], v[0, 0, 0], atol=1e-15)
        np.testing.assert_allclose(lse[0, h, 0], D ** -0.5 * q[0, h, 0] @ k[0, 0, 0], atol=1e-14)
        assert np.all(dq[0, h, 0] == 0.0)

    # Two keys, D = 1, bs = 1: row t=1 lists blocks {0, 1}.
    a, k0, k1, v0, v1, g = 0.7, -1.3, 0.4, 2.0, -0.5, 1.7
    q2 = np.array([[[[0.0], [a]]]])
    k2 = np.array([[[[k0], [k1]]]])
    v2 = np.array([[[[v0], [v1]]]])
    dO2 = np.array([[[[0.0], [g]]]])
    idx2 = np.array([[[[0, -1], [1, 0]]]], dtype=np.int32)
    o2, lse2 = oracle.fwd(q2, k2, v2, idx2, 1)
    dq2, dk2, dv2, _, _ = oracle.bwd(q2, k2, v2, dO2, idx2, 1)
    s0, s1 = a * k0, a * k1                       # scale = 1 for D = 1
    p1 = 1.0 / (1.0 + math.exp(s0 - s1))
    p0 = 1.0 - p1
    assert abs(o2[0, 0, 1, 0] - (p0 * v0 + p1 * v1)) < 1e-15
    assert abs(lse2[0, 0, 1] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-14
    # d o / d s1 = p0 p1 (v1 - v0); s1 = a k1, s0 = a k0.
    dsig = p0 * p1 * (v1 - v0) * g
    assert abs(dq2[0, 0, 1, 0] - dsig * (k1 - k0)) < 1e-14
    assert abs(dk2[0, 0, 1, 0] - dsig * a) < 1e-14
    assert abs(dk2[0, 0, 0, 0] - (-dsig * a)) < 1e-14
    assert abs(dv2[0, 0, 1, 0] - p1 * g) < 1e-15
    # key 0 also serves row 0 (whose dO is 0 here), so dv0 = p0 g.
    assert abs(dv2[0, 0, 0, 0] - p0 * g) < 1e-15


def test_slot_order_padding_and_duplicates_change_nothing():
    """O7: permuting a row's slots, adding -1 / >= NB entries or repeating a
    listed block leaves every output unchanged."""
    q, k, v, idx, dO = _case(51, 1, 4, 2, 32, 4, 4, 4)
    bs, NB = 4, 8
    rng = np.random.default_rng(0)
    base = oracle.bwd(q, k, v, dO, idx, bs)
    perm = idx[..., rng.permutation(idx.shape[-1])]
    wide = np.concatenate([idx, np.full(idx.shape[:-1] + (3,), -1, np.int32)], axis=-1)
    wide[..., -2] = NB + 5
    wide[..., -1] = idx[..., 0]
    for alt in (perm, wide):
        other = oracle.bwd(q, k, v, dO, alt, bs)
        for a, b in zip(base, other):
            np.testing.assert_array_equal(a, b)


def test_selection_sentinels():
    """Keys a row must not see (unlisted blocks, keys after t inside a listed
    block) do not move that row; keys it must see do."""
    q, k, v, idx, dO = _case(61, 1, 2, 1, 24, 4, 4, 3)
    bs = 4
    t = 14  # block 3
    idx[0, 0, t] = [3, 1, -1]
    o, lse = oracle.fwd(q, k, v, idx, bs)
    hidden = [j for j in range(24) if not (j // bs == 1 or (j // bs == 3 and j <= t))]
    seen = [j for j in range(24) if j not in hidden]
    assert 15 in hidden and 12 in seen and 4 in seen and 0 in hidden
    for j in hidden:
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, j] += 3.0
        v2[0, 0, j] -= 2.0
        o2, lse2 = oracle.fwd(q, k2, v2, idx, bs)
        np.testing.assert_array_equal(o2[0, :, t], o[0, :, t])
        np.testing.assert_array_equal(lse2[0, :, t], lse[0, :, t])
    for j in seen:
        v2 = v.copy()
        v2[0, 0, j] += 1.0
        o2, _ = oracle.fwd(q, k, v2, idx, bs)
        assert np.all(np.abs(o2[0, :, t] - o[0, :, t]) > 1e-6)


def test_inversion_brute_force():
    """O9: per (b, hkv, block u) the ascending tokens t >= u*bs listing u,
    once each, against plain Python dict-of-lists."""
    rng = np.random.default_rng(71)
    B, Hkv, T, bs, S = 2, 3, 50, 4, 5
    idx = _weird_idx(rng, B, Hkv, T, bs, S)
    NB = -(-T // bs)
    counts, tokens = oracle.invert(idx, bs)
    expect = {}
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                for u in set(int(x) for x in idx[b, h, t]):
                    if 0 <= u < NB and u * bs <= t:
                        expect.setdefault((b, h, u), []).append(t)
    pos = 0
    for b in range(B):
        for h in range(Hkv):
            for u in range(NB):
                lst = expect.get((b, h, u), [])
                assert counts[b, h, u] == len(lst)
                assert tokens[pos:pos + len(lst)].tolist() == lst
                pos += len(lst)
    assert pos == len(tokens)


def test_count_pairs_brute_force():
    """N = sum over rows of |A| against a Python set construction."""
    rng = np.random.default_rng(81)
    B, Hq, Hkv, T, bs, S = 2, 4, 2, 27, 4, 4
    idx = _weird_idx(rng, B, Hkv, T, bs, S)
    NB = -(-T // bs)
    n = 0
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                blocks = {int(u) for u in idx[b, h, t] if 0 <= u < NB}
                n += (Hq // Hkv) * sum(1 for j in range(t + 1) if j // bs in blocks)
    assert oracle.count_pairs(idx, Hq, bs) == n


def test_packed_sequences_are_independent():
    """A packed batch equals its sequences run alone, and changing one
    sequence's K/V leaves the other sequences' outputs bitwise equal."""
    w = workloads.make_thd([12, 20, 8], 4, 2, 4, 3, 4, "f32", "own_first_random", seed=3)
    o, lse = oracle.fwd_thd(w.q, w.k, w.v, w.block_idx, w.cu_seqlens, 4)
    k2 = w.k.copy()
    k2[12:32] += np.random.default_rng(9).standard_normal(k2[12:32].shape)  # sequence 1
    o2, lse2 = oracle.fwd_thd(w.q, k2, w.v, w.block_idx, w.cu_seqlens, 4)
    np.testing.assert_array_equal(o[:12], o2[:12])
    np.testing.assert_array_equal(o[32:], o2[32:])
    assert np.abs(o[12:32] - o2[12:32]).max() > 1e-3
    a, b = 12, 32
    o1, l1 = oracle.fwd(w.q[a:b].transpose(1, 0, 2)[None], w.k[a:b].transpose(1, 0, 2)[None],
                        w.v[a:b].transpose(1, 0, 2)[None], w.block_idx[:, a:b][None], 4)
    np.testing.assert_array_equal(o[a:b], o1[0].transpose(1, 0, 2))
