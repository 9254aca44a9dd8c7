"""Pins of the oracle's packed (THD) split and of its row / key subset calls.

The packed helpers (oracle.fwd_thd / oracle.bwd_thd) run one dense problem per
sequence.  Here they are tied to a formulation that never splits the batch:
the whole packed batch as one Ttot x Ttot masked softmax per query head, the
mask block-diagonal over the sequences (page 3 of the reference text, the
cudnn-frontend SM80 backward pull request: packed THD tensors described by one
cumulative-length array for queries and keys, so no key crosses a sequence),
sequence-local block numbers mapped onto global key positions, and torch
autograd in float64 for the gradients.

The subset calls fwd_rows(rows=R), bwd_rows(rows=R) and dkdv_keys(keys=K)
decode each flat index into (b, h, t) or (b, hkv, j) and write result i at
slot i.  They are tied to the full call (rows / keys omitted), which the dense
autograd pin of test_oracle_pins.py ties to the definition, on irregular R and
K: unsorted, repeated, spanning several batch entries and heads.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _irregular_lists(rng, Hkv, L, bs, S, nb_other):
    """Own block + random earlier blocks of one sequence of L tokens, then
    sprinkled with: -1 and other negatives in any slot, repeats, blocks past
    this sequence's end that would be valid in a longer sequence (nb_other),
    future blocks, and one row listing nothing."""
    idx = workloads.block_idx_own_random(rng, Hkv, L, bs, S)
    if L == 0:
        return idx
    NB = -(-L // bs)
    flat = idx.reshape(-1, S)
    n = flat.shape[0]
    for r in rng.choice(n, size=max(1, n // 3), replace=False):
        s = rng.integers(0, S)
        kind = rng.integers(0, 5)
        if kind == 0:
            flat[r, s] = -1 if rng.random() < 0.5 else -3
        elif kind == 1:
            flat[r, s] = flat[r, 0]
        elif kind == 2:
            flat[r, s] = NB + rng.integers(0, max(1, nb_other - NB + 1))
        else:
            flat[r, s] = rng.integers(0, NB)
    flat[rng.integers(0, n)] = -1
    return idx


def _packed_case(seed, lengths, Hq, Hkv, D, bs, S):
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    Tt = int(cu[-1])
    q = rng.standard_normal((Tt, Hq, D))
    k = rng.standard_normal((Tt, Hkv, D))
    v = rng.standard_normal((Tt, Hkv, D))
    nb_max = -(-max(lengths) // bs)
    idx = np.full((Hkv, Tt, S), -1, dtype=np.int32)
    for z, L in enumerate(lengths):
        idx[:, cu[z]:cu[z + 1]] = _irregular_lists(rng, Hkv, L, bs, S, nb_max)
    dO = rng.standard_normal((Tt, Hq, D))
    return q, k, v, idx, dO, cu


def _packed_mask(idx, cu, bs, Hq):
    """[Hq, Ttot, Ttot] visibility: query t sees key j iff both lie in the
    same sequence, j <= t, and t's row lists j's sequence-local block (a
    block number in [0, ceil(len / bs)) of that sequence)."""
    Hkv, Tt, S = idx.shape
    G = Hq // Hkv
    m = np.zeros((Hkv, Tt, Tt), dtype=bool)
    for z in range(len(cu) - 1):
        a, b = int(cu[z]), int(cu[z + 1])
        nb = -(-(b - a) // bs)
        for h in range(Hkv):
            for t in range(a, b):
                listed = {int(u) for u in idx[h, t] if 0 <= u < nb}
                for j in range(a, t + 1):
                    m[h, t, j] = (j - a) // bs in listed
    return np.repeat(m, G, axis=0)


def _packed_autograd(q, k, v, dO, idx, cu, bs, scale):
    """o [Ttot,Hq,D], lse [Hq,Ttot] and dq/dk/dv of the whole packed batch as
    one masked softmax per head (library logsumexp, torch autograd)."""
    Tt, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    mask = torch.from_numpy(_packed_mask(idx, cu, bs, Hq))
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    qh = qt.permute(1, 0, 2)
    kh = kt.permute(1, 0, 2).repeat_interleave(G, dim=0)
    vh = vt.permute(1, 0, 2).repeat_interleave(G, dim=0)
    s = scale * torch.matmul(qh, kh.transpose(-1, -2).contiguous())
    s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    lse_safe = torch.where(torch.isinf(lse), torch.zeros_like(lse), lse)
    p = torch.exp(s - lse_safe[..., None])
    o = torch.matmul(p, vh).permute(1, 0, 2)
    o.backward(torch.tensor(dO))
    return (o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(),
            vt.grad.numpy())


PACKED = [
    dict(seed=1, lengths=[10, 0, 17, 6, 13], Hq=4, Hkv=2, D=5, bs=4, S=4),   # G=2, empty seq
    dict(seed=2, lengths=[9, 22, 3], Hq=3, Hkv=1, D=4, bs=5, S=3),           # G=3, ragged tails
    dict(seed=3, lengths=[16, 1, 11], Hq=2, Hkv=2, D=6, bs=2, S=6),          # G=1, S > NB
]


@pytest.mark.parametrize("c", PACKED)
def test_packed_batch_equals_block_diagonal_autograd(c):
    """fwd_thd / bwd_thd (one dense call per sequence) equal one unsplit
    block-diagonal masked softmax over the packed batch, differentiated by
    torch autograd in float64: o, lse, dq, dk, dv, and Delta = <dO, o>."""
    q, k, v, idx, dO, cu = _packed_case(**c)
    bs = c["bs"]
    scale = c["D"] ** -0.5
    o, lse = oracle.fwd_thd(q, k, v, idx, cu, bs)
    dq, dk, dv, lse2, delta = oracle.bwd_thd(q, k, v, dO, idx, cu, bs)
    o_r, lse_r, dq_r, dk_r, dv_r = _packed_autograd(q, k, v, dO, idx, cu, bs, scale)
    empty = np.isinf(lse_r)
    assert empty.any() and not empty.all()          # the case holds empty rows
    assert np.array_equal(np.isinf(lse), empty) and np.array_equal(np.isinf(lse2), empty)
    np.testing.assert_allclose(lse[~empty], lse_r[~empty], atol=1e-12, rtol=0)
    np.testing.assert_array_equal(lse, lse2)
    np.testing.assert_allclose(o, o_r, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, dq_r, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, dk_r, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, dv_r, atol=1e-12, rtol=0)
    np.testing.assert_allclose(delta, np.sum(dO * o, axis=-1).T, atol=1e-12, rtol=0)
    assert np.abs(dk).max() > 1e-3 and np.abs(dq).max() > 1e-3  # not vacuous


def test_packed_backward_isolation():
    """Changing one sequence's q, k, v and dO leaves every output of the
    other sequences (dq, dk, dv, lse, Delta) bitwise unchanged, and moves
    that sequence's."""
    q, k, v, idx, dO, cu = _packed_case(**PACKED[0])
    bs = PACKED[0]["bs"]
    base = oracle.bwd_thd(q, k, v, dO, idx, cu, bs)
    z = 2
    a, b = int(cu[z]), int(cu[z + 1])
    rng = np.random.default_rng(17)
    q2, k2, v2, dO2 = q.copy(), k.copy(), v.copy(), dO.copy()
    for x in (q2, k2, v2, dO2):
        x[a:b] += rng.standard_normal(x[a:b].shape)
    alt = oracle.bwd_thd(q2, k2, v2, dO2, idx, cu, bs)
    for name, x, y in zip(("dq", "dk", "dv"), base[:3], alt[:3]):
        np.testing.assert_array_equal(x[:a], y[:a], err_msg=name)
        np.testing.assert_array_equal(x[b:], y[b:], err_msg=name)
        assert np.abs(x[a:b] - y[a:b]).max() > 1e-3, name
    for name, x, y in zip(("lse", "delta"), base[3:], alt[3:]):
        np.testing.assert_array_equal(x[:, :a], y[:, :a], err_msg=name)
        np.testing.assert_array_equal(x[:, b:], y[:, b:], err_msg=name)


def _dense_case(seed=5, B=2, Hq=6, Hkv=2, T=21, D=4, bs=4, S=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    idx = np.stack([_irregular_lists(rng, Hkv, T, bs, S, -(-T // bs)) for _ in range(B)])
    dO = rng.standard_normal((B, Hq, T, D))
    return q, k, v, idx, dO, bs


def test_row_and_key_subsets_equal_full_call():
    """fwd_rows / bwd_rows with a row list and dkdv_keys with a key list
    return, at slot i, the full call's entry for row / key i of the list:
    unsorted lists with repeats across both batch entries and every head."""
    q, k, v, idx, dO, bs = _dense_case()
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    rng = np.random.default_rng(23)
    o_all, lse_all = oracle.fwd_rows(q, k, v, idx, bs)
    lse_b, delta_all, dq_all = oracle.bwd_rows(q, k, v, dO, idx, bs)
    dk_all, dv_all = oracle.dkdv_keys(q, k, v, dO, idx, bs, lse_b, delta_all)
    n_rows, n_keys = B * Hq * T, B * Hkv * T
    rows = rng.permutation(n_rows)[:n_rows // 3]
    rows = np.concatenate([rows, rows[:5], [n_rows - 1, 0]])     # repeats, both ends
    keys = rng.permutation(n_keys)[:n_keys // 3]
    keys = np.concatenate([keys, keys[:4], [n_keys - 1, 0]])
    # the lists touch every batch entry and head
    assert len(set((rows // T) % Hq)) == Hq and len(set(rows // (T * Hq))) == B
    assert len(set((keys // T) % Hkv)) == Hkv and len(set(keys // (T * Hkv))) == B
    o, lse = oracle.fwd_rows(q, k, v, idx, bs, rows)
    lse2, delta, dq = oracle.bwd_rows(q, k, v, dO, idx, bs, rows)
    dk, dv = oracle.dkdv_keys(q, k, v, dO, idx, bs, lse_b, delta_all, keys)
    np.testing.assert_array_equal(o, o_all[rows])
    np.testing.assert_array_equal(lse, lse_all[rows])
    np.testing.assert_array_equal(lse2, lse_b[rows])
    np.testing.assert_array_equal(delta, delta_all[rows])
    np.testing.assert_array_equal(dq, dq_all[rows])
    np.testing.assert_array_equal(dk, dk_all[keys])
    np.testing.assert_array_equal(dv, dv_all[keys])
    # the full call's flat order is (b, h, t) / (b, hkv, j): ties the decode
    # to the dense layout the other pins use
    o4, _ = oracle.fwd(q, k, v, idx, bs)
    dq4, dk4, dv4, _, _ = oracle.bwd(q, k, v, dO, idx, bs)
    np.testing.assert_array_equal(o_all.reshape(B, Hq, T, D), o4)
    np.testing.assert_array_equal(dq_all.reshape(B, Hq, T, D), dq4)
    np.testing.assert_array_equal(dk_all.reshape(B, Hkv, T, D), dk4)
    np.testing.assert_array_equal(dv_all.reshape(B, Hkv, T, D), dv4)
