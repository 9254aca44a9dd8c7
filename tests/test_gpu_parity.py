"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs.  Gates are page 1's max-abs tolerances (2e-3 fp32,
6e-2 bf16) applied to o, lse, dq, dk, dv; the block -> query inversion is
compared bit for bit."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads
from _harness import (TOL, assert_close, gpu_keys, gpu_rows, oracle_block_keys, oracle_full,
                      oracle_rows, run_gpu, say, to_dev)

pytestmark = pytest.mark.gpu


def _full_parity(w):
    tol = TOL[w.dtype]
    say(f"[{w.name}] dtype={w.dtype} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"S={w.S} bs={w.block_size} packed={w.packed}")
    got = run_gpu(w)
    ref = oracle_full(w)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, got[name], ref[name], tol)


@pytest.mark.parametrize("name", ["f32_T256", "bf16_T1024"])
def test_small_workloads_full(name):
    """The f32 T 256 (G=2, D32, bs16) and bf16 T 1024 (G=3, D64, bs32) workloads: every
    output element against the oracle."""
    _full_parity(workloads.make_workload(name))


def _weird_block_idx(rng, B, Hkv, T, bs, S):
    """Random own+earlier lists sprinkled with -1 anywhere, other negatives,
    duplicates, out-of-range blocks, future blocks and fully empty rows."""
    NB = -(-T // bs)
    idx = np.stack([workloads.block_idx_own_random(rng, Hkv, T, bs, S) for _ in range(B)])
    flat = idx.reshape(-1, S)
    n = flat.shape[0]
    sel = rng.random(n) < 0.3
    for r in np.nonzero(sel)[0]:
        s = rng.integers(0, S)
        kind = rng.integers(0, 5)
        flat[r, s] = [-1, -5, flat[r, 0], NB + 3, rng.integers(0, NB)][kind]
    flat[rng.choice(n, size=max(1, n // 50), replace=False)] = -1
    return idx


@pytest.mark.parametrize("case", [
    dict(name="G1-D64-bs64", B=2, Hq=2, Hkv=2, T=700, D=64, S=5, bs=64),
    dict(name="G4-D128-bs32-ragged", B=1, Hq=8, Hkv=2, T=333, D=128, S=6, bs=32),
    dict(name="G3-D32-bs128", B=1, Hq=6, Hkv=2, T=520, D=32, S=3, bs=128),
    dict(name="G16-D128-bs64", B=1, Hq=32, Hkv=2, T=450, D=128, S=4, bs=64),
    dict(name="G32-D64-bs64", B=1, Hq=32, Hkv=1, T=300, D=64, S=3, bs=64),
    dict(name="G6-D64-bs32", B=1, Hq=12, Hkv=2, T=200, D=64, S=4, bs=32),
])
def test_bf16_shapes_with_irregular_lists(case):
    """Tiles and ragged tails: G = 1, 3, 4, 6, 16, 32; D 32/64/128; bs
    32/64/128; T not a multiple of bs; lists with -1 anywhere, duplicates,
    out-of-range and future blocks, empty rows; S > valid count."""
    rng = np.random.default_rng(7)
    c = dict(case)
    name = c.pop("name")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], c["bs"], c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=11, name=name, block_idx=idx)
    _full_parity(w)


def test_f32_irregular_lists_packed():
    """fp32 path on packed sequences (one of length 0, ragged lengths) with
    irregular lists."""
    rng = np.random.default_rng(8)
    w = workloads.make_thd([40, 0, 77, 16], 4, 2, 32, 3, 16, "f32", "own_random", seed=4,
                           name="f32-packed")
    for z in range(4):
        a, b = w.cu_seqlens[z], w.cu_seqlens[z + 1]
        if b > a:
            part = _weird_block_idx(rng, 1, 2, int(b - a), 16, 3)[0]
            w.block_idx[:, a:b] = part
    _full_parity(w)


def _idx_counts_brute(groups, bs):
    """Padding, out-of-range, future and repeated entries of block lists,
    counted row by row in plain Python: groups yields (rows [L, S], L)."""
    c = [0, 0, 0, 0]
    for rows, L in groups:
        nb = -(-L // bs)
        for t in range(L):
            seen = set()
            for u in rows[t].tolist():
                if u < 0:
                    c[0] += 1
                elif u >= nb:
                    c[1] += 1
                else:
                    c[2] += u * bs > t
                    c[3] += u in seen
                    seen.add(u)
    return dict(zip(("padding", "out_of_range", "future", "repeated"), c))


def test_check_block_idx_counts_exact():
    """nsa_sel_check_block_idx against a brute-force count, dense and packed
    (empty sequence included), on lists with -1 and other negatives anywhere,
    repeats, out-of-range and future blocks; S > 64 covers several passes of
    a row.  (f32 problems: they take any block size.)"""
    rng = np.random.default_rng(21)
    for B, Hkv, T, bs, S in ((2, 2, 300, 32, 6), (1, 1, 200, 16, 70)):
        idx = _weird_block_idx(rng, B, Hkv, T, bs, S)
        w = workloads.make_dense(B, 2 * Hkv, Hkv, T, 32, S, bs, "f32", seed=3, block_idx=idx)
        d = to_dev(w)
        got = nsa.nsa_sel_check_block_idx(d["q"], d["k"], d["idx"], bs)
        want = _idx_counts_brute(((idx[b, h], T) for b in range(B) for h in range(Hkv)), bs)
        say(f"[check dense B{B} T{T} S{S}] {got}")
        assert got == want and all(v > 0 for v in want.values())
    w = workloads.make_thd([90, 0, 130, 7], 4, 2, 32, 5, 16, "f32", "own_random", seed=4,
                           name="chk-packed")
    for z in range(4):
        a, b = w.cu_seqlens[z], w.cu_seqlens[z + 1]
        if b > a:
            w.block_idx[:, a:b] = _weird_block_idx(rng, 1, 2, int(b - a), 16, 5)[0]
    d = to_dev(w)
    got = nsa.nsa_sel_check_block_idx(d["q"], d["k"], d["idx"], 16, d["cu"], w.max_seqlen)
    groups = ((w.block_idx[h, w.cu_seqlens[z]:w.cu_seqlens[z + 1]],
               int(w.cu_seqlens[z + 1] - w.cu_seqlens[z])) for z in range(4) for h in range(2))
    want = _idx_counts_brute(groups, 16)
    say(f"[check packed] {got}")
    assert got == want


def test_bf16_packed_small_d64():
    """Packed bf16 at D=64 (page 3's review: a packed backward built for the
    wrong head dimension wrote out of bounds) with ragged lengths."""
    w = workloads.make_thd([64, 200, 5, 130], 8, 2, 64, 6, 32, "bf16", "own_first_random",
                           seed=5, name="thd-d64")
    _full_parity(w)


def test_packed_different_totals_same_count():
    """Two packed draws with the same number of sequences but different token
    totals both match the oracle (page 3's review asks for genuinely different
    totals and checked gradients)."""
    for lens in ([96, 160], [64, 256]):
        w = workloads.make_thd(lens, 4, 1, 128, 4, 64, "bf16", "own_first_random", seed=6,
                               name=f"thd-{lens}")
        _full_parity(w)



def test_bf16_packed_many_and_empty_sequences():
    """Packed bf16 with empty sequences among short ones, both with at most 64
    sequences (the order of non-empty windows is computed per wave from the
    lengths) and with more (every window of every sequence in turn)."""
    rng = np.random.default_rng(12)
    for n_seq in (12, 70):
        lens = [int(x) for x in rng.integers(0, 97, size=n_seq)]
        lens[0] = 0
        lens[n_seq // 2] = 0
        lens[-1] = 160
        w = workloads.make_thd(lens, 4, 2, 64, 4, 32, "bf16", "own_first_random", seed=13,
                               name=f"thd-{n_seq}-seqs")
        _full_parity(w)


@pytest.mark.parametrize("case", [
    dict(name="prefix-G4-D128-bs64", B=1, Hq=8, Hkv=2, T=300, D=128, S=5, bs=64),
    dict(name="prefix-G2-D64-bs128", B=2, Hq=4, Hkv=2, T=250, D=64, S=2, bs=128),
])
def test_bf16_whole_prefix_selection(case):
    """Selections that can cover a token's whole causal prefix (S * block_size
    >= T: forward and dQ take the walk with a barrier per job), with irregular
    lists."""
    rng = np.random.default_rng(14)
    c = dict(case)
    name = c.pop("name")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], c["bs"], c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=15, name=name, block_idx=idx)
    _full_parity(w)

@pytest.mark.parametrize("case", [
    dict(name="full-G4-D128-bs64", B=2, Hq=8, Hkv=2, T=250, D=128, bs=64),
    dict(name="full-G3-D64-bs32-odd", B=1, Hq=6, Hkv=2, T=330, D=64, bs=32),
    dict(name="full-G2-D128-bs64-odd", B=1, Hq=4, Hkv=2, T=400, D=128, bs=64),
    dict(name="full-G16-D32-bs64-one", B=1, Hq=16, Hkv=1, T=60, D=32, bs=64),
])
def test_bf16_full_prefix_pairs(case):
    """Every row lists every block up to its own (dense causal, -1 beyond) and
    every list fits one work item (T * G <= 1024 here): the dK/dV stage runs
    on pairs of blocks.  Ragged T, an odd number of blocks (the last pair
    holds one block), a single block, and the same problem with one entry
    removed (not a whole prefix any more: the per-block launch runs)."""
    c = dict(case)
    name = c.pop("name")
    B, Hkv, T, bs = c["B"], c["Hkv"], c["T"], c["bs"]
    NB = -(-T // bs)
    S = NB
    t = np.arange(T)
    idx = np.where(np.arange(S)[None, :] <= (t // bs)[:, None], np.arange(S)[None, :], -1)
    idx = np.broadcast_to(idx, (B, Hkv, T, S)).astype(np.int32).copy()
    w = workloads.make_dense(B, c["Hq"], Hkv, T, c["D"], S, bs, "bf16", seed=16, name=name,
                             block_idx=idx)
    _full_parity(w)
    idx2 = idx.copy()
    idx2[0, 0, T - 1, 0] = -1  # the last token no longer lists block 0
    w2 = workloads.make_dense(B, c["Hq"], Hkv, T, c["D"], S, bs, "bf16", seed=16,
                              name=name + "-holed", block_idx=idx2)
    _full_parity(w2)


# ---- sampled outputs + invariants (used where the oracle cannot do every row) ----

def _sampled_parity(w, out, rng, n_rows=48, blocks=None):
    tol = TOL[w.dtype]
    G = w.Hq // w.Hkv
    Z = w.n_seqs
    errs = {"o": 0.0, "lse": 0.0, "dq": 0.0}
    for _ in range(6):
        z = int(rng.integers(0, Z))
        if w.packed:
            L = int(w.cu_seqlens[z + 1] - w.cu_seqlens[z])
        else:
            L = w.T
        if L == 0:
            continue
        h = int(rng.integers(0, w.Hq))
        t = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, size=n_rows // 6)]))
        o_r, lse_r, dq_r = oracle_rows(w, z, h, t)
        o_g, lse_g, dq_g = gpu_rows(w, out, z, h, t)
        for name, a, b in (("o", o_g, o_r), ("lse", lse_g, lse_r), ("dq", dq_g, dq_r)):
            errs[name] = max(errs[name], float(np.max(np.abs(a - b))))
    for name, e in errs.items():
        say(f"  sampled {name}: max|err| = {e:.3e} (tol {tol:g})")
        assert e <= tol, (name, e)
    for (z, hkv, u) in blocks:
        j, dk_r, dv_r, ntok = oracle_block_keys(w, z, hkv, u)
        dk_g, dv_g = gpu_keys(w, out, z, hkv, j)
        e1, e2 = float(np.max(np.abs(dk_g - dk_r))), float(np.max(np.abs(dv_g - dv_r)))
        say(f"  block (z={z}, hkv={hkv}, u={u}) rows={ntok * G}: dk err {e1:.3e} "
            f"(max|dk| {np.abs(dk_r).max():.3g}), dv err {e2:.3e}")
        assert e1 <= tol and e2 <= tol


def _invariants(w, out, d):
    """Sum over keys of dk is 0 per (entry, KV head); sum of dv equals the sum
    of dO over the group's rows (every row here has its own block)."""
    G = w.Hq // w.Hkv
    if w.packed:
        segs = [(int(w.cu_seqlens[z]), int(w.cu_seqlens[z + 1])) for z in range(w.n_seqs)]
        for a, b in segs[:3]:
            sdk = out["dk"][a:b].sum(axis=0)
            sdv = out["dv"][a:b].sum(axis=0)
            sdo = w.dO[a:b].astype(np.float64).reshape(b - a, w.Hkv, G, w.D).sum(axis=(0, 2))
            scale = np.abs(out["dk"][a:b]).max()
            say(f"  seq [{a},{b}): |sum dk| {np.abs(sdk).max():.3e} (max|dk| {scale:.3g}), "
                f"|sum dv - sum dO| {np.abs(sdv - sdo).max():.3e}")
            assert np.abs(sdk).max() < 1e-2 * (b - a) ** 0.5 * max(scale, 1)
            assert np.abs(sdv - sdo).max() < 1e-2 * (b - a) ** 0.5 * G
    else:
        sdk = out["dk"].sum(axis=2)
        sdv = out["dv"].sum(axis=2)
        sdo = w.dO.astype(np.float64).reshape(w.B, w.Hkv, G, w.T, w.D).sum(axis=(2, 3))
        say(f"  |sum dk| {np.abs(sdk).max():.3e}, |sum dv - sum dO| {np.abs(sdv - sdo).max():.3e}")
        assert np.abs(sdk).max() < 1e-2 * w.T ** 0.5 * max(np.abs(out["dk"]).max(), 1)
        assert np.abs(sdv - sdo).max() < 1e-2 * w.T ** 0.5 * G


@pytest.mark.parametrize("name", ["select_T8192", "causal_B4_T4096", "packed_8seq"])
def test_full_size_workloads_elementwise(name):
    """The three D128 workloads at full size, in the launch configuration the
    benchmark times: every element of o, lse, dq, dk and dv against the
    float64 oracle on the same seeded draw (page 1's gate: max-abs error over
    whole tensors), plus the sum invariants over every key.  Block 0 of the
    first-block workloads is listed by every row (the longest lists, split
    into the most fp32 partials)."""
    w = workloads.make_workload(name)
    say(f"[{name}] full size: B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} S={w.S} "
        f"bs={w.block_size} packed={w.packed}")
    d = to_dev(w)
    got = run_gpu(w, d)
    for key in got:
        assert np.isfinite(got[key][~np.isinf(got[key])]).all(), key
    ref = oracle_full(w)
    tol = TOL[w.dtype]
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert_close(key, got[key], ref[key], tol)
    # block 0 of every (entry, KV head) on its own: the largest reductions
    dk0, dv0 = got["dk"], got["dv"]
    if w.packed:
        parts = [(slice(int(w.cu_seqlens[z]), int(w.cu_seqlens[z]) + w.block_size),)
                 for z in range(w.n_seqs)]
        e = max(float(np.abs(dk0[p] - ref["dk"][p]).max()) for p in parts)
    else:
        sl = (slice(None), slice(None), slice(0, w.block_size))
        e = float(np.abs(dk0[sl] - ref["dk"][sl]).max())
    say(f"  block 0 dk: max|err| = {e:.3e}")
    assert e <= tol
    _invariants(w, got, d)


# ---- inversion: bit-exact -----------------------------------------------

def _inversion_matches(w, window=0):
    d = to_dev(w)
    ms = w.max_seqlen if w.packed else None
    offsets, tokens = nsa.nsa_sel_invert(d["q"], d["k"], d["idx"], w.block_size, d["cu"], ms,
                                         window=window)
    torch.cuda.synchronize()
    offsets = offsets.cpu().numpy()
    tokens = tokens.cpu().numpy()
    Smin = min(w.S, max(1, -(-(w.max_seqlen if w.packed else w.T) // w.block_size)))
    n_checked = 0
    for z in range(w.n_seqs):
        if w.packed:
            a, b = int(w.cu_seqlens[z]), int(w.cu_seqlens[z + 1])
            idx_z = np.ascontiguousarray(w.block_idx[:, a:b])[None]
        else:
            idx_z = w.block_idx[z:z + 1]
        counts, ref = oracle.invert(idx_z, w.block_size, window)
        L = idx_z.shape[2]
        NBz = -(-L // w.block_size)
        pos = 0
        for hkv in range(w.Hkv):
            r0 = (hkv * w.T + a) if w.packed else ((z * w.Hkv + hkv) * w.T)
            base = Smin * r0
            off = offsets[z, hkv]
            assert off[0] == 0
            for u in range(offsets.shape[2] - 1):
                c = int(counts[0, hkv, u]) if u < NBz else 0
                assert off[u + 1] - off[u] == c, (z, hkv, u)
                got = tokens[base + off[u]: base + off[u + 1]]
                np.testing.assert_array_equal(got, ref[pos:pos + c])
                pos += c
                n_checked += c
    say(f"  inversion: {n_checked} entries bit-exact")


def test_inversion_bit_exact_dense_irregular():
    rng = np.random.default_rng(3)
    idx = _weird_block_idx(rng, 2, 3, 777, 32, 9)
    w = workloads.make_dense(2, 3, 3, 777, 32, 9, 32, "bf16", block_idx=idx, name="inv")
    _inversion_matches(w)


@pytest.mark.parametrize("name", ["bf16_T1024", "select_T8192", "packed_8seq"])
def test_inversion_bit_exact_workloads(name):
    _inversion_matches(workloads.make_workload(name))


@pytest.mark.parametrize("name,window", [("bf16_T1024", 100), ("packed_8seq", 700)])
def test_inversion_bit_exact_with_window(name, window):
    """With a sliding window only rows whose window reaches the block are
    listed (dense and packed)."""
    _inversion_matches(workloads.make_workload(name), window)


# ---- masking sentinels: bitwise ------------------------------------------

def test_hidden_keys_do_not_move_rows_bitwise():
    """Rows' o, lse and dq are bitwise unchanged when K/V change at keys the
    rows must not see: unlisted blocks, keys after t in the own block, keys
    aliased by -1 or out-of-range entries.  dk/dv of keys no row attends to
    are exactly zero."""
    T, bs, S, Hq, Hkv, D = 256, 64, 3, 8, 2, 64
    idx = np.full((1, Hkv, T, S), -1, np.int32)
    idx[0, :, :, 0] = np.arange(T) // bs          # own block
    idx[0, :, 128:, 1] = 0                        # tokens >= 128 also see block 0
    idx[0, :, 128:, 2] = 99                       # out of range: ignored
    w = workloads.make_dense(1, Hq, Hkv, T, D, S, bs, "bf16", seed=2, block_idx=idx, name="sent")
    base = run_gpu(w)
    # keys of block 1 are seen only by tokens 64..127; block 0 by 0..63 and 128..255
    w2 = workloads.make_dense(1, Hq, Hkv, T, D, S, bs, "bf16", seed=2, block_idx=idx, name="sent2")
    rng = np.random.default_rng(0)
    w2.k[0, :, 64:128] = workloads.round_to_bf16(rng.standard_normal(w2.k[0, :, 64:128].shape).astype(np.float32))
    w2.v[0, :, 64:128] = workloads.round_to_bf16(rng.standard_normal(w2.v[0, :, 64:128].shape).astype(np.float32))
    w2.k[0, :, 200:] += 1.0
    w2.v[0, :, 200:] -= 1.0
    alt = run_gpu(w2)
    # tokens 0..63 see only block 0 -> unchanged; tokens 128..199 see block 0 and own
    # keys <= t (< 200) -> unchanged
    for sl in (slice(0, 64), slice(128, 200)):
        for name in ("o", "lse", "dq"):
            a, b = base[name][0, :, sl], alt[name][0, :, sl]
            assert np.array_equal(a, b), (name, sl)
    assert not np.array_equal(base["o"][0, :, 64:128], alt["o"][0, :, 64:128])
    # nobody attends keys of block 1 except tokens 64..127 via own block; keys
    # j > t inside own blocks are masked, so the last key of the sequence is
    # attended only by token 255 itself.
    idx2 = idx.copy()
    idx2[0, :, 64:128, 0] = -1                    # block 1 listed by nobody
    w3 = workloads.make_dense(1, Hq, Hkv, T, D, S, bs, "bf16", seed=2, block_idx=idx2, name="sent3")
    out3 = run_gpu(w3)
    assert np.all(out3["dk"][0, :, 64:128] == 0.0) and np.all(out3["dv"][0, :, 64:128] == 0.0)
    assert np.all(out3["o"][0, :, 64:128] == 0.0)
    assert np.all(np.isneginf(out3["lse"][0, :, 64:128]))
    assert np.all(out3["dq"][0, :, 64:128] == 0.0)


@pytest.mark.parametrize("G", [4, 16])
def test_packed_sequences_isolated_bitwise(G):
    """Packed sequences do not see each other: changing every input (q, k,
    v, dO) of one sequence leaves o, lse, dq, dk and dv of the other
    sequences bitwise unchanged, and moves that sequence's outputs."""
    lens = [200, 96, 333, 64, 150]
    w = workloads.make_thd(lens, 2 * G, 2, 128, 8, 64, "bf16", "own_first_random", seed=41,
                           name=f"iso-G{G}")
    base = run_gpu(w)
    z = 2
    a, b = int(w.cu_seqlens[z]), int(w.cu_seqlens[z + 1])
    rng = np.random.default_rng(42)
    for x in (w.q, w.k, w.v, w.dO):
        x[a:b] = workloads.round_to_bf16(rng.standard_normal(x[a:b].shape).astype(np.float32))
    alt = run_gpu(w)
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(base[name][:a], alt[name][:a]), name
        assert np.array_equal(base[name][b:], alt[name][b:]), name
        assert np.abs(base[name][a:b] - alt[name][a:b]).max() > 1e-2, name
    assert np.array_equal(base["lse"][:, :a], alt["lse"][:, :a])
    assert np.array_equal(base["lse"][:, b:], alt["lse"][:, b:])
    say(f"  [iso-G{G}] sequences other than {z} bitwise unchanged")


@pytest.mark.parametrize("name", ["select_T8192", "causal_B4_T4096"])
def test_deterministic_bitwise(name):
    """Two full passes give identical bits (NSA lists with fp32 partials; the
    dense causal workload on the paired dK/dV path with its flag and iota
    lists rebuilt by each call)."""
    w = workloads.make_workload(name)
    d = to_dev(w)
    a = run_gpu(w, d)
    b = run_gpu(w, d)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name", ["bf16_T1024", "select_T8192", "causal_B4_T4096", "packed_8seq"])
def test_staged_backward_equals_one_call(name):
    """prepare, dkdv_blocks, dkdv_reduce, dq in order equal nsa_sel_bwd bit for
    bit (the T 8192, G 16 workload has lists long enough to be split into fp32
    partials, and its dQ takes over the dK/dV kernel's dS)."""
    w = workloads.make_workload(name)
    d = to_dev(w)
    cu = d.get("cu")
    ms = w.max_seqlen if w.packed else None
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms)
    dq, dk, dv = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                                 w.scale, cu, ms)
    st = nsa.BwdStages(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms)
    st.prepare(o, d["dO"])
    st.dkdv_blocks(d["dO"], lse)
    dk2, dv2 = st.dkdv_reduce()
    dq2 = st.dq_stage(d["dO"], lse)
    torch.cuda.synchronize()
    for a, b, n in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a, b), n


@pytest.mark.parametrize("name", ["select_T8192", "causal_B4_T4096", "packed_8seq"])
def test_two_stream_schedule_equals_one_call(name):
    """The inversion on a second stream beside the forward, and the dK/dV
    reduce beside dQ, equal nsa_sel_bwd bit for bit, over three steps that
    reuse one workspace (the order the two-stream step of the benchmark uses)."""
    w = workloads.make_workload(name)
    d = to_dev(w)
    cu = d.get("cu")
    ms = w.max_seqlen if w.packed else None
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms)
    dq, dk, dv = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                                 w.scale, cu, ms)
    torch.cuda.synchronize()
    st = nsa.BwdStages(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    for it in range(3):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            st.prepare_lists()
        nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms,
                        out=o2, lse=lse2)
        st.prepare_delta(o2, d["dO"])
        main.wait_stream(side)
        st.dkdv_blocks(d["dO"], lse2)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            dk2, dv2 = st.dkdv_reduce()
        dq2 = st.dq_stage(d["dO"], lse2)
        main.wait_stream(side)
        torch.cuda.synchronize()
        for a, b, n in ((o, o2, "o"), (lse, lse2, "lse"), (dq, dq2, "dq"), (dk, dk2, "dk"),
                        (dv, dv2, "dv")):
            assert torch.equal(a, b), f"step {it}: {n}"


def test_runs_on_caller_stream():
    """All work is queued on the caller's (non-default) stream."""
    w = workloads.make_workload("bf16_T1024")
    d = to_dev(w)
    ref = run_gpu(w, d)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale)
        dq, dk, dv = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"],
                                     w.block_size, w.scale)
    s.synchronize()
    assert np.array_equal(dk.float().cpu().numpy(), ref["dk"])
    assert np.array_equal(o.float().cpu().numpy(), ref["o"])


def test_empty_problem():
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, 1, 0, 64, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(1, 1, 0, 4, dtype=torch.int32, device="cuda")
    o, lse = nsa.nsa_sel_fwd(q, k, k, idx, 64)
    dq, dk, dv = nsa.nsa_sel_bwd(q, k, k, o, lse, q, idx, 64)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dk.numel() == 0


def test_autograd_function():
    """selection_attn's autograd gradients equal the direct C-ABI calls."""
    w = workloads.make_workload("bf16_T1024")
    d = to_dev(w)
    ref = run_gpu(w, d)
    q, k, v = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = nsa.selection_attn(q, k, v, d["idx"], w.block_size)
    o.backward(d["dO"])
    torch.cuda.synchronize()
    assert np.array_equal(q.grad.float().cpu().numpy(), ref["dq"])
    assert np.array_equal(k.grad.float().cpu().numpy(), ref["dk"])
