"""GPU parity on a seeded mix of small problems that combine the options the
other files test one at a time: dtype, group size (the dS hand-off's 4-, 8-
and 16-head tiles and the recomputing dQ), head dimension, 16- to 128-key
blocks, more keys than queries, sliding windows, packed sequences, and
irregular lists (-1 anywhere, repeats, out-of-range and future blocks,
empty rows).  Every output element against the float64 oracle at page 1's
gates, which assume unit-scale values (its pass rule is atol + rtol * 1):
where a draw makes an output larger (short windows concentrate P, so dv
can reach ~20), each bf16 element's gate adds its own output rounding,
|err| <= atol + 2^-8 |ref| (half a bf16 ulp is at most 2^-9 |x|)."""
import numpy as np
import pytest

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads
from _harness import TOL, say, to_dev
from test_gpu_parity import _weird_block_idx
from test_gpu_window import _run

pytestmark = pytest.mark.gpu


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = "f32" if i % 5 == 4 else "bf16"
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    Hkv = int(rng.integers(1, 3))
    D = int(rng.choice([32, 64, 128]))
    bs = int(rng.choice([16, 32, 64, 128] if dtype == "bf16" else [8, 16, 32]))
    S = int(rng.integers(1, 9))
    W = int(rng.choice([0, 0, 0, int(rng.integers(1, 200))]))
    packed = i % 4 == 3
    if packed:
        lens = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 5)))]
        w = workloads.make_thd(lens, G * Hkv, Hkv, D, S, bs, dtype, "own_first_random",
                               seed=2000 + i, name=f"mix{i}")
        return w, W
    T = int(rng.integers(1, 400))
    Tk = T + int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    B = int(rng.integers(1, 3))
    full = _weird_block_idx(rng, B, Hkv, Tk, bs, S)
    idx = np.ascontiguousarray(full[:, :, Tk - T:])
    w = workloads.make_dense(B, G * Hkv, Hkv, T, D, S, bs, dtype, seed=2000 + i, name=f"mix{i}",
                             block_idx=idx, Tk=Tk)
    return w, W


@pytest.mark.parametrize("i", range(24))
def test_mixed_problem(i):
    w, W = _draw(i)
    Tk = w.k.shape[2] if not w.packed else w.T
    say(f"[{w.name}] dtype={w.dtype} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} Tk={Tk} D={w.D} "
        f"S={w.S} bs={w.block_size} window={W} packed={w.packed}")
    d = to_dev(w)
    ms = w.max_seqlen if w.packed else None
    p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale, d["cu"], ms, W)
    say(f"  dS hand-off: {nsa.ds_handoff(p)}")
    got = _run(w, W, d)
    if w.packed:
        o, lse = oracle.fwd_thd(w.q, w.k, w.v, w.block_idx, w.cu_seqlens, w.block_size, w.scale,
                                window=W)
        dq, dk, dv, _, _ = oracle.bwd_thd(w.q, w.k, w.v, w.dO, w.block_idx, w.cu_seqlens,
                                          w.block_size, w.scale, window=W)
    else:
        o, lse = oracle.fwd(w.q, w.k, w.v, w.block_idx, w.block_size, w.scale, window=W)
        dq, dk, dv, _, _ = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, w.block_size, w.scale,
                                      window=W)
    ref = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    rel = 2.0 ** -8 if w.dtype == "bf16" else 0.0
    for name in ("o", "lse", "dq", "dk", "dv"):
        a, b = got[name], ref[name]
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin), f"{name}: infinities differ"
        err = np.abs(a[fin] - b[fin])
        gate = TOL[w.dtype] + rel * np.abs(b[fin])
        worst = float((err - gate).max()) if err.size else -1.0
        say(f"  {name}: max|err| = {float(err.max()) if err.size else 0.0:.3e} "
            f"(max|ref| = {float(np.abs(b[fin]).max()) if err.size else 0.0:.3g}, "
            f"worst margin {worst:.2e})")
        assert worst <= 0.0, f"{name}: error above atol + {rel} |ref|"
