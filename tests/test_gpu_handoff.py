"""GPU parity of the backward that hands dS from the dK/dV kernel over to dQ
(bf16, G in {4, 8} or a multiple of 16, block_size >= 32, S <= 64, no
window, lists that cannot cover whole causal prefixes): dq = scale dS K
from the stored dS (page 1's gradients; the dQ of the plain masked softmax
attention).  Every output element against the float64 oracle at page 1's
bf16 gate, on tile shapes of 4, 2 and 1 tokens of 16 rows (the last at
head dims 32, 64 and 128 and block sizes 32, 64 and 128), ragged tails,
lists with -1 padding, duplicates, out-of-range and future blocks and empty
rows (the dS of a block is taken from its first listing in the row), and
packed sequences with an empty one.  Each case also checks that the library
reports the hand-off for it."""
import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import workloads
from _harness import say, to_dev
from test_gpu_parity import _full_parity, _weird_block_idx

pytestmark = pytest.mark.gpu


def _handoff_on(w):
    d = to_dev(w)
    ms = w.max_seqlen if w.packed else None
    p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale, d["cu"], ms)
    return nsa.ds_handoff(p)


@pytest.mark.parametrize("case", [
    dict(name="ho-G4-D128-bs64", B=2, Hq=8, Hkv=2, T=777, D=128, S=5, bs=64),
    dict(name="ho-G8-D64-bs32", B=1, Hq=16, Hkv=2, T=530, D=64, S=6, bs=32),
    dict(name="ho-G16-D128-bs128", B=1, Hq=16, Hkv=1, T=900, D=128, S=3, bs=128),
    dict(name="ho-G32-D32-bs64", B=1, Hq=64, Hkv=2, T=420, D=32, S=4, bs=64),
    dict(name="ho-G16-D64-bs64", B=2, Hq=16, Hkv=1, T=611, D=64, S=5, bs=64),
    dict(name="ho-G16-D128-bs32", B=1, Hq=16, Hkv=1, T=389, D=128, S=7, bs=32),
    dict(name="ho-G4-D64-S>NB", B=1, Hq=8, Hkv=2, T=300, D=64, S=9, bs=32),
])
def test_handoff_irregular_lists(case):
    rng = np.random.default_rng(81)
    c = dict(case)
    name = c.pop("name")
    idx = _weird_block_idx(rng, c["B"], c["Hkv"], c["T"], c["bs"], c["S"])
    w = workloads.make_dense(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["S"], c["bs"], "bf16",
                             seed=82, name=name, block_idx=idx)
    assert _handoff_on(w)
    _full_parity(w)


@pytest.mark.parametrize("G", [4, 8])
def test_handoff_packed(G):
    """Packed sequences (one empty, one shorter than a block) with the
    first-block lists of the packed workload: a workgroup's 64 (G = 4) or
    32 (G = 8) tokens stay inside one sequence."""
    w = workloads.make_thd([700, 0, 40, 1100, 257], 2 * G, 2, 128, 6, 64, "bf16",
                           "own_first_random", seed=83 + G, name=f"ho-packed-G{G}")
    assert _handoff_on(w)
    _full_parity(w)


def test_handoff_bitwise_repeatable():
    """Two backward calls on the same inputs give bitwise the same dq (the
    dS store and the dQ walk have fixed orders)."""
    w = workloads.make_dense(1, 8, 2, 1500, 128, 8, 64, "bf16", "own_first_random", seed=85,
                             name="ho-repeat")
    assert _handoff_on(w)
    d = to_dev(w)
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale)
    a = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size, w.scale)
    b = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size, w.scale)
    for x, y, n in zip(a, b, ("dq", "dk", "dv")):
        assert bool((x == y).all()), n
    say("[ho-repeat] dq, dk, dv bitwise equal over two calls")


def _persistent_case(name):
    if name == "ho-persist-G8":
        return workloads.make_thd([3000, 0, 1500, 2049], 16, 2, 128, 6, 64, "bf16",
                                  "own_first_random", seed=87, name=name)
    return workloads.make_workload(name)


@pytest.mark.parametrize("name", ["select_T8192", "packed_8seq", "ho-persist-G8"])
def test_persistent_schedule_is_bitwise_the_same(name):
    """sched_policy 1 (a persistent grid of one workgroup per CU taking the
    hand-off dQ's items from a workspace counter, longest first) gives the
    same dq, dk, dv bit for bit as the default launch, on problems with more
    items than CUs (tiles of 1, 4 and 2 tokens); two backward calls on one
    workspace, and the dQ stage run twice after one prepare, check that the
    counter starts from zero each time."""
    w = _persistent_case(name)
    assert _handoff_on(w)
    d = to_dev(w)
    cu = d["cu"]
    ms = w.max_seqlen if w.packed else None
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms)
    ref = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                          w.scale, cu, ms)
    ws = torch.empty(nsa.bwd_workspace_bytes(nsa.make_problem(d["q"], d["k"], d["idx"],
                                                               w.block_size, w.scale, cu, ms)),
                     dtype=torch.uint8, device="cuda")
    for it in range(2):
        got = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                              w.scale, cu, ms, workspace=ws, sched_policy=1)
        for a, b, n in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"call {it}: {n}"
    st = nsa.BwdStages(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms,
                       sched_policy=1)
    st.prepare(o, d["dO"])
    st.dkdv_blocks(d["dO"], lse)
    st.dkdv_reduce()
    for it in range(2):
        st.dq.zero_()  # an item the walk skipped would stay zero
        dq = st.dq_stage(d["dO"], lse)
        assert torch.equal(dq, ref[0]), f"dQ stage run {it}"
    torch.cuda.synchronize()
    say(f"[{name}] persistent hand-off dQ: bitwise equal to the default launch "
        f"(two calls, and the dQ stage twice after one prepare)")
