"""nsa_sel_bwd_noalloc (the backward for callers that cannot allocate: its
workspace is a fixed device array inside the library) against nsa_sel_bwd on
the same inputs, through the C ABI: two calls in a row, the second with a
smaller problem (the array keeps the first call's contents), each bitwise
equal to nsa_sel_bwd and within the bf16 gate of the float64 oracle.  With
16 heads per KV head and sparse lists the dK/dV kernel hands dS over to dQ:
bitwise equal again while that fits the array, and with dQ recomputing dS
when it does not (dk, dv bitwise, dq within the gate)."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_nsa_amd as nsa
import workloads
from block_sparse_attention_nsa_amd import _lib
from _harness import TOL, assert_close, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(w, d, o, lse):
    """dq, dk, dv from nsa_sel_bwd_noalloc, called through ctypes."""
    cu = d["cu"]
    ms = w.max_seqlen if w.packed else None
    p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale, cu, ms)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    nsa.set_strides(p, q=d["q"], k=d["k"], v=d["v"], o=o, dO=d["dO"], dq=dq, dk=dk, dv=dv)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = _lib.load().nsa_sel_bwd_noalloc(
        ctypes.byref(p), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(o), ptr(lse), ptr(d["dO"]),
        ptr(d["idx"]), ptr(cu), ptr(dq), ptr(dk), ptr(dv),
        torch.cuda.current_stream().cuda_stream)
    _lib.check("nsa_sel_bwd_noalloc", st)
    return dq, dk, dv


def test_noalloc_backward_equals_workspace_backward_twice():
    cases = [
        # lists long enough to be split into fp32 partials (the largest part
        # of the workspace), then a smaller packed problem
        workloads.make_dense(2, 8, 2, 2048, 128, 8, 64, "bf16", "own_first_random", seed=61,
                             name="noalloc-dense"),
        workloads.make_thd([300, 0, 77, 160], 6, 2, 64, 5, 32, "bf16", "own_first_random",
                           seed=62, name="noalloc-packed"),
    ]
    for w in cases:
        say(f"[{w.name}] B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} S={w.S} "
            f"bs={w.block_size} packed={w.packed}")
        d = to_dev(w)
        ms = w.max_seqlen if w.packed else None
        o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, d["cu"], ms)
        dq0, dk0, dv0 = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"],
                                        w.block_size, w.scale, d["cu"], ms)
        dq1, dk1, dv1 = _noalloc(w, d, o, lse)
        torch.cuda.synchronize()
        for name, a, b in (("dq", dq0, dq1), ("dk", dk0, dk1), ("dv", dv0, dv1)):
            assert torch.equal(a, b), f"{name}: nsa_sel_bwd_noalloc differs from nsa_sel_bwd"
        ref = oracle_full(w)
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        for name, a in (("dq", dq1), ("dk", dk1), ("dv", dv1)):
            assert_close(name, f(a), ref[name], TOL[w.dtype])
    assert nsa.wait_timeouts() == 0


def _workspace_bytes(w, d):
    cu = d["cu"]
    ms = w.max_seqlen if w.packed else None
    p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale, cu, ms)
    return int(_lib.load().nsa_sel_bwd_workspace_bytes(ctypes.byref(p)))


def test_noalloc_with_ds_handoff():
    cases = [
        # the hand-off fits the 64 MiB array: bitwise equal
        (workloads.make_dense(1, 16, 1, 1024, 128, 4, 64, "bf16", "own_first_random", seed=63,
                              name="noalloc-handoff"), True),
        # its dS (about 256 MiB) does not: dQ recomputes dS
        (workloads.make_dense(1, 32, 1, 4096, 32, 16, 64, "bf16", "own_first_random", seed=64,
                              name="noalloc-handoff-too-big"), False),
    ]
    for w, fits in cases:
        say(f"[{w.name}] B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} S={w.S} bs={w.block_size}")
        d = to_dev(w)
        assert (_workspace_bytes(w, d) <= 64 << 20) == fits
        o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale)
        dq0, dk0, dv0 = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"],
                                        w.block_size, w.scale)
        dq1, dk1, dv1 = _noalloc(w, d, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(dk0, dk1) and torch.equal(dv0, dv1)
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        if fits:
            assert torch.equal(dq0, dq1)
        else:
            assert_close("dq (hand-off vs recomputed)", f(dq1), f(dq0), TOL[w.dtype])
        ref = oracle_full(w)
        for name, a in (("dq", dq1), ("dk", dk1), ("dv", dv1), ("dq (nsa_sel_bwd)", dq0)):
            assert_close(name, f(a), ref[name.split()[0]], TOL[w.dtype])
    assert nsa.wait_timeouts() == 0


def test_noalloc_backward_under_graph_capture():
    """The callers this entry point is for: forward (preallocated outputs) and
    nsa_sel_bwd_noalloc captured into one HIP graph and replayed three
    times, with other eager work and a synchronisation between replays;
    every replay's o, lse, dq, dk, dv must equal the eager results bitwise.
    Covers the hand-off (16 heads per KV head, sparse lists) and a packed
    4-head problem.  The first call on the device (the scratch address
    lookup) happens before the capture."""
    cases = [
        workloads.make_dense(1, 16, 1, 1024, 128, 4, 64, "bf16", "own_first_random", seed=65,
                             name="graph-handoff"),
        workloads.make_thd([300, 0, 77, 160], 8, 2, 64, 5, 32, "bf16", "own_first_random",
                           seed=66, name="graph-packed"),
    ]
    for w in cases:
        say(f"[{w.name}] graph capture: B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D}")
        d = to_dev(w)
        ms = w.max_seqlen if w.packed else None
        o = torch.empty_like(d["q"])
        lse = torch.empty((w.B, w.Hq, w.T) if not w.packed else (w.Hq, w.T), dtype=torch.float32,
                          device=d["q"].device)
        nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, d["cu"], ms,
                        out=o, lse=lse)
        dq0, dk0, dv0 = _noalloc(w, d, o, lse)
        torch.cuda.synchronize()
        ref = [x.clone() for x in (o, lse, dq0, dk0, dv0)]

        cu, p = d["cu"], None
        p = nsa.make_problem(d["q"], d["k"], d["idx"], w.block_size, w.scale, cu, ms)
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        nsa.set_strides(p, q=d["q"], k=d["k"], v=d["v"], o=o, dO=d["dO"], dq=dq, dk=dk, dv=dv)
        lib = _lib.load()
        ptr = lambda t: None if t is None else t.data_ptr()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, cu, ms,
                                out=o, lse=lse)
                st = lib.nsa_sel_bwd_noalloc(
                    ctypes.byref(p), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(o), ptr(lse),
                    ptr(d["dO"]), ptr(d["idx"]), ptr(cu), ptr(dq), ptr(dk), ptr(dv),
                    torch.cuda.current_stream().cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        _lib.check("nsa_sel_bwd_noalloc (captured)", st)
        for rep in range(3):
            for x in (o, lse, dq, dk, dv):
                x.fill_(7.0)                      # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
                assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        say(f"  3 replays bitwise equal to the eager call")
    assert nsa.wait_timeouts() == 0
