"""Benchmark: NSA selection attention fwd + bwd on one MI355X.

    python bench.py [--steps K] [--warmup W]
        [--workload select_T8192|causal_B4_T4096|packed_8seq|bf16_T1024]

Without --workload the line's headline is select_T8192 (B1 Hq32 Hkv2 T8192
bs64 S16, with the CPU oracle baseline) and "also" holds the same figures for
the other D128 workloads, causal_B4_T4096 and packed_8seq, timed after it in
the same process; with --workload only that one is timed.

A step is one pass of the whole hot path over one batch of synthetic input:
nsa_sel_fwd, then the backward's stages (Delta + block->query inversion +
plan, the dK/dV block kernel, the dK/dV partial reduction, dQ).  Inputs are
resident in HBM before timing.  By default the inversion runs on a second
stream beside the forward and the reduction beside dQ (--serial: one stream).
The metric is useful TFLOP/s: F_fwd = 4*D*N and F_bwd = 10*D*N with N the
exact number of (query-head row, key) pairs the block lists select (counted
here from block_idx), per step, over the wall time of K steps bracketed by
device synchronisation.  Per-stage times come from a separate pass of K
steps with events at every stage boundary on the streams the kernels run
on; the timed region itself records only the dominant kernel's two events
(its duration for the roofline), since each timing event holds its stream
back a little.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0

# Workloads the benchmark runs (the f32 one is a parity case only).
BENCH_WORKLOADS = ("select_T8192", "causal_B4_T4096", "packed_8seq", "bf16_T1024")
HEADLINE = "select_T8192"
ALSO = ("causal_B4_T4096", "packed_8seq")
# Algorithmic flops per (row, key) pair of each timed stage, in units of D:
# fwd S and PV; dq recomputes S and dP and forms dS K (or, when the dK/dV
# kernel hands its dS over, forms dS K alone); dkdv recomputes S and dP and
# forms dV and dK.
STAGE_FLOPS_PER_PAIR_D = {"fwd": 4, "dq": 6, "dkdv": 8}
DQ_HANDOFF_FLOPS_PER_PAIR_D = 2
# The one kernel each of these stages launches (bf16 path).
STAGE_KERNEL = {"fwd": "fwd_q_kernel", "dq": "dq_q_kernel", "dkdv": "dkdv_kernel"}
DQ_HANDOFF_KERNEL = "dq_ds_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def useful_pairs(block_idx: np.ndarray, G: int, bs: int, lengths, window: int = 0) -> int:
    """N = sum over query-head rows of |A|: a row (z, hkv, t) counts each
    distinct listed block u with 0 <= u < ceil(len/bs) and u*bs <= t, for
    min((u+1)*bs, t+1) - max(u*bs, t-window+1) keys (no lower limit without
    a window); times G heads."""
    total = 0
    for rows, L in lengths:  # rows: [n, S] int array for tokens 0..L-1 of one (z, hkv)
        if L == 0:
            continue
        t = np.arange(L)[:, None]
        u = rows.astype(np.int64)
        nb = -(-L // bs)
        ok = (u >= 0) & (u < nb) & (u * bs <= t)
        u = np.where(ok, u, -1)
        u.sort(axis=1)
        dup = np.zeros_like(ok)
        dup[:, 1:] = (u[:, 1:] == u[:, :-1])
        keep = (u >= 0) & ~dup
        lo = u * bs if window <= 0 else np.maximum(u * bs, t - window + 1)
        keys = np.maximum(np.minimum((u + 1) * bs, t + 1) - lo, 0)
        total += int(np.where(keep, keys, 0).sum())
    return total * G


def row_groups(w):
    """(rows [L, S], L) per (z, hkv) of a workload."""
    if w.packed:
        for z in range(w.n_seqs):
            a, b = int(w.cu_seqlens[z]), int(w.cu_seqlens[z + 1])
            for h in range(w.Hkv):
                yield w.block_idx[h, a:b], b - a
    else:
        for z in range(w.B):
            for h in range(w.Hkv):
                yield w.block_idx[z, h], w.T


def git_sha() -> str:
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True).stdout.strip() or "unknown"
    except OSError:
        return "unknown"


def stored_traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, n_tokens: int, window: int = 0, sink=None):
    """The float64 oracle on the first n_tokens of every (entry, head) of the
    same draw (a closed causal sub-problem), full forward + backward (with
    the same window and sink logits, and the sink gradient, if any)."""
    import oracle

    if w.packed:
        z = int(np.argmax(np.diff(w.cu_seqlens)))
        a = int(w.cu_seqlens[z])
        L = min(n_tokens, int(w.cu_seqlens[z + 1]) - a)
        tr = lambda x: np.ascontiguousarray(x[a:a + L].transpose(1, 0, 2))[None]
        q, k, v, dO = tr(w.q), tr(w.k), tr(w.v), tr(w.dO)
        idx = np.ascontiguousarray(w.block_idx[:, a:a + L])[None]
        what = f"first {L} tokens of packed sequence {z}, all heads"
    else:
        L = min(n_tokens, w.T)
        sl = (slice(None), slice(None), slice(0, L))
        q, k, v, dO, idx = (np.ascontiguousarray(x[sl]) for x in (w.q, w.k, w.v, w.dO, w.block_idx))
        what = f"first {L} of {w.T} tokens of every batch entry and head"
    G = w.Hq // w.Hkv
    n = useful_pairs(idx, G, w.block_size,
                     ((idx[b, h], idx.shape[2]) for b in range(idx.shape[0]) for h in range(w.Hkv)),
                     window)
    sk = None if sink is None else np.asarray(sink, dtype=np.float64)
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, idx, w.block_size, w.scale, sink=sk, window=window)
    r = oracle.bwd(q, k, v, dO, idx, w.block_size, w.scale, sink=sk, window=window)
    if sk is not None:
        oracle.dsink(sk, r[3], r[4], head_axis=1)
    dt = time.perf_counter() - t0
    flops = 14.0 * w.D * n
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{what} (N={n} pairs), float64 fwd+bwd"}


def _recorder(evs):
    """ev(i) records timing event i of a step's list, if that list has one."""
    if evs is None:
        return lambda i: None
    return lambda i: evs[i].record() if evs[i] is not None else None


def run_workload(name, args, dev, cpu_leg: bool):
    """Times K steps of one workload; returns its part of the JSON line."""
    import torch

    import block_sparse_attention_nsa_amd as nsa
    import workloads

    w = workloads.make_workload(name, seed=args.seed)
    G = w.Hq // w.Hkv
    N = useful_pairs(w.block_idx, G, w.block_size, row_groups(w), args.window)
    f_fwd, f_bwd = 4.0 * w.D * N, 10.0 * w.D * N
    log(f"[bench] {name}: {workloads.WORKLOADS[name]}; N = {N} pairs, "
        f"F_fwd = {f_fwd:.4g}, F_bwd = {f_bwd:.4g}")

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt).contiguous()
    q, k, v, dO = up(w.q), up(w.k), up(w.v), up(w.dO)
    idx = torch.from_numpy(np.ascontiguousarray(w.block_idx)).to(dev)
    cu = None if not w.packed else torch.from_numpy(w.cu_seqlens).to(dev)
    ms = w.max_seqlen if w.packed else None
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T) if not w.packed else (w.Hq, w.T), dtype=torch.float32, device=dev)
    stages = nsa.BwdStages(q, k, v, idx, w.block_size, w.scale, cu, ms, window=args.window,
                           sched_policy=args.sched)
    serial = args.serial
    names = (("fwd", "prepare", "dkdv", "dkdv_reduce", "dq") if serial else
             ("fwd", "prepare_lists", "prepare_delta", "dkdv", "dkdv_reduce", "dq")) + \
        (("dsink",) if args.sink else ())
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sink = None
    if args.sink:
        sink = torch.from_numpy(np.random.default_rng(args.seed + 1).normal(0.0, 1.0, w.Hq)
                                .astype(np.float32)).to(dev)
        dsink = torch.empty_like(sink)

    def step_overlapped(evs=None):
        # Two streams, default priority.  The inversion needs only block_idx:
        # it runs on the side stream during the forward (after the previous
        # step's dK/dV and dQ have read the lists it overwrites).  The dK/dV
        # reduce and dQ read and write disjoint data: the reduce runs on the
        # side stream beside dQ.
        ev = _recorder(evs)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            ev(1)
            stages.prepare_lists()
            ev(2)
        ev(0)
        nsa.nsa_sel_fwd(q, k, v, idx, w.block_size, w.scale, cu, ms, out=o, lse=lse, sink=sink,
                        window=args.window)
        ev(3)
        stages.prepare_delta(o, dO)
        ev(4)
        main.wait_stream(side)
        stages.dkdv_blocks(dO, lse)
        ev(5)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            ev(6)
            stages.dkdv_reduce()
            ev(7)
        stages.dq_stage(dO, lse)
        ev(8)
        if sink is not None:
            stages.dsink_stage(lse, sink, out=dsink)
        ev(10)
        main.wait_stream(side)
        ev(9)

    def step(evs=None):
        if not serial:
            return step_overlapped(evs)
        ev = _recorder(evs)
        ev(0)
        nsa.nsa_sel_fwd(q, k, v, idx, w.block_size, w.scale, cu, ms, out=o, lse=lse, sink=sink,
                        window=args.window)
        ev(1)
        stages.prepare(o, dO)
        ev(2)
        stages.dkdv_blocks(dO, lse)
        ev(3)
        stages.dkdv_reduce()
        ev(4)
        stages.dq_stage(dO, lse)
        ev(5)
        if sink is not None:
            stages.dsink_stage(lse, sink, out=dsink)
            ev(6)

    n_ev = len(names) + 1 if serial else 11
    # (event pairs of each stage; overlapped: the side stream's stages run
    # beside the main stream's, so the stage times overlap)
    pairs = ({n: (j, j + 1) for j, n in enumerate(names)} if serial else
             {"fwd": (0, 3), "prepare_lists": (1, 2), "prepare_delta": (3, 4), "dkdv": (4, 5),
              "dkdv_reduce": (6, 7), "dq": (5, 8), "dsink": (8, 10)})
    pairs = {n: ab for n, ab in pairs.items() if n in names}

    def stage_times(n_steps):
        """Per-stage mean times and whole-step event times over n_steps steps
        with an event at every stage boundary."""
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
                  for _ in range(n_steps)]
        for i in range(n_steps):
            step(events[i])
        torch.cuda.synchronize()
        acc = {n: sum(evs[a].elapsed_time(evs[b]) for evs in events) / n_steps
               for n, (a, b) in pairs.items()}
        last = len(names) if serial else 9
        return acc, sorted(evs[0].elapsed_time(evs[last]) for evs in events)

    # W warm-up steps; with W >= 3 the last three carry every stage's events
    # to find the dominant kernel.  Each timing event holds its stream back a
    # little (a few us), so the timed region records only that kernel's two
    # events (all three candidates' with fewer warm-up steps, whose first
    # calls are too cold to rank the kernels).
    n_pre = 3 if args.warmup >= 3 else 0
    for _ in range(args.warmup - n_pre):
        step()
    cands = ("fwd", "dq", "dkdv")
    if n_pre:
        pre, _ = stage_times(n_pre)
        cands = (max(cands, key=lambda n: pre[n]),)
    torch.cuda.synchronize()

    # Timed region: K steps between two synchronisations, host clock; the
    # dominant kernel's own events (on its launch stream) give its duration.
    dom_events = []
    for _ in range(args.steps):
        row = [None] * n_ev
        for n in cands:
            for j in pairs[n]:
                row[j] = torch.cuda.Event(enable_timing=True)
        dom_events.append(row)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(dom_events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cand_ms = {n: sum(r[pairs[n][0]].elapsed_time(r[pairs[n][1]]) for r in dom_events) / args.steps
               for n in cands}
    dom = max(cands, key=lambda n: cand_ms[n])
    launch_ms = cand_ms[dom]
    ms_step = wall * 1e3 / args.steps
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    # Stage pass (K more steps, after the timed region): the breakdown.
    stage_ms, per_step = stage_times(args.steps)
    step_stats = {"median": round(float(np.median(per_step)), 4), "min": round(per_step[0], 4),
                  "max": round(per_step[-1], 4)}
    # The backward's share of the step: everything after the forward.
    bwd_ms = ms_step - stage_ms["fwd"]
    log(f"[bench] ms/step {ms_step:.3f}; stages (ms, stage pass): " +
        ", ".join(f"{n} {v:.3f}" for n, v in stage_ms.items()) +
        f"; {dom} in the timed region {launch_ms:.3f}")

    # The dominant kernel and its algorithmic flops per launch.
    kernel_of = dict(STAGE_KERNEL)
    flops_d = dict(STAGE_FLOPS_PER_PAIR_D)
    if stages.ds_handoff:
        kernel_of["dq"], flops_d["dq"] = DQ_HANDOFF_KERNEL, DQ_HANDOFF_FLOPS_PER_PAIR_D
    achieved = flops_d[dom] * w.D * N / (launch_ms * 1e-3) / 1e12
    from block_sparse_attention_nsa_amd.traffic import source_hash
    kern = kernel_of[dom]
    src = source_hash(kern)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(kern, name, src), "kernel": kern,
                "flops_per_launch": flops_d[dom] * w.D * N,
                "launch_ms": round(launch_ms, 4)}

    if args.calibrate_copy_mb:
        src_t = torch.randn(args.calibrate_copy_mb << 19, device=dev).to(torch.bfloat16)
        dst_t = torch.empty(src_t.numel(), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {src_t.numel() * 2} bytes read, "
            f"{dst_t.numel() * 4} bytes written")
        del src_t, dst_t

    cpu = None
    if cpu_leg:
        log(f"[bench] CPU oracle sample ({args.cpu_tokens} tokens per head) ...")
        cpu = cpu_baseline(w, args.cpu_tokens, args.window,
                           None if sink is None else sink.cpu().numpy())
        log(f"[bench] CPU oracle: {cpu['value'] * 1e3:.2f} GFLOP/s in {cpu['seconds']} s "
            f"on {cpu['cores']} threads")

    if w.packed:
        config = {"workload": name, "description": workloads.WORKLOADS[name],
                  "n_seqs": w.n_seqs, "total_tokens": w.T, "max_seqlen": w.max_seqlen,
                  "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "block_size": w.block_size, "S": w.S}
    else:
        config = {"workload": name, "description": workloads.WORKLOADS[name], "B": w.B,
                  "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "block_size": w.block_size,
                  "S": w.S}
    config["useful_pairs"] = N
    if args.window:
        config["window"] = args.window
    if args.sink:
        config["sink"] = "per-head logits ~ N(0, 1)"
    if args.sched:
        config["sched_policy"] = args.sched
    out = {
        "metric": "fwd+bwd useful TFLOP/s (bf16, D128) + % of MI355X bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": config,
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(f_fwd / (stage_ms["fwd"] * 1e-3) / 1e12, 3),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 3),
        "bwd_frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "schedule": "serial" if serial else "overlapped (inversion beside the forward, "
                                            "dK/dV reduce beside dQ; two streams)",
        "timing": "value / ms_per_step: K steps between device synchronisations, host clock, "
                  "events only around the dominant kernel; stage_ms / step_ms_events: K further "
                  "steps with an event at every stage boundary",
        "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "step_ms_events": step_stats,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ds_handoff": bool(stages.ds_handoff),
        "kernel_source_hash": src,
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=BENCH_WORKLOADS,
                    help="time only this workload (default: select_T8192, then the other D128 ones)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens per (entry, head) of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window of this many keys (0: none); a variant, not the metric's workload")
    ap.add_argument("--sink", action="store_true",
                    help="per-head attention-sink logits (forward with sink, dsink stage timed too)")
    ap.add_argument("--sched", type=int, default=0, choices=(0, 1),
                    help="scheduling policy of the hand-off dQ (nsa_sel_problem.sched_policy): "
                         "0 one workgroup per item, longest first; 1 a persistent grid taking "
                         "the items from a counter")
    ap.add_argument("--serial", action="store_true",
                    help="run every stage on one stream (default: the inversion beside the "
                         "forward and the dK/dV reduce beside dQ, on a second stream)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the timed steps, convert a bf16 tensor of this many MiB to "
                         "float32 once (a kernel of known traffic for scaling counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU: the path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_nsa_amd as nsa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    name = args.workload or HEADLINE
    out = run_workload(name, args, dev, cpu_leg=not args.no_cpu_baseline)
    if args.workload is None:
        out["also"] = []
        for other in ALSO:
            torch.cuda.empty_cache()
            r = run_workload(other, args, dev, cpu_leg=False)
            out["also"].append({k: r[k] for k in ("config", "value", "ms_per_step", "frac_of_peak",
                                                   "fwd_tflops", "bwd_tflops", "bwd_frac_of_peak",
                                                   "stage_ms", "step_ms_events", "roofline", "schedule",
                                                   "ds_handoff")})
    out["git"] = nsa.build_git()
    if out["git"] == "unknown":
        out["git"] = git_sha()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
