"""HBM traffic per launch of one kernel, from rocprofv3 counters.

Two counter runs of bench.py (each with --calibrate-copy-mb M), one with
FETCH_SIZE and one with WRITE_SIZE, give per-dispatch KiB for every kernel.
The calibration dispatch converts M MiB of bf16 to float32: it reads exactly
M MiB and writes 2M MiB, so read and write counts are scaled by
known / counted of that dispatch.  The result is written as JSON with the
hash of the kernel sources it was taken on; bench.py reports it as
roofline.traffic only while that hash still matches.

    rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "(dq_q_kernel|copy)" \\
        --output-format csv -d <F> -o run -- python bench.py --workload select_T8192 \\
        --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy-mb 512
    (the same with WRITE_SIZE into <W>)
    python -m block_sparse_attention_nsa_amd.traffic --kernel dq_q_kernel \\
        --workload select_T8192 --copy-mb 512 --fetch <F>/run_counter_collection.csv \\
        --write <W>/run_counter_collection.csv --out profiles/dq_q_kernel_select_T8192_traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


# The sources a kernel's memory traffic depends on: its own file, the shared
# device headers, the launch parameters chosen in nsa_api.hip, and for the
# dK/dV kernel the inversion and plan that lay out its row lists and items.
_COMMON = ("nsa_device.h", "nsa_internal.h", "nsa_api.hip")
KERNEL_SOURCES = {
    "fwd_q_kernel": ("nsa_query.hip",) + _COMMON,
    "dq_q_kernel": ("nsa_query.hip",) + _COMMON,
    # reads the dS the dK/dV kernel stores and the inversion's slot positions
    "dq_ds_kernel": ("nsa_query.hip", "nsa_dkdv.hip", "nsa_common.hip") + _COMMON,
    "dkdv_kernel": ("nsa_dkdv.hip", "nsa_common.hip") + _COMMON,
}


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def _code_only(text: str) -> str:
    """Source text without comments and blank-line/indent noise, so that a
    comment edit does not invalidate a traffic record."""
    lines = (ln.strip() for ln in _COMMENT.sub("", text).splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash(kernel: str = None) -> str:
    """Hash of the code (comments stripped) of the HIP sources a kernel's
    traffic depends on (all HIP sources and the public header when kernel is
    None or unknown)."""
    h = hashlib.sha256()
    files = KERNEL_SOURCES.get(kernel)
    for d in (os.path.join(HERE, "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h")) and (files is None or f in files or d.endswith("include")):
                with open(os.path.join(d, f), encoding="utf-8", errors="replace") as fh:
                    h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str):
    """[(dispatch id, kernel name, KiB)] of one counter collection."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            key = int(row["Dispatch_Id"])
            name, val = row["Kernel_Name"], float(row["Counter_Value"])
            prev = out.get(key)
            out[key] = (name, val + (prev[1] if prev else 0.0))
    return [(k, n, v) for k, (n, v) in sorted(out.items())]


def _kernel_mean(disp, pattern: str) -> float:
    """KiB per launch of the stage the pattern names.  A stage may launch
    more than one instantiation per step (dK/dV on whole-prefix selections:
    the paired kernel and the per-block one, which then exits at once), so
    this is the total over all matching dispatches divided by the number of
    steps (the dispatch count of each instantiation)."""
    per_name = {}
    for _, n, v in disp:
        if re.search(pattern, n):
            c, t = per_name.get(n, (0, 0.0))
            per_name[n] = (c + 1, t + v)
    if not per_name:
        raise SystemExit(f"no dispatch of {pattern!r} in the counter file")
    steps = max(c for c, _ in per_name.values())
    return sum(t for _, t in per_name.values()) / steps


def _copy_value(disp) -> float:
    """KiB of the calibration conversion: bench.py runs it after every other
    kernel, so it is the last copy dispatch."""
    vals = [v for _, n, v in disp if "copy" in n]
    if not vals:
        raise SystemExit("no copy kernel dispatch in the counter file")
    return vals[-1]


def stats_table(path: str, header: str) -> str:
    """A rocprofv3 kernel_stats.csv as a fixed-width text table (microseconds),
    kernel names cut before their argument lists."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            cut = name.find("(")
            name = (name[:cut] if cut > 0 else name).replace("void ", "")
            rows.append((name[:58], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines = [header.rstrip("\n"),
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for n, c, av, mn, mx, pc in rows:
        lines.append(f"{n:58s} {c:6d} {av:9.1f} {mn:9.1f} {mx:9.1f} {pc:6.2f}")
    return "\n".join(lines) + "\n"


SIMDS = 1024            # 256 CUs x 4 SIMDs
CLOCK_GHZ = 2.4         # peak engine clock the MFMA peak is quoted at


def stats_avg_ns(path: str, pattern: str) -> float:
    """Summed average duration (ns) of the kernels a regex matches in a
    kernel_stats.csv (a stage that launches two instantiations per step)."""
    t = 0.0
    with open(path) as f:
        for r in csv.DictReader(f):
            if re.search(pattern, r["Name"]):
                t += float(r["AverageNs"])
    return t if t > 0 else float("nan")


def sq_table(paths, kernels, header: str, stats: str = None) -> str:
    """SQ counters of one workload's passes (run_counter_collection.csv each)
    as per-launch whole-device totals for each kernel regex, their shares of
    SQ_WAVE_CYCLES, and the MFMA-busy share of all SIMD cycles at the peak
    clock (kernel time from a kernel_stats.csv of an unprofiled-counter run
    if given, else from the counter dispatches' own timestamps)."""
    tot = {k: {} for k in kernels}
    launches = {k: {} for k in kernels}  # counter -> {kernel name: dispatches}
    dur = {k: {} for k in kernels}
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                for k in kernels:
                    if not re.search(k, row["Kernel_Name"]):
                        continue
                    c = row["Counter_Name"]
                    tot[k][c] = tot[k].get(c, 0.0) + float(row["Counter_Value"])
                    launches[k].setdefault(c, {}).setdefault(row["Kernel_Name"], set()).add(row["Dispatch_Id"])
                    if "End_Timestamp" in row and path == paths[0]:
                        dur[k][row["Dispatch_Id"]] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    counters = sorted({c for k in kernels for c in tot[k]})
    # Per stage launch: a stage may launch two instantiations per step (the
    # paired dK/dV kernel and the per-block one, which then exits at once),
    # so totals are divided by the most-launched instantiation's count.
    per = {k: {c: tot[k][c] / max(1, max((len(v) for v in launches[k].get(c, {}).values()), default=1))
               for c in tot[k]} for k in kernels}
    avg_ns = {k: (sum(dur[k].values()) / max(1, max((len(v) for c in launches[k]
                                                       for v in launches[k][c].values()), default=1))
                  if dur[k] else float("nan")) for k in kernels}
    if stats:
        avg_ns = {k: stats_avg_ns(stats, k) for k in kernels}
    w = max(14, *(len(k) + 2 for k in kernels))
    lines = [header.rstrip("\n"), f"{'counter':30s}" + "".join(f"{k:>{w}s}" for k in kernels)]
    for c in counters:
        lines.append(f"{c:30s}" + "".join(f"{per[k].get(c, float('nan')):>{w}.4g}" for k in kernels))
    lines.append("")
    lines.append("shares of SQ_WAVE_CYCLES (resident wave time):")
    for c in counters:
        if c.startswith(("SQ_ACTIVE_INST", "SQ_WAIT")):
            lines.append(f"{c:30s}" + "".join(
                f"{per[k].get(c, float('nan')) / per[k].get('SQ_WAVE_CYCLES', float('nan')):>{w}.2f}"
                for k in kernels))
    lines.append("")
    lines.append(f"{'kernel time per launch (us)':30s}" + "".join(f"{avg_ns[k] / 1e3:>{w}.1f}" for k in kernels))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
        lines.append(f"{'MFMA busy share of SIMD cycles':30s}" + "".join(
            f"{per[k].get('SQ_VALU_MFMA_BUSY_CYCLES', float('nan')) / (SIMDS * avg_ns[k] * CLOCK_GHZ):>{w}.3f}"
            for k in kernels))
    return "\n".join(lines) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--stats", help="format this kernel_stats.csv into --out instead (with "
                                    "--command and --workload in its header)")
    ap.add_argument("--kernel", help="regex of the kernel name (e.g. dq_q_kernel)")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--copy-mb", type=int)
    ap.add_argument("--fetch", help="run_counter_collection.csv with FETCH_SIZE")
    ap.add_argument("--write", help="run_counter_collection.csv with WRITE_SIZE")
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="", help="the profiling commands, recorded in the output")
    ap.add_argument("--sq", nargs="+", help="format these SQ counter passes (run_counter_collection.csv "
                                            "each) for the --kernels into --out instead")
    ap.add_argument("--kernels", default="fwd_q_kernel,dq_q_kernel,dq_ds_kernel,dkdv_kernel",
                    help="comma-separated kernel regexes (--sq)")
    a = ap.parse_args()
    if a.sq:
        ks = [k for k in a.kernels.split(",") if k]
        head = (f"# rocprofv3 SQ counters, per launch (whole device), workload {a.workload}\n"
                f"# command: {a.command}\n"
                f"# kernel sources hash: {source_hash()}\n")
        text = sq_table(a.sq, ks, head, a.stats)
        with open(a.out, "w") as f:
            f.write(text)
        print(text, end="")
        return
    if a.stats:
        head = (f"# rocprofv3 kernel statistics, workload {a.workload}\n"
                f"# command: {a.command}\n"
                f"# kernel sources hash: {source_hash()}\n")
        text = stats_table(a.stats, head)
        with open(a.out, "w") as f:
            f.write(text)
        print(text, end="")
        return
    if not (a.kernel and a.copy_mb and a.fetch and a.write):
        ap.error("--kernel, --copy-mb, --fetch and --write are needed for a traffic record")
    fd, wd = _per_dispatch(a.fetch, "FETCH_SIZE"), _per_dispatch(a.write, "WRITE_SIZE")
    read_known, write_known = a.copy_mb * 2 ** 20, 2 * a.copy_mb * 2 ** 20
    f_scale = read_known / (_copy_value(fd) * 1024.0)
    w_scale = write_known / (_copy_value(wd) * 1024.0)
    fetch = _kernel_mean(fd, a.kernel) * 1024.0 * f_scale
    write = _kernel_mean(wd, a.kernel) * 1024.0 * w_scale
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "source_hash": source_hash(a.kernel),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "copy_calibration": {"mib": a.copy_mb, "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
        "command": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
