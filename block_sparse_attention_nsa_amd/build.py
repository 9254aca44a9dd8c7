"""Builds libnsa_sel.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m block_sparse_attention_nsa_amd.build

Every source is compiled on each call (the build is the "does it build"
check); objects go to csrc/_build/, the library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libnsa_sel.so")
SOURCES = ["nsa_api.hip", "nsa_common.hip", "nsa_query.hip", "nsa_dkdv.hip", "nsa_f32.hip"]
# Kernels that keep matrix-core accumulators in AGPRs (one wave per SIMD,
# up to 512 registers): built without the VGPR-only accumulator option.
AGPR_SOURCES = {"nsa_dkdv.hip"}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # No packed-fp32 VALU instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Matrix-core accumulators in VGPRs: avoids the AGPR<->VGPR copies the
# register allocator otherwise inserts around loop-carried MFMA chains.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _git_commit() -> str:
    """Short commit of the checkout, "+dirty" if the library's sources or
    header differ from it; "unknown" outside a git checkout."""
    try:
        sha = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True, timeout=30)
        if sha.returncode != 0 or not sha.stdout.strip():
            return "unknown"
        dirty = subprocess.run(["git", "status", "--porcelain", "--", CSRC, INCLUDE], cwd=ROOT,
                               capture_output=True, text=True, timeout=30).stdout.strip()
        return sha.stdout.strip() + ("+dirty" if dirty else "")
    except (OSError, subprocess.SubprocessError):
        return "unknown"


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    commit = _git_commit()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        objs.append(obj)
        extra = [] if src in AGPR_SOURCES else VGPR_FORM
        if src == "nsa_api.hip":
            extra = extra + [f'-DNSA_BUILD_GIT="{commit}"']
        cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that
        # warning is expected and dropped.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines and (verbose or pr.returncode):
            print("\n".join(lines), file=sys.stderr)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
