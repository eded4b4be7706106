"""Build libcsa2.so (HIP, gfx950) in-tree with hipcc.

    python -m fp4_compressed_sparse_csa2_amd.build

Compiles every ``csrc/*.hip`` with ``--offload-arch=gfx950`` into
``fp4_compressed_sparse_csa2_amd/libcsa2.so``.  Packed FP32 instructions are
disabled for the device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcsa2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa2.so)")


def flags(debug: bool = False) -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O1" if debug else "-O3",
        "-std=c++17",
        "-fPIC",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile all HIP sources (in parallel) and link libcsa2.so; returns its path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for s in srcs:
        o = os.path.join(obj_dir, os.path.basename(s)[:-4] + ".o")
        objs.append(o)
        cmd = [cc, *flags(), "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub a compile pass failed to emit
    # fails the link here instead of the first dlopen
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
            "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libcsa2.so failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


def _wait(item) -> None:
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the device-only target feature; that note is harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
