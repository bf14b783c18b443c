"""Build libtokengate.so (all HIP sources, gfx950) in-tree.

    python -m learned_token_pruning_06_amd.build        # or build() from Python

Each source compiles to an object under ``_build/`` in parallel, then one
hipcc link produces ``learned_token_pruning_06_amd/libtokengate.so``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtokengate.so")
ARCH = os.environ.get("TG_OFFLOAD_ARCH", "gfx950")

# Packed fp32 vector instructions are disabled for every device pass.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libtokengate.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]

    def comp(pair):
        src, obj = pair
        return _run([cc, *HIPCC_FLAGS, "-c", src, "-o", obj], verbose)

    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        logs = list(ex.map(comp, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    warn = "\n".join(l for l in logs if l.strip())
    if warn and not verbose:
        print(warn, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
