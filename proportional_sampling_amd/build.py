"""Builds libpsamp.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m proportional_sampling_amd.build        # or build() from Python
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpsamp.so")
SOURCES = ["api.hip", "scan.hip", "sample.hip", "isw.hip", "tree.hip", "resample.hip",
           "scatter.hip", "per_round.hip", "pf.hip",
           "replay.hip", "ceiling.hip", "check.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # fp64/fp32 arithmetic exactly as written: no contraction into FMAs
    # except where fma() is spelled out.
    "-ffp-contract=off",
    # packed fp32 ops are kept out of the code objects.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the CPU test of
# the argument validation (the device code is built as usual).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def _compile(src: str, objdir: str = OBJ, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitize_host: bool = False, out: str | None = None) -> str:
    """Compile every kernel source for gfx950 and link libpsamp.so (or, with
    sanitize_host, a copy whose host code carries ASan + UBSan, at `out`)."""
    lib = out or LIB
    objdir = OBJ if not sanitize_host else os.path.join(os.path.dirname(lib), "_obj_sanitize")
    os.makedirs(objdir, exist_ok=True)
    extra = SANITIZE_HOST if sanitize_host else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, objdir, extra), SOURCES))
    tmp = lib + ".tmp"
    # (a sanitized build leaves the sanitizer runtime's symbols to the
    # runtime the process preloads)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def clean() -> None:
    shutil.rmtree(OBJ, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build()
