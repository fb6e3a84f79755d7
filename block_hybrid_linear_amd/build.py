"""Build libhybrid_attn.so in-tree with hipcc for gfx950.

    python -m block_hybrid_linear_amd.build        # or build_library()

Each HIP source compiles to an object (in parallel), then one shared library
is linked next to this file.  Packed-fp32 instruction selection is switched
off for device code (-packed-fp32-ops); hipcc's host pass warns that it does
not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhybrid_attn.so")
SOURCES = ("api.hip", "step_kernels.hip", "state_kernels.hip", "exact_kernels.hip")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    for line in (r.stdout + r.stderr).splitlines():
        if line.strip() and noise not in line:
            print(line, file=sys.stderr)


def build_library(extra_flags: list[str] | None = None, out: str = LIB) -> str:
    """Compile every HIP source and link ``libhybrid_attn.so``; returns its path."""
    extra = list(extra_flags or [])
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(sys.argv[1:]))
