"""Build libks_norm.so (the HIP kernels for gfx950 plus the C ABI) in-tree.

    python -m rmsnorm_row_normalisation_amd.build

Each translation unit compiles in parallel into ``_build/``; the shared
library is linked next to this file.  hipcc cross-compiles for gfx950, so no
GPU is needed to build.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libks_norm.so")
# the benchmark's reference streams (plain reads, writes and copies), a library of their own
STREAMREF_SRC = os.path.join(PKG, "streamref", "ks_streamref.hip")
STREAMREF_LIB = os.path.join(PKG, "libks_streamref.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every multiply and add in the kernels rounds as written
#   (the one fused step, the sum of squares, is an explicit fmaf).
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code.
# -amdgpu-kernarg-preload-count=16: kernels whose arguments are scalars get
#   up to 16 SGPRs of them preloaded at wave launch (the row kernels' 48 bytes
#   fit); a kernel taking a struct is unaffected.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def source_id() -> str:
    """The git commit the sources were built from (+dirty when the tree differs
    from it), or "unknown" outside a git checkout; ks_version() reports it."""
    try:
        res = subprocess.run(["git", "-C", ROOT, "describe", "--always", "--dirty", "--abbrev=12"],
                             capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return "unknown"
    out = res.stdout.strip()
    return out if res.returncode == 0 and re.fullmatch(r"[0-9a-zA-Z.+_-]+", out) else "unknown"


def _compile(src: str, defines: tuple[str, ...] = ()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *defines, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4) // 2), 8)
    defines = (f'-DKS_BUILD_GIT="{source_id()}"',)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, defines if src.endswith("ks_api.cpp") else ()), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    tmp = STREAMREF_LIB + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", STREAMREF_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"reference streams build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, STREAMREF_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
