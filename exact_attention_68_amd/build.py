"""Build libattn.so in place with hipcc for gfx950.

    python -m exact_attention_68_amd.build

Compiles the C ABI (csrc/attn_api.cpp) and the kernels (csrc/attn_fwd.hip)
into exact_attention_68_amd/libattn.so. Every call compiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip"]
HEADERS = ["kernel_common.hpp", "launch.hpp", "tile_plan.hpp", "validate.hpp"]

# Packed fp32 VALU forms are switched off for all device code; the kernels rely on
# plain fp32 arithmetic only. The kernels never produce or test NaN (masked scores
# are -inf, maxima start from a finite sentinel), so NaN-quieting of max operands
# is dropped with -fno-honor-nans; infinities keep their IEEE behaviour.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build_library(verbose: bool = False) -> str:
    """Compile libattn.so; returns its path. Raises RuntimeError on a failed build."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_kernel_stubs(path: str) -> None:
    """Fail if the library references a kernel launch stub it does not define."""
    nm = shutil.which("nm") or "/opt/rocm/lib/llvm/bin/llvm-nm"
    res = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{nm} failed on {path}:\n{res.stderr}")
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.unlink(path)
        raise RuntimeError(f"built library lacks kernel launch stubs: {missing}")


def ensure_built() -> str:
    """Build only when no library exists yet (tests, smoke check and bench use this)."""
    if not os.path.exists(LIB):
        build_library()
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
