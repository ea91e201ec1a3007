"""Build the gfx950 MoE library (libmoe.so) in-tree with hipcc.

    python -m token_routing_expert_amd.build [--debug]

--debug builds libmoe_debug.so instead: the same kernels with the device-side
contract checks of MOE_DCHECK compiled in (expert ids in [-1, E), monotone
offsets, row indices in range, finite logits); a value outside its contract
stops the kernel with a trap.  For valid input its results equal the release
library's bit for bit.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops; the host pass
warns that it does not know the feature, which is harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmoe.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libmoe_debug.so")
SOURCES = ["api.hip", "route.hip", "permute.hip", "grouped_ffn.hip", "combine.hip", "wgrad.hip"]
ARCH = "gfx950"

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, ("debug_" if debug else "") + os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *(["-DMOE_DEVICE_CHECKS"] if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libmoe.so (libmoe_debug.so
    with debug=True); returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    lib_path = DEBUG_LIB_PATH if debug else LIB_PATH
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
