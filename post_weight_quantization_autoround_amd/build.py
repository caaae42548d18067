"""Build libautoround.so (HIP for gfx950) in the package directory.

    python post_weight_quantization_autoround_amd/build.py

Compiles every csrc/*.hip in parallel with hipcc and links one shared
library; the measurement aid csrc_probe/*.hip (on-box peaks) links into
libarpeaks.so beside it.  Flags: -O3, no FMA contraction (the quantizer's codes must be
reproducible bit for bit), packed-fp32 instructions disabled, hidden
visibility except for the C ABI.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libautoround.so")
PROBE_SRC = os.path.join(PKG, "csrc_probe")
PROBE_LIB = os.path.join(PKG, "libarpeaks.so")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (ROCm is required to build libautoround)")
    return found


def _compile_and_link(srcs, lib_path, tag, verbose):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, tag + "_" + os.path.basename(src) + ".o")
        cmd = [cc, *CFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib_path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)


def build(verbose: bool = False) -> str:
    """Compile all sources and link the library (and the peak probe);
    returns the library's path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    _compile_and_link(srcs, LIB, "ar", verbose)
    probe = sorted(glob.glob(os.path.join(PROBE_SRC, "*.hip")))
    if probe:
        _compile_and_link(probe, PROBE_LIB, "probe", verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
