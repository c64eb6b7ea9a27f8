"""Build libtls.so (the gfx950 HIP library behind include/tls.h) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libtls.so"
BUILD = PKG / "_build"
SOURCES = ["k_build.hip", "k_select.hip", "k_decode.hip", "k_step.hip", "k_copy.hip", "tls_api.cpp", "offload.cpp"]
ARCH = os.environ.get("TLS_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU ops are kept out of the device code (-packed-fp32-ops).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-I", str(PKG.parent / "include")]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every source and link libtls.so (always rebuilds)."""
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libtls.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
