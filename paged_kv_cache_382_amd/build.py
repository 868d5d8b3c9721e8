"""Build ``libpa.so`` (HIP kernels for gfx950 + C ABI + host allocator).

Usage: ``python -m paged_kv_cache_382_amd.build`` or ``build()`` from Python.
Each call recompiles everything; objects go to ``_build/`` and the library to
``paged_kv_cache_382_amd/lib/libpa.so`` (both git-ignored).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libpa.so")
# The streaming-read probe (a measurement helper, include/pa_probe.h) is a
# library of its own, so that the attention library holds only the path.
PROBE_LIB = os.path.join(LIB_DIR, "libpa_probe.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Device code: gfx950 only.  Packed-fp32 instructions are switched off.
HIP_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]

SOURCES = [
    ("allocator.cpp", "host"),
    ("capi.cpp", "hip-host"),
    ("store_kvcache.hip", "hip"),
    ("decode.hip", "hip"),
    ("prefill.hip", "hip"),
]
PROBE_SOURCES = [("probe.hip", "hip")]


def _compile(src, kind, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if kind == "host":
        cmd = ["g++"] + HOST_FLAGS + ["-c", path, "-o", obj]
    elif kind == "hip-host":
        cmd = [HIPCC, "-x", "hip"] + HIP_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + HIP_FLAGS + list(extra) + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False, extra_hip_flags=()):
    """Compile every source and link ``libpa.so``; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda sk: _compile(sk[0], sk[1], extra_hip_flags), SOURCES + PROBE_SOURCES))
    n_main = len(SOURCES)
    for target, parts in ((LIB, objs[:n_main]), (PROBE_LIB, objs[n_main:])):
        tmp = target + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + parts
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        shutil.move(tmp, target)
        if verbose:
            print(f"built {target}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_hip_flags=sys.argv[1:])
