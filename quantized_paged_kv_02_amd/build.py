"""Build libkvq.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: ``python -m quantized_paged_kv_02_amd.build`` (or ``build_library()``).
Always recompiles; the output lands next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libkvq.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["kvq_api.cpp", "kvq_write.hip", "kvq_decode.hip", "kvq_calibrate.hip",
           "kvq_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # correctly rounded fp32 division: quantization codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc_path() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


def build_library(verbose: bool = False, out: str = LIB_PATH, defines=(),
                  objdir: str | None = None) -> str:
    """Compile every source and link ``libkvq.so`` (or ``out``); ``defines``
    are extra ``-D`` flags.  Returns the library path."""
    hipcc = hipcc_path()
    objdir = objdir or os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC,
               *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


PROBE_SOURCE = "kvq_probe.hip"
PROBE_PATH = os.path.join(PKG_DIR, "libkvq_probe.so")


def build_probe(verbose: bool = False, out: str = PROBE_PATH) -> str:
    """Compile the read-bandwidth probe (bench.py --probe) into its own
    shared library; it is measurement tooling, not part of libkvq."""
    hipcc = hipcc_path()
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", CSRC, "-x", "hip", "-shared",
           os.path.join(CSRC, PROBE_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
