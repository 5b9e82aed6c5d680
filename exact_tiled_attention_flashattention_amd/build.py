"""Build libfa.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m exact_tiled_attention_flashattention_amd.build``.  Every
call recompiles every source; objects go to ``_build/`` at the repo root and
the library to this package directory, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd_rowwise.hip", "fa_fwd_mfma.hip", "fa_fwd_mfma_wide.hip", "fa_decode.hip",
           "fa_decode_mfma.hip", "fa_bwd.hip", "fa_bwd_mfma.hip",
           "fa_fwd_mfma_generic.hip", "fa_bwd_mfma32.hip", "fa_bwd_dq_mfma32.hip"]
# A second library, libfa_serial.so, differs only in the SERIAL_SOURCES, built
# with FA_SERIAL_COPIES=1: every copy into LDS is waited for, between
# barriers, before it is read.  Its results must equal libfa.so's bit for
# bit (a race check of the staging); only the tests load it.
SERIAL_SOURCES = ["fa_fwd_mfma_wide.hip", "fa_bwd_mfma32.hip", "fa_bwd_dq_mfma32.hip"]
SERIAL_LIBRARY = os.path.join(PKG, "libfa_serial.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _compile(src: str, serial: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ("_serial" if serial else "") + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *(["-DFA_SERIAL_COPIES=1"] if serial else []), "-c",
           path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "hip", "-c", path, "-o", obj] + DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, src) for src in SOURCES]
        futs_serial = {src.replace(".hip", ".o"): ex.submit(_compile, src, True)
                       for src in SERIAL_SOURCES}
        objs = [f.result() for f in futs]
        objs_serial = {name: f.result() for name, f in futs_serial.items()}
    serial_objs = [objs_serial.get(os.path.basename(o), o) for o in objs]
    for lib, parts in ((LIBRARY, objs), (SERIAL_LIBRARY, serial_objs)):
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *parts, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
