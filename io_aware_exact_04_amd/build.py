"""Build libfa355.so (the C-ABI HIP library) in-tree for gfx950.

    python -m io_aware_exact_04_amd.build        # or build() from Python

Every source is compiled with hipcc for gfx950 only; packed-fp32 VALU
instructions are disabled (the target feature ``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa355.so")
# Measurement aid for bench.py (matrix-core peak probe), a library of its own.
PROBE_LIB = os.path.join(PKG, "libfa355_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]

SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_bwd_dkdv_bf16.hip",
           "fa_bwd_dq_bf16.hip", "fa_bwd_aux.hip", "fa_f32.hip",
           "fa_splitkv.hip", "fa_fp8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
         f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-source extra flags.  The forward kernel keeps its MFMA accumulators in
# VGPRs (the AGPR form makes the register allocator copy them between the two
# files on every tile).
EXTRA = {"fa_fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool, exports: str):
    # Only the C ABI is exported (a version script hides the internals).
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           f"-Wl,--version-script={os.path.join(CSRC, exports)}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, lib)


def build(verbose: bool = False, jobs: int = 5) -> str:
    """Compile every source and link libfa355.so (and the probe library)
    next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose),
                           SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB, verbose, "fa355.map")
    _link(objs[len(SOURCES):], PROBE_LIB, verbose, "fa355_probe.map")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
