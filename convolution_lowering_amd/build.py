"""Compile the HIP library libconvlower.so for gfx950, in-tree.

Run as ``python -m convolution_lowering_amd.build``.  Every call recompiles
from source.  The main-loop source igemm_inst.hip is compiled once per
(dtype, feed) pair so the template variants build in parallel.
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libconvlower.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _units():
    units = [("conv_api", "conv_api.cpp", []),
             ("igemm_dispatch", "igemm_dispatch.hip", []),
             ("lowering_kernels", "lowering_kernels.hip", []),
             ("direct_conv", "direct_conv.hip", []),
             ("patch_conv", "patch_conv.hip", []),
             ("igemm_ablate", "igemm_ablate.hip", [])]
    for dt, tag in ((1, "bf16"), (2, "f16"), (0, "f32")):  # IGEMM_DTYPE: 0 fp32, 1 bf16, 2 fp16
        for feed in range(10):  # the Feed values of conv_internal.h
            units.append((f"igemm_{tag}_feed{feed}", "igemm_inst.hip",
                          [f"-DIGEMM_DTYPE={dt}", f"-DIGEMM_FEED={feed}"]))
    # fp8 e4m3 (IGEMM_DTYPE 3): the window-row feed (7) only
    units.append(("igemm_fp8_feed7", "igemm_inst.hip", ["-DIGEMM_DTYPE=3", "-DIGEMM_FEED=7"]))
    return units


def _compile(unit):
    name, src, defs = unit
    out = os.path.join(OBJ, name + ".o")
    cmd = [HIPCC] + FLAGS + defs + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {name} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, _units()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # Every kernel entry point the host code launches must be defined in the
    # library (a template kernel whose host stub was not emitted would
    # otherwise only show up as a load failure on the GPU).
    r = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.strip() for ln in r.stdout.splitlines() if "convlower::" in ln]
    if missing:
        raise RuntimeError("undefined library symbols:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
