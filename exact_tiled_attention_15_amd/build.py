"""Compile the gfx950 HIP library ``libfa.so`` in-tree with hipcc.

Usage: ``python -m exact_tiled_attention_15_amd.build [--asm DIR]``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = [os.path.join(CSRC, "fa_kernels.hip"), os.path.join(CSRC, "fa_bwd.hip"),
           os.path.join(CSRC, "fa_api.cpp")]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
# Kernel units only: the kernels never need NaN-preserving max/min (no
# input-quieting v_max x, x before each v_max of an MFMA result).  The C ABI
# unit keeps IEEE comparisons, which its argument checks (NaN scales) rely on.
KERNEL = ["-fno-honor-nans"]
# MFMA destinations and accumulators in VGPRs instead of AGPRs.
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]

# Compile units: (object name, source, extra flags).  The two kernel sources
# are each compiled twice; a macro picks which head dimensions a unit holds,
# so that only the kernels that gain from VGPR-form MFMAs get that flag (the
# forward at D = 256 and the backward at D = 32 and 64; the forward at D = 64
# and the backward at D = 128 lose with it).
UNITS = [
    ("fwd", os.path.join(CSRC, "fa_kernels.hip"), [*KERNEL]),
    ("fwd_d256", os.path.join(CSRC, "fa_kernels.hip"), [*KERNEL, "-DFA_FWD_D256", *VGPR_MFMA]),
    ("bwd", os.path.join(CSRC, "fa_bwd.hip"), [*KERNEL]),
    ("bwd_small_d", os.path.join(CSRC, "fa_bwd.hip"), [*KERNEL, "-DFA_BWD_SMALL_D", *VGPR_MFMA]),
    ("bwd32", os.path.join(CSRC, "fa_bwd32.hip"), [*KERNEL]),
    ("api", os.path.join(CSRC, "fa_api.cpp"), []),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd, cwd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build_library(verbose: bool = False, asm_dir: str | None = None) -> str:
    """Compile every unit to an object (in parallel), then link libfa.so.

    With asm_dir, the intermediate files (device assembly included) of each
    unit are kept there, named after the unit.
    """
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory() as tmp:
        objdir = asm_dir or tmp
        if asm_dir:
            os.makedirs(asm_dir, exist_ok=True)
        objs = [os.path.join(objdir, name + ".o") for name, _, _ in UNITS]
        cmds = []
        for (name, src, extra), obj in zip(UNITS, objs):
            cmd = [hipcc(), *FLAGS, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
            if asm_dir:
                cmd.append("-save-temps=obj")
            cmds.append(cmd)
        with ThreadPoolExecutor(len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, objdir, verbose), cmds))
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp"], objdir, verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    asm = None
    if "--asm" in sys.argv:
        asm = sys.argv[sys.argv.index("--asm") + 1]
    print(build_library(verbose=True, asm_dir=asm))
