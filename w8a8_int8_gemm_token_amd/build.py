"""Build libq8.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m w8a8_int8_gemm_token_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -ffp-contract=off          no implicit multiply-add fusion (the epilogues
                             and the group-128 fmaf chain are written out);
  no fast-math               '/' and sqrtf stay correctly rounded, denormals
                             are kept (the codes depend on exact quotients);
  -target-feature -packed-fp32-ops
                             plain (unpacked) fp32 VALU code only;
  -mllvm -amdgpu-mfma-vgpr-form
                             MFMA results in ordinary VGPRs, not AGPRs: the
                             per-block folds of the group-scaled and FP8
                             GEMMs read every accumulator with VALU
                             instructions, which cannot take AGPR operands
                             (one v_accvgpr_read per element and block
                             otherwise).  No kernel's occupancy changes.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq8.so")
SOURCES = [os.path.join(CSRC, "q8_abi.hip")]
# measurement kernels for the benchmark (ceilings of this board), a library
# of their own: nothing of the layer calls them
CEIL_LIB = os.path.join(PKG, "libq8_ceilings.so")
CEIL_SOURCES = [os.path.join(CSRC, "ceilings.hip")]
HEADERS = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")] + \
    [os.path.join(ROOT, "include", "q8.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(sources, lib, verbose, extra):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """Compile libq8.so and the benchmark's libq8_ceilings.so (always
    recompiles)."""
    _compile(SOURCES, LIB, verbose, extra)
    _compile(CEIL_SOURCES, CEIL_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
