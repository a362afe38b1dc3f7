"""Build the native library ``libbsa.so`` in-tree for gfx950.

    python -m block_sparse_attention_csr_amd.build

The host pattern builder is plain C++ (g++); the kernels and their entry
points (forward.hip, backward.hip, decode.hip) are HIP (hipcc --offload-arch=gfx950).
Then tests/c/bsa_c_forward.c, a plain C program that drives the library
through its C ABI, is compiled with gcc and linked against it (``C_DEMO``).
Every build recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbsa.so")
C_DEMO_SRC = os.path.join(ROOT, "tests", "c", "bsa_c_forward.c")
C_DEMO = os.path.join(PKG, "bsa_c_forward")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
CC = os.environ.get("CC", "gcc")

# Packed fp32 VALU instructions are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators in ordinary VGPRs: no AGPR copies around each block
             "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Wno-inline-asm"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}")
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if out.strip() and verbose:
        print(out)


def build(verbose: bool = False, extra_hip_flags=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    pattern_o = os.path.join(BUILD, "pattern.o")
    sources = ("forward.hip", "backward.hip", "decode.hip")
    objs = [os.path.join(BUILD, n.replace(".hip", ".o")) for n in sources]
    _run([CXX, *CXX_FLAGS, f"-I{INCLUDE}", "-c", os.path.join(CSRC, "pattern.cpp"),
          "-o", pattern_o], verbose)
    for src, obj in zip(sources, objs):
        _run([HIPCC, *HIP_FLAGS, *(extra_hip_flags or []), f"-I{INCLUDE}", "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", pattern_o, *objs, "-o", tmp],
         verbose)
    shutil.move(tmp, LIB)
    _run([CC, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
          f"-I{INCLUDE}", f"-I{ROCM}/include", C_DEMO_SRC, "-o", C_DEMO, f"-L{PKG}",
          "-l:libbsa.so", f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,$ORIGIN:{ROCM}/lib"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
