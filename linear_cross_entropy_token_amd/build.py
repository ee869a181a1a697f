"""Builds libflce.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m linear_cross_entropy_token_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflce.so")
SOURCES = ["flce_kernels.hip", "flce_fused.hip", "flce_rmsnorm.hip", "flce_api.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler must not form v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "flce_c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c", "flce_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_client() -> str:
    """Compiles the plain-C test client of the ABI (C99, gcc) against LIB and the HIP runtime."""
    tmp = C_CLIENT + ".tmp"
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), C_CLIENT_SRC,
          "-L", PKG, "-lflce", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
          "-Wl,-rpath,$ORIGIN/../../linear_cross_entropy_token_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", tmp])
    os.replace(tmp, C_CLIENT)
    return C_CLIENT


def build(verbose: bool = False) -> str:
    """Compiles every source and links LIB, then the C test client.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if os.path.exists(C_CLIENT_SRC):
        build_c_client()
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
