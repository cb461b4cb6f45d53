"""Build libgemm_rs.so (the HIP kernels + C ABI) in-tree for gfx950.

Run as ``python -m tensor_gemm_reduce_amd.build``.  hipcc cross-compiles the
device code for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def library_path() -> str:
    return os.path.join(PKG, "libgemm_rs.so")


def sources():
    return [os.path.join(CSRC, "gemm_rs.hip")]


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep hand-free of packed FP32 instructions (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=off", "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False, extra=()) -> str:
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *compile_flags(), *extra, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
