"""Build liboracle.so from oracle.c with gcc (host code only, OpenMP).

TEST INFRASTRUCTURE ONLY; see the package docstring.
Run as ``python -m oracle.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")


def library_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle.c; returns the path of the shared library.

    -ffp-contract=off keeps every addition a separately rounded FP32 add (the
    products of BF16 values are exact, so this changes nothing but makes the
    intent explicit); no -ffast-math, so the k-ascending order is kept.
    """
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O3", "-mavx2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SOURCE]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
