"""Builds the CPU oracle (``liboracle.so``) with gcc. Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "msa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")


def build(src: str = SOURCE, out: str = LIBRARY, verbose: bool = False) -> str:
    """Compiles `src` into the shared library `out` (atomically replaced)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
