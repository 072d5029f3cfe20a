"""Builds ``libmsa_indexer.so`` (the HIP kernels and the C ABI) for gfx950
with hipcc, in place next to this file: every source is compiled to its own
object (in parallel), then the objects are linked."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmsa_indexer.so")
SOURCES = ["msa_abi.hip", "score_decode.hip", "top16.hip", "prefill.hip", "stream_probe.hip",
           "contraction_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 ALU ops stay off for the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source flags. The prefill scorer takes block maxima of MFMA results,
# which hold no NaN (its inputs carry no NaN codes by contract); without NaN
# semantics its maxima need no canonicalising instruction per value and fold
# into v_max3_f32 (-inf keeps its meaning: only NaNs are assumed absent).
SOURCE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


def compile_flags(src: str) -> list[str]:
    """hipcc flags of one source (without -c/-o)."""
    return [*HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          out: str = LIBRARY) -> str:
    """Compiles every source under csrc/ and links them into `out`
    (atomically replaced)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory(prefix="msa_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *compile_flags(src), *(extra_flags or []), "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp_out = out + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_out, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
