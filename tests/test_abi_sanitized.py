"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is built a second time with -fsanitize=address,undefined on its
host code only (each flag behind -Xarch_host; the kernels are compiled as
usual), and the host-side ABI tests (tests/test_abi_host.py: exported
symbols, every argument check and its message) run against that build in a
child process with clang's ASan runtime preloaded. Any sanitizer report
fails the test. No GPU is needed: nothing here launches a kernel.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_block_msa_amd", "csrc")
# the library's own sources and per-source flags
from sparse_attention_block_msa_amd.build import SOURCES, compile_flags  # noqa: E402
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm",
                                          "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def test_abi_host_checks_clean_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if not os.path.exists(HIPCC) or asan is None or shutil.which("ld") is None:
        pytest.skip("hipcc or clang's ASan runtime is not available")

    def compile_one(src):
        obj = tmp_path / (src + ".o")
        subprocess.run([HIPCC, *compile_flags(src), "-O2", "-g", *SAN, "-c", "-o", str(obj),
                        os.path.join(CSRC, src)],
                       check=True, capture_output=True)
        return str(obj)

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    lib = tmp_path / "libmsa_indexer_sanitized.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", str(lib),
                    *objs], check=True, capture_output=True)

    child = ("import sys; sys.path.insert(0, sys.argv[1]); "
             "import sparse_attention_block_msa_amd as msa; msa.load(sys.argv[2]); "
             "import pytest; sys.exit(pytest.main([sys.argv[3], '-q', '-p', 'no:cacheprovider']))")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", child, ROOT, str(lib),
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         env=env, capture_output=True, text=True, timeout=600, cwd=str(tmp_path))
    report = (res.stdout[-2000:] + res.stderr[-3000:])
    assert res.returncode == 0, report
    assert "passed" in res.stdout, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
