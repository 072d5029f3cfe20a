"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C source is built a second time with
-fsanitize=address,undefined (no recovery) and every entry point runs on
small inputs that reach its edge paths: empty and short requests, both page
sizes, every decode_query_len, block-table entries out of range, a plane too
narrow, num_valid_pages out of range, many ranges, sharded planes and mapped
ids. The run happens in a child process with the ASan runtime preloaded (the
Python interpreter itself is not instrumented, so leak checking is off); any
sanitizer report fails the test. CPU only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "msa_oracle.c")

DRIVER = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, sys.argv[2])
    import oracle

    o = oracle.Oracle(sys.argv[1])
    o.set_num_threads(4)
    rng = np.random.default_rng(5)

    def codes(shape):
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] ^= 1  # no NaN codes
        return c

    assert o.e4m3fn_table().shape == (256,)
    o.dots(codes((9, 128)), codes((9, 128)))
    for page_size in (128, 256):
        for dql in (1, 3, 8):
            seqs = np.array([0, 1, dql, 127, 128, 129, 300, 1000], dtype=np.int32)
            B = seqs.shape[0]
            pages = [(int(s) + page_size - 1) // page_size for s in seqs]
            pool = sum(pages) + 1
            k = codes((pool, page_size, 128))
            q = codes((B * dql, 4, 128))
            width = max(pages) + 1
            bt = np.full((B, width), pool - 1, dtype=np.int32)
            off = 0
            for b, n in enumerate(pages):
                bt[b, :n] = np.arange(off, off + n)
                off += n
            bad = bt.copy()
            bad[6, 0] = -1
            bad[7, 1] = pool + 5
            cols = max(4, (max((int(s) + 127) // 128 for s in seqs) + 3) // 4 * 4)
            for table in (bt, bad):
                for c in (cols, 4):  # 4: too narrow for the long requests
                    plane, amax, nbad = o.score_decode(q, k, table, seqs, page_size=page_size,
                                                       decode_query_len=dql, cols=c,
                                                       want_amax=True)
            plane = np.nan_to_num(plane, nan=-1.0)
            rows = np.arange(0, B * dql * 4, 7, dtype=np.int64)
            cidx = (rows * 3) % cols
            o.score_sampled(q, k, bt, seqs, rows, cidx, page_size=page_size,
                            decode_query_len=dql)
            T = B * dql
            nvp = rng.integers(-2, cols + 3, size=T).astype(np.int32)
            for R in (1, 3, cols):
                ps, pi, _ = o.top16_select(plane, nvp, init_blocks=2, local_blocks=3,
                                           num_ranges=R)
                o.top16_merge(ps, pi, np.clip(nvp, 0, cols), init_blocks=2, local_blocks=3)
            for ws in (2, 4):
                r = page_size // ws
                for rank in range(ws):
                    shard = np.ascontiguousarray(k[:, rank * r:(rank + 1) * r, :])
                    sp, _, _ = o.score_decode_sharded(q, shard, bad, seqs, page_size=page_size,
                                                      decode_query_len=dql, rank=rank,
                                                      world_size=ws, cols=cols, want_amax=True)
                    sp = np.nan_to_num(sp, nan=-1.0)
                    scale, offset = (1, 0) if page_size == 128 else (2, rank * 2 // ws)
                    o.top16_select_mapped(sp, nvp, init_blocks=1, local_blocks=2, num_ranges=2,
                                          index_scale=scale, index_offset=offset)
            # prefill chunks: empty, single-token, whole-request and ragged chunks
            qlens = np.minimum(np.array([0, 1, 1, 127, 5, 129, 300, 999], dtype=np.int64), seqs)
            qo = np.zeros(B + 1, dtype=np.int32)
            qo[1:] = np.cumsum(qlens)
            qp = codes((int(qo[-1]), 4, 128))
            for table in (bt, bad):
                for c in (cols, 4):
                    o.score_prefill(qp, k, table, qo, seqs, page_size=page_size, cols=c,
                                    want_amax=True)
            o.score_prefill(qp, k, bt, qo, seqs, page_size=page_size, cols=cols,
                            tokens=np.array([int(qo[-1]) - 1, 0, 3], dtype=np.int64))
    print("sanitized oracle ok")
""")


def _asan_runtime():
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    path = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return os.path.realpath(path) if path and os.path.exists(path) else None


def test_oracle_clean_under_address_and_undefined_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc with the ASan runtime is not available")
    lib = tmp_path / "liboracle_sanitized.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(lib), SOURCE, "-lm"], check=True)
    driver = tmp_path / "driver.py"
    driver.write_text(DRIVER)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, str(driver), str(lib), ROOT], env=env,
                         capture_output=True, text=True, timeout=600)
    report = res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "sanitized oracle ok" in res.stdout, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
