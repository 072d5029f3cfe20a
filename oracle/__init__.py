"""Plain CPU oracle for the decode-time sparse-attention block indexer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it. The product path (the HIP library and its
Python binding) never imports it, and it shares no code with that path.

This module is a thin ctypes wrapper over ``msa_oracle.c`` (numpy arrays in,
numpy arrays out). Every definition lives in the C file, which cites the
FlashInfer msa_ops pages it follows:

* "flashinfer.msa_ops.msa_icp_decode_index_score_sharded" (description,
  index_q, index_k, block_table, seq_lens, score_out): the score plane;
* "flashinfer.msa_ops.msa_icp_topk_select_publish" (description, scores,
  num_valid_pages): the Top16 row;
* "flashinfer.msa_ops.prepare_msa_icp_indexer" (decode; init_blocks,
  local_blocks): the decode chain and its merge, the forced blocks.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

HEADS = 4
DIM = 128
TOPK = 16


class Oracle:
    """ctypes binding of one build of ``msa_oracle.c``."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(lib_path):
            from . import build as _build

            _build.build()
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_e4m3fn_table.argtypes = [P]
        lib.oracle_e4m3fn_table.restype = None
        lib.oracle_dots.argtypes = [P, P, i64, P, P]
        lib.oracle_dots.restype = None
        lib.oracle_written_columns.argtypes = [i64]
        lib.oracle_written_columns.restype = i64
        lib.oracle_score_decode.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, P, i32, P]
        lib.oracle_score_decode.restype = i64
        lib.oracle_score_sampled.argtypes = [P, P, i64, P, i64, P, i32, i32, P, P, i64, P, P]
        lib.oracle_score_sampled.restype = i64
        lib.oracle_top16_select.argtypes = [P, i32, i32, P, i32, i32, i32, P]
        lib.oracle_top16_select.restype = i64
        lib.oracle_top16_merge.argtypes = [P, i32, i32, P, i32, i32, P]
        lib.oracle_top16_merge.restype = i64
        lib.oracle_written_columns_sharded.argtypes = [i64, i32]
        lib.oracle_written_columns_sharded.restype = i64
        lib.oracle_score_decode_sharded.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, i32,
                                                    i32, P, i32, P]
        lib.oracle_score_decode_sharded.restype = i64
        lib.oracle_top16_select_mapped.argtypes = [P, i32, i32, P, i32, i32, i32, i32, i32, P]
        lib.oracle_top16_select_mapped.restype = i64
        lib.oracle_score_prefill.argtypes = [P, P, i64, P, i64, P, P, i32, i32, P, i64, P, i32,
                                             P]
        lib.oracle_score_prefill.restype = i64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib
        self.path = lib_path

    def e4m3fn_table(self) -> np.ndarray:
        """float64[256]: decoded value of every e4m3fn byte code (NaN codes -> nan)."""
        out = np.empty(256, dtype=np.float64)
        self.lib.oracle_e4m3fn_table(_ptr(out))
        return out

    def dots(self, q: np.ndarray, k: np.ndarray):
        """Row-wise q[i] . k[i] of uint8 e4m3fn rows [n, 128].

        Returns (float32[n] rounded once, float64[n] exact)."""
        q = _c(q, np.uint8).reshape(-1, DIM)
        k = _c(k, np.uint8).reshape(-1, DIM)
        assert q.shape == k.shape
        n = q.shape[0]
        f = np.empty(n, dtype=np.float32)
        e = np.empty(n, dtype=np.float64)
        self.lib.oracle_dots(_ptr(q), _ptr(k), n, _ptr(f), _ptr(e))
        return f, e

    def set_num_threads(self, n: int) -> None:
        """Threads later plane calls may use (takes effect at once)."""
        self.lib.oracle_set_num_threads(int(n))

    def num_threads(self) -> int:
        """OpenMP threads the plane functions use."""
        return int(self.lib.oracle_num_threads())

    def written_columns(self, seq_len: int) -> int:
        return int(self.lib.oracle_written_columns(int(seq_len)))

    def score_decode(self, index_q, index_k, block_table, seq_lens, *, page_size: int,
                     decode_query_len: int, cols: int, plane: np.ndarray | None = None,
                     want_amax: bool = False):
        """Score plane [T, 4, cols] float32 (written columns only; the rest of
        `plane` is left as given, default all NaN). Returns (plane, amax|None, bad)."""
        q = _c(index_q, np.uint8)
        k = _c(index_k, np.uint8)
        bt = _c(block_table, np.int32)
        sl = _c(seq_lens, np.int32)
        batch = sl.shape[0]
        T = batch * decode_query_len
        assert q.size == T * HEADS * DIM
        assert k.ndim == 3 and k.shape[1] == page_size and k.shape[2] == DIM
        if plane is None:
            plane = np.full((T, HEADS, cols), np.nan, dtype=np.float32)
        else:
            plane = np.array(plane, dtype=np.float32, order="C", copy=True)
        amax = np.zeros((T, HEADS, cols), dtype=np.float64) if want_amax else None
        bad = self.lib.oracle_score_decode(
            _ptr(q), _ptr(k), k.shape[0], _ptr(bt), bt.shape[1], _ptr(sl), batch, page_size,
            decode_query_len, _ptr(plane), cols, _ptr(amax) if want_amax else None)
        return plane, amax, int(bad)

    def score_sampled(self, index_q, index_k, block_table, seq_lens, rows, cols_idx, *,
                      page_size: int, decode_query_len: int):
        """Plane elements (rows[i], cols_idx[i]), row = (b*dql + j)*4 + h.
        Returns (float32[n], amax float64[n], bad)."""
        q = _c(index_q, np.uint8)
        k = _c(index_k, np.uint8)
        bt = _c(block_table, np.int32)
        sl = _c(seq_lens, np.int32)
        r = _c(rows, np.int64)
        c = _c(cols_idx, np.int64)
        n = r.shape[0]
        s = np.empty(n, dtype=np.float32)
        a = np.empty(n, dtype=np.float64)
        bad = self.lib.oracle_score_sampled(
            _ptr(q), _ptr(k), k.shape[0], _ptr(bt), bt.shape[1], _ptr(sl), page_size,
            decode_query_len, _ptr(r), _ptr(c), n, _ptr(s), _ptr(a))
        return s, a, int(bad)

    def score_prefill(self, index_q, index_k, block_table, qo_indptr, seq_lens, *,
                      page_size: int, cols: int, tokens=None, plane: np.ndarray | None = None,
                      want_amax: bool = False):
        """Prefill score plane: request b's query tokens are rows
        [qo_indptr[b], qo_indptr[b+1]) of index_q [Tq, 4, 128], token j at
        position seq_len[b] - q_len_b + j. Returns (plane [n, 4, cols],
        amax|None, bad) for every token (n = Tq) or for the token rows in
        `tokens` (in that order); unwritten columns keep `plane`'s values
        (default NaN)."""
        q = _c(index_q, np.uint8)
        k = _c(index_k, np.uint8)
        bt = _c(block_table, np.int32)
        qo = _c(qo_indptr, np.int32)
        sl = _c(seq_lens, np.int32)
        batch = sl.shape[0]
        assert qo.shape == (batch + 1,)
        total = int(qo[-1])
        assert q.size == total * HEADS * DIM
        assert k.ndim == 3 and k.shape[1] == page_size and k.shape[2] == DIM
        tk = None if tokens is None else _c(tokens, np.int64)
        n = total if tk is None else tk.shape[0]
        if plane is None:
            plane = np.full((n, HEADS, cols), np.nan, dtype=np.float32)
        else:
            plane = np.array(plane, dtype=np.float32, order="C", copy=True)
        assert plane.shape == (n, HEADS, cols)
        amax = np.zeros((n, HEADS, cols), dtype=np.float64) if want_amax else None
        bad = self.lib.oracle_score_prefill(
            _ptr(q), _ptr(k), k.shape[0], _ptr(bt), bt.shape[1], _ptr(qo), _ptr(sl), batch,
            page_size, None if tk is None else _ptr(tk), n, _ptr(plane), cols,
            _ptr(amax) if want_amax else None)
        if bad < 0:
            raise ValueError("oracle_score_prefill: invalid arguments")
        return plane, amax, int(bad)

    def written_columns_sharded(self, seq_len: int, page_size: int) -> int:
        return int(self.lib.oracle_written_columns_sharded(int(seq_len), int(page_size)))

    def score_decode_sharded(self, index_q, index_k_shard, block_table, seq_lens, *,
                             page_size: int, decode_query_len: int, rank: int, world_size: int,
                             cols: int, plane: np.ndarray | None = None,
                             want_amax: bool = False):
        """Rank `rank`'s plane [T, 4, cols] of a cache whose pages are split
        by rows over world_size ranks (index_k_shard [pages, page_size /
        world_size, 128]). Returns (plane, amax|None, bad)."""
        q = _c(index_q, np.uint8)
        k = _c(index_k_shard, np.uint8)
        bt = _c(block_table, np.int32)
        sl = _c(seq_lens, np.int32)
        batch = sl.shape[0]
        T = batch * decode_query_len
        assert q.size == T * HEADS * DIM
        assert k.ndim == 3 and k.shape[1] * world_size == page_size and k.shape[2] == DIM
        if plane is None:
            plane = np.full((T, HEADS, cols), np.nan, dtype=np.float32)
        else:
            plane = np.array(plane, dtype=np.float32, order="C", copy=True)
        amax = np.zeros((T, HEADS, cols), dtype=np.float64) if want_amax else None
        bad = self.lib.oracle_score_decode_sharded(
            _ptr(q), _ptr(k), k.shape[0], _ptr(bt), bt.shape[1], _ptr(sl), batch, page_size,
            decode_query_len, rank, world_size, _ptr(plane), cols,
            _ptr(amax) if want_amax else None)
        if bad < 0:
            raise ValueError("oracle_score_decode_sharded: invalid arguments")
        return plane, amax, int(bad)

    def top16_select_mapped(self, scores, num_valid_pages, *, init_blocks: int,
                            local_blocks: int, num_ranges: int = 1, index_scale: int = 1,
                            index_offset: int = 0):
        """Top16 rows with plane column c standing for global id
        index_scale * c + index_offset. Returns (scores, ids, bad) as
        top16_select."""
        s = _c(scores, np.float32)
        T, H, cols = s.shape
        assert H == HEADS
        nvp = _c(num_valid_pages, np.int32)
        assert nvp.shape == (T,)
        out = np.empty((T, HEADS, num_ranges), dtype=_ROW)
        bad = self.lib.oracle_top16_select_mapped(_ptr(s), T, cols, _ptr(nvp), init_blocks,
                                                  local_blocks, num_ranges, index_scale,
                                                  index_offset, _ptr(out))
        if bad < 0:
            raise ValueError("oracle_top16_select_mapped: invalid arguments")
        return out["score"].copy(), out["id"].copy(), int(bad)

    def top16_select(self, scores, num_valid_pages, *, init_blocks: int, local_blocks: int,
                     num_ranges: int = 1):
        """Top16 rows of every (token, head, range). Returns
        (scores float32[T,4,R,16], ids int32[T,4,R,16], bad)."""
        s = _c(scores, np.float32)
        T, H, cols = s.shape
        assert H == HEADS
        nvp = _c(num_valid_pages, np.int32)
        assert nvp.shape == (T,)
        out = np.empty((T, HEADS, num_ranges), dtype=_ROW)
        bad = self.lib.oracle_top16_select(_ptr(s), T, cols, _ptr(nvp), init_blocks,
                                           local_blocks, num_ranges, _ptr(out))
        if bad < 0:
            raise ValueError("oracle_top16_select: invalid arguments")
        return out["score"].copy(), out["id"].copy(), int(bad)

    def top16_merge(self, part_scores, part_ids, num_valid_pages, *, init_blocks: int,
                    local_blocks: int):
        """Merge of R partial rows per (token, head). part_*: [T, 4, R, 16].
        Returns (scores float32[T,4,16], ids int32[T,4,16], rows_missing_forced)."""
        ps = _c(part_scores, np.float32)
        pi = _c(part_ids, np.int32)
        T, H, R, K = ps.shape
        assert H == HEADS and K == TOPK and pi.shape == ps.shape
        rows = np.empty((T, HEADS, R), dtype=_ROW)
        rows["score"] = ps
        rows["id"] = pi
        nvp = _c(num_valid_pages, np.int32)
        out = np.empty((T, HEADS), dtype=_ROW)
        missing = self.lib.oracle_top16_merge(_ptr(rows), T, R, _ptr(nvp), init_blocks,
                                              local_blocks, _ptr(out))
        if missing < 0:
            raise ValueError("oracle_top16_merge: invalid arguments")
        return out["score"].copy(), out["id"].copy(), int(missing)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


_ROW = np.dtype([("score", np.float32, (TOPK,)), ("id", np.int32, (TOPK,))])

_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def set_threads(n: int) -> None:
    """OpenMP thread count for the plane functions (read when the library
    first starts its thread pool, so set it before the first call)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))


def e4m3fn_table():
    return default().e4m3fn_table()


def dots(q, k):
    return default().dots(q, k)


def written_columns(seq_len):
    return default().written_columns(seq_len)


def score_decode(*args, **kwargs):
    return default().score_decode(*args, **kwargs)


def score_sampled(*args, **kwargs):
    return default().score_sampled(*args, **kwargs)


def top16_select(*args, **kwargs):
    return default().top16_select(*args, **kwargs)


def top16_merge(*args, **kwargs):
    return default().top16_merge(*args, **kwargs)


def written_columns_sharded(seq_len, page_size):
    return default().written_columns_sharded(seq_len, page_size)


def score_decode_sharded(*args, **kwargs):
    return default().score_decode_sharded(*args, **kwargs)


def top16_select_mapped(*args, **kwargs):
    return default().top16_select_mapped(*args, **kwargs)


def score_prefill(*args, **kwargs):
    return default().score_prefill(*args, **kwargs)
