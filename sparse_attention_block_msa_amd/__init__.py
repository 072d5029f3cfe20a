"""Python binding of ``libmsa_indexer.so``, the MI355X (gfx950) decode-time
sparse-attention block indexer.

The functions carry the C-ABI names declared in ``include/msa_indexer.h``
and only marshal arguments. They check dtype, shape, device and contiguity,
pass raw device pointers and the current HIP stream, and turn error codes
into exceptions. Every step of the computation runs in the library's HIP
kernels. PyTorch provides the device memory and the streams.

The operations follow the FlashInfer msa_ops API pages
"msa_icp_decode_index_score_sharded" (score plane),
"msa_icp_topk_select_publish" (Top16 rows) and "prepare_msa_icp_indexer"
(the decode chain score -> select -> merge and the forced init/local blocks).
fp8 tensors may be passed as ``torch.float8_e4m3fn`` or as their raw
``torch.uint8`` codes.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa_indexer.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_LAUNCH = -2
NUM_HEADS = 4
HEAD_DIM = 128
BLOCK_TOKENS = 128
TOPK = 16
ROW_WORDS = 32  # one Top16 row: 16 float32 scores then 16 int32 ids (128 bytes)

STREAM_PROBE_SINK_WORDS = 1024  # MSA_STREAM_PROBE_SINK_WORDS
STREAM_PROBE_PERSISTENT = 0     # MSA_STREAM_PROBE_PERSISTENT

EXPORTS = ("msa_score_decode", "msa_score_decode_sharded", "msa_score_select",
           "msa_top16_select", "msa_top16_select_mapped", "msa_top16_merge_dedup", "msa_top16_merge", "msa_top16_select_merge",
           "msa_score_columns", "msa_warmup", "msa_last_error", "msa_stream_read_probe",
           "msa_contraction_probe", "msa_prefill_plan_words", "msa_prefill_window_plan",
           "msa_prefill_local", "msa_prefill_merge", "msa_score_select_workspace_words",
           "msa_score_select_noalloc")

NOALLOC_SCRATCH_WORDS = 4 * 1024 * 1024  # MSA_NOALLOC_SCRATCH_WORDS

PREFILL_WINDOW_TOKENS = 64  # MSA_PREFILL_WINDOW_TOKENS
PREFILL_PLAN_HEADER_WORDS = 8
PREFILL_ITEM_WORDS = 8

# MFMA forms of msa_contraction_probe (MSA_PROBE_* in msa_indexer.h)
PROBE_BF16 = 0
PROBE_FP8_16X16X32 = 1
PROBE_F8F6F4_16X16X128 = 2


class MsaError(RuntimeError):
    """A failed call into the library (the message is msa_last_error())."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the library once. Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; "
            "g.build()' or python sparse_attention_block_msa_amd/build.py)")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.msa_score_decode.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, P, i32, P, P]
    lib.msa_score_decode.restype = ctypes.c_int
    lib.msa_score_select.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, P, i32, P, i32, i32,
                                     i32, P, P, P, i64, P, P]
    lib.msa_score_select_workspace_words.argtypes = [i32, i32, i32, i32, i32]
    lib.msa_score_select_workspace_words.restype = i64
    lib.msa_score_select.restype = ctypes.c_int
    lib.msa_score_select_noalloc.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, P, i32, P, i32,
                                             i32, i32, P, P, P, P]
    lib.msa_score_select_noalloc.restype = ctypes.c_int
    lib.msa_score_decode_sharded.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, i32, i32, P,
                                             i32, P, P]
    lib.msa_score_decode_sharded.restype = ctypes.c_int
    lib.msa_top16_select_mapped.argtypes = [P, i32, i32, P, i32, i32, i32, i32, i32, P, P, P]
    lib.msa_top16_select_mapped.restype = ctypes.c_int
    lib.msa_top16_merge_dedup.argtypes = [P, i32, i32, P, i32, i32, P, P, P]
    lib.msa_top16_merge_dedup.restype = ctypes.c_int
    lib.msa_top16_select.argtypes = [P, i32, i32, P, i32, i32, i32, P, P, P]
    lib.msa_top16_select.restype = ctypes.c_int
    lib.msa_top16_merge.argtypes = [P, i32, i32, P, i32, i32, P, P, P]
    lib.msa_top16_merge.restype = ctypes.c_int
    lib.msa_top16_select_merge.argtypes = [P, i32, i32, P, i32, i32, i32, P, P, P, P]
    lib.msa_top16_select_merge.restype = ctypes.c_int
    lib.msa_score_columns.argtypes = [i64]
    lib.msa_score_columns.restype = i32
    lib.msa_warmup.argtypes = []
    lib.msa_warmup.restype = ctypes.c_int
    lib.msa_stream_read_probe.argtypes = [P, i64, i32, P, P]
    lib.msa_stream_read_probe.restype = ctypes.c_int
    lib.msa_prefill_plan_words.argtypes = [i64, i32, i32]
    lib.msa_prefill_plan_words.restype = i64
    lib.msa_prefill_window_plan.argtypes = [P, P, i32, i32, i32, P, i64, P, P]
    lib.msa_prefill_window_plan.restype = ctypes.c_int
    lib.msa_prefill_local.argtypes = [P, P, i64, P, i64, i32, i32, P, i64, P, i32, i32, P, i32,
                                      i32, i32, P, P, P]
    lib.msa_prefill_local.restype = ctypes.c_int
    lib.msa_prefill_merge.argtypes = [P, i32, i32, P, i32, i32, P, P, P]
    lib.msa_prefill_merge.restype = ctypes.c_int
    lib.msa_contraction_probe.argtypes = [P, P, i64, i32, P, P]
    lib.msa_contraction_probe.restype = ctypes.c_int
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != MSA_OK:
        msg = load().msa_last_error()
        raise MsaError(rc, msg.decode() if msg else "")


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError(f"{name}: expected float8_e4m3fn or uint8 codes, got {t.dtype}")
    return t


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(*ts: torch.Tensor) -> None:
    dev = ts[0].device
    for t in ts:
        _need(t.is_cuda, "all tensors must be on a GPU device")
        _need(t.device == dev, "all tensors must be on the same device")


def _errors_ptr(errors):
    if errors is None:
        return None
    _need(errors.dtype == torch.int32 and errors.numel() >= 1 and errors.is_cuda,
          "errors: expected a device int32 tensor with >= 1 element")
    return errors.data_ptr()


def new_rows(*shape, device="cuda") -> torch.Tensor:
    """An int32 tensor [*shape, 32] holding Top16 rows."""
    return torch.empty((*shape, ROW_WORDS), dtype=torch.int32, device=device)


def row_scores(rows: torch.Tensor) -> torch.Tensor:
    """float32 view [..., 16] of the scores of Top16 rows."""
    return rows[..., :TOPK].view(torch.float32)


def row_ids(rows: torch.Tensor) -> torch.Tensor:
    """int32 view [..., 16] of the block ids of Top16 rows."""
    return rows[..., TOPK:]


def msa_score_columns(max_seq_len: int) -> int:
    """Plane width roundup4(ceil(max_seq_len / 128)) (host only)."""
    cols = load().msa_score_columns(int(max_seq_len))
    _check(min(cols, 0))
    return int(cols)


def msa_warmup() -> None:
    """Loads every kernel into the current device's context."""
    _check(load().msa_warmup())


def msa_stream_read_probe(src: torch.Tensor, sink: torch.Tensor, *, nbytes: int | None = None,
                          blocks_per_wave: int = 2, stream=None) -> None:
    """Measurement aid: a plain streaming read of the first `nbytes` (default
    all) of the contiguous device tensor `src`, `blocks_per_wave` (2, 4, 8 or
    16) consecutive 16 KiB blocks per wave, or STREAM_PROBE_PERSISTENT (one
    contiguous run per wave, one wave per SIMD), xoring every dword into the words
    of `sink` (int32 [>= 1024] on the device; the xor of its words is the xor
    of the bytes read)."""
    _dev(src, sink)
    _need(src.is_contiguous(), "src: contiguous")
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    _need(0 < nbytes <= total, f"nbytes must be in (0, {total}]")
    _need(sink.dtype == torch.int32 and sink.numel() >= STREAM_PROBE_SINK_WORDS and
          sink.is_contiguous(), f"sink: contiguous int32 [>= {STREAM_PROBE_SINK_WORDS}]")
    _check(load().msa_stream_read_probe(src.data_ptr(), nbytes, int(blocks_per_wave),
                                        sink.data_ptr(), _stream_handle(stream)))


def msa_contraction_probe(q: torch.Tensor, k: torch.Tensor, out: torch.Tensor, *, form: int,
                          stream=None) -> None:
    """Measurement aid: out[t, i, j] = q[t, i, :] . k[t, j, :] for e4m3fn codes
    q, k [tiles, 16, 128], through the MFMA form `form` (PROBE_*); out is
    float32 [tiles, 16, 16]."""
    q = _u8(q, "q")
    k = _u8(k, "k")
    _dev(q, k, out)
    _need(q.dim() == 3 and q.shape[1:] == (16, HEAD_DIM) and q.is_contiguous(),
          "q: contiguous [tiles, 16, 128]")
    _need(k.shape == q.shape and k.is_contiguous(), "k: contiguous, shaped like q")
    _need(out.dtype == torch.float32 and out.shape == (q.shape[0], 16, 16) and
          out.is_contiguous(), "out: contiguous float32 [tiles, 16, 16]")
    _check(load().msa_contraction_probe(q.data_ptr(), k.data_ptr(), q.shape[0], int(form),
                                        out.data_ptr(), _stream_handle(stream)))


def _score_args(index_q, index_k, block_table, seq_lens, score_out, page_size,
                decode_query_len, world_size=1):
    q = _u8(index_q, "index_q")
    k = _u8(index_k, "index_k")
    _dev(q, k, block_table, seq_lens, score_out)
    B = seq_lens.numel()
    _need(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens: int32 [B]")
    _need(q.shape == (B * decode_query_len, NUM_HEADS, HEAD_DIM) and q.is_contiguous(),
          f"index_q: expected contiguous [{B * decode_query_len}, 4, 128], got {tuple(q.shape)}")
    rows = page_size // world_size
    _need(k.dim() == 3 and k.shape[1] == rows and k.shape[2] == HEAD_DIM and k.is_contiguous(),
          f"index_k: expected contiguous [pages, {rows}, 128], got {tuple(k.shape)}")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and
          block_table.shape[0] == B and block_table.is_contiguous(),
          "block_table: contiguous int32 [B, width]")
    _need(score_out.dtype == torch.float32 and score_out.dim() == 3 and
          score_out.shape[:2] == (B * decode_query_len, NUM_HEADS) and score_out.is_contiguous(),
          "score_out: contiguous float32 [T, 4, cols]")
    return (q.data_ptr(), k.data_ptr(), k.shape[0], block_table.data_ptr(), block_table.shape[1],
            seq_lens.data_ptr(), B, page_size, decode_query_len, score_out.data_ptr(),
            score_out.shape[2])


def msa_score_decode(index_q: torch.Tensor, index_k: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, score_out: torch.Tensor, *, page_size: int,
                     decode_query_len: int, errors: torch.Tensor | None = None,
                     stream=None) -> None:
    """Writes the score plane score_out [T, 4, cols] (columns past each
    request's roundup4(ceil(seq_len/128)) untouched). See msa_indexer.h."""
    args = _score_args(index_q, index_k, block_table, seq_lens, score_out, page_size,
                       decode_query_len)
    _check(load().msa_score_decode(*args, _errors_ptr(errors), _stream_handle(stream)))


def msa_score_decode_sharded(index_q: torch.Tensor, index_k_shard: torch.Tensor,
                             block_table: torch.Tensor, seq_lens: torch.Tensor,
                             score_out: torch.Tensor, *, page_size: int, decode_query_len: int,
                             rank: int, world_size: int, errors: torch.Tensor | None = None,
                             stream=None) -> None:
    """Rank `rank`'s score plane of a cache whose pages are split by rows over
    world_size ranks: index_k_shard [pages, page_size / world_size, 128] holds
    rows [rank*R, rank*R + R) of every page; column c is the request's page c.
    See msa_indexer.h."""
    _need(world_size in (2, 4) and page_size % world_size == 0,
          "world_size must be 2 or 4")
    args = _score_args(index_q, index_k_shard, block_table, seq_lens, score_out, page_size,
                       decode_query_len, world_size)
    _check(load().msa_score_decode_sharded(*args[:9], rank, world_size, *args[9:],
                                           _errors_ptr(errors), _stream_handle(stream)))


def msa_score_select_workspace_words(batch: int, decode_query_len: int, cols: int,
                                     num_ranges: int, pool: bool = False) -> int:
    """int32 words of msa_score_select's workspace (with the pool plane when
    pool is set, i.e. for calls without a score plane)."""
    n = load().msa_score_select_workspace_words(int(batch), int(decode_query_len), int(cols),
                                                int(num_ranges), 1 if pool else 0)
    _check(min(int(n), 0))
    return int(n)


def score_select_workspace(batch: int, decode_query_len: int, cols: int, num_ranges: int,
                           pool: bool = False, device="cuda") -> torch.Tensor:
    """A zeroed int32 workspace for msa_score_select. Each launch leaves it
    zeroed, so one workspace serves every later call of these sizes or
    smaller on the same stream."""
    return torch.zeros(msa_score_select_workspace_words(batch, decode_query_len, cols,
                                                        num_ranges, pool),
                       dtype=torch.int32, device=device)


def _score_select_args(index_q, index_k, block_table, seq_lens, score_out, num_valid_pages, out,
                       page_size, decode_query_len, num_ranges, cols, merged):
    """Checked arguments of msa_score_select up to `merged` (marshalling only)."""
    q = _u8(index_q, "index_q")
    k = _u8(index_k, "index_k")
    B = seq_lens.numel()
    T = B * decode_query_len
    if score_out is not None:
        args = _score_args(index_q, index_k, block_table, seq_lens, score_out, page_size,
                           decode_query_len)
    else:
        _need(cols is not None, "cols: needed when score_out is None")
        _dev(q, k, block_table, seq_lens)
        _need(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens: int32 [B]")
        _need(q.shape == (T, NUM_HEADS, HEAD_DIM) and q.is_contiguous(),
              f"index_q: expected contiguous [{T}, 4, 128], got {tuple(q.shape)}")
        _need(k.dim() == 3 and k.shape[1] == page_size and k.shape[2] == HEAD_DIM and
              k.is_contiguous(), f"index_k: expected contiguous [pages, {page_size}, 128]")
        _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and
              block_table.shape[0] == B and block_table.is_contiguous(),
              "block_table: contiguous int32 [B, width]")
        args = (q.data_ptr(), k.data_ptr(), k.shape[0], block_table.data_ptr(),
                block_table.shape[1], seq_lens.data_ptr(), B, page_size, decode_query_len,
                None, int(cols))
    _dev(q, num_valid_pages, out)
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, num_ranges, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, {num_ranges}, 32]")
    if merged is not None:
        _dev(out, merged)
        _need(merged.dtype == torch.int32 and merged.shape == (T, NUM_HEADS, ROW_WORDS) and
              merged.is_contiguous(), f"merged: contiguous int32 [{T}, 4, 32]")
    return (*args, num_valid_pages.data_ptr())


def msa_score_select(index_q: torch.Tensor, index_k: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, score_out: torch.Tensor | None,
                     num_valid_pages: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                     *, page_size: int, decode_query_len: int, init_blocks: int,
                     local_blocks: int, num_ranges: int = 1, cols: int | None = None,
                     merged: torch.Tensor | None = None, errors: torch.Tensor | None = None,
                     stream=None) -> None:
    """Score plane (or, with score_out None, the workspace's pool of `cols`
    columns), per-range Top16 rows `out` [T, 4, R, 32] and optionally their
    merge `merged` [T, 4, 32], in one launch. `workspace` is a zeroed int32
    tensor (see score_select_workspace)."""
    args = _score_select_args(index_q, index_k, block_table, seq_lens, score_out,
                              num_valid_pages, out, page_size, decode_query_len, num_ranges,
                              cols, merged)
    _dev(out, workspace)
    _need(workspace.dtype == torch.int32 and workspace.dim() == 1 and workspace.is_contiguous(),
          "workspace: contiguous int32 [words]")
    _check(load().msa_score_select(*args, init_blocks, local_blocks, num_ranges, out.data_ptr(),
                                   merged.data_ptr() if merged is not None else None,
                                   workspace.data_ptr(), workspace.numel(), _errors_ptr(errors),
                                   _stream_handle(stream)))


def msa_score_select_noalloc(index_q: torch.Tensor, index_k: torch.Tensor,
                             block_table: torch.Tensor, seq_lens: torch.Tensor,
                             score_out: torch.Tensor | None, num_valid_pages: torch.Tensor,
                             out: torch.Tensor, *, page_size: int, decode_query_len: int,
                             init_blocks: int, local_blocks: int, num_ranges: int = 1,
                             cols: int | None = None, merged: torch.Tensor | None = None,
                             errors: torch.Tensor | None = None, stream=None) -> None:
    """msa_score_select on the library's own device scratch array (no
    workspace argument, nothing allocated); calls on one device must not
    overlap."""
    args = _score_select_args(index_q, index_k, block_table, seq_lens, score_out,
                              num_valid_pages, out, page_size, decode_query_len, num_ranges,
                              cols, merged)
    _check(load().msa_score_select_noalloc(*args, init_blocks, local_blocks, num_ranges,
                                           out.data_ptr(),
                                           merged.data_ptr() if merged is not None else None,
                                           _errors_ptr(errors), _stream_handle(stream)))


def msa_top16_select(scores: torch.Tensor, num_valid_pages: torch.Tensor, out: torch.Tensor, *,
                     init_blocks: int, local_blocks: int, num_ranges: int = 1,
                     errors: torch.Tensor | None = None, stream=None) -> None:
    """Top16 rows [T, 4, R] of scores [T, 4, cols] over R column ranges.
    `out` is an int32 tensor [T, 4, R, 32] (see new_rows)."""
    _dev(scores, num_valid_pages, out)
    _need(scores.dtype == torch.float32 and scores.dim() == 3 and scores.shape[1] == NUM_HEADS and
          scores.is_contiguous(), "scores: contiguous float32 [T, 4, cols]")
    T, _, cols = scores.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, num_ranges, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, {num_ranges}, 32]")
    lib = load()
    _check(lib.msa_top16_select(scores.data_ptr(), T, cols, num_valid_pages.data_ptr(),
                                init_blocks, local_blocks, num_ranges, out.data_ptr(),
                                _errors_ptr(errors), _stream_handle(stream)))


def msa_top16_select_mapped(scores: torch.Tensor, num_valid_pages: torch.Tensor,
                            out: torch.Tensor, *, init_blocks: int, local_blocks: int,
                            num_ranges: int = 1, index_scale: int = 1, index_offset: int = 0,
                            errors: torch.Tensor | None = None, stream=None) -> None:
    """Top16 rows [T, 4, R] with plane column c standing for global block id
    index_scale * c + index_offset."""
    _dev(scores, num_valid_pages, out)
    _need(scores.dtype == torch.float32 and scores.dim() == 3 and scores.shape[1] == NUM_HEADS and
          scores.is_contiguous(), "scores: contiguous float32 [T, 4, cols]")
    T, _, cols = scores.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, num_ranges, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, {num_ranges}, 32]")
    _check(load().msa_top16_select_mapped(scores.data_ptr(), T, cols, num_valid_pages.data_ptr(),
                                          init_blocks, local_blocks, num_ranges, index_scale,
                                          index_offset, out.data_ptr(), _errors_ptr(errors),
                                          _stream_handle(stream)))


def msa_top16_merge_dedup(partial: torch.Tensor, num_valid_pages: torch.Tensor,
                          out: torch.Tensor, *, init_blocks: int, local_blocks: int,
                          errors: torch.Tensor | None = None, stream=None) -> None:
    """Merges partial rows [T, 4, R, 32] in any order, an id in several rows
    keeping its highest score, into rows [T, 4, 32] (R <= 64)."""
    _dev(partial, num_valid_pages, out)
    _need(partial.dtype == torch.int32 and partial.dim() == 4 and partial.shape[1] == NUM_HEADS
          and partial.shape[3] == ROW_WORDS and partial.is_contiguous(),
          "partial: contiguous int32 [T, 4, R, 32]")
    T, _, R, _ = partial.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, 32]")
    _check(load().msa_top16_merge_dedup(partial.data_ptr(), T, R, num_valid_pages.data_ptr(),
                                        init_blocks, local_blocks, out.data_ptr(),
                                        _errors_ptr(errors), _stream_handle(stream)))


def msa_top16_merge(partial: torch.Tensor, num_valid_pages: torch.Tensor, out: torch.Tensor, *,
                    init_blocks: int, local_blocks: int, errors: torch.Tensor | None = None,
                    stream=None) -> None:
    """Merges partial rows [T, 4, R, 32] into rows [T, 4, 32]."""
    _dev(partial, num_valid_pages, out)
    _need(partial.dtype == torch.int32 and partial.dim() == 4 and partial.shape[1] == NUM_HEADS
          and partial.shape[3] == ROW_WORDS and partial.is_contiguous(),
          "partial: contiguous int32 [T, 4, R, 32]")
    T, _, R, _ = partial.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, 32]")
    lib = load()
    _check(lib.msa_top16_merge(partial.data_ptr(), T, R, num_valid_pages.data_ptr(), init_blocks,
                               local_blocks, out.data_ptr(), _errors_ptr(errors),
                               _stream_handle(stream)))


def msa_top16_select_merge(scores: torch.Tensor, num_valid_pages: torch.Tensor, out: torch.Tensor,
                           *, init_blocks: int, local_blocks: int, num_ranges: int,
                           partial: torch.Tensor | None = None,
                           errors: torch.Tensor | None = None, stream=None) -> None:
    """Select over num_ranges column ranges and merge, in one launch: `out`
    [T, 4, 32] receives the merged rows and `partial` [T, 4, R, 32] (optional)
    the per-range rows."""
    _dev(scores, num_valid_pages, out)
    _need(scores.dtype == torch.float32 and scores.dim() == 3 and scores.shape[1] == NUM_HEADS and
          scores.is_contiguous(), "scores: contiguous float32 [T, 4, cols]")
    T, _, cols = scores.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (T,),
          "num_valid_pages: int32 [T]")
    _need(out.dtype == torch.int32 and out.shape == (T, NUM_HEADS, ROW_WORDS) and
          out.is_contiguous(), f"out: contiguous int32 [{T}, 4, 32]")
    if partial is not None:
        _dev(scores, partial)
        _need(partial.dtype == torch.int32 and
              partial.shape == (T, NUM_HEADS, num_ranges, ROW_WORDS) and partial.is_contiguous(),
              f"partial: contiguous int32 [{T}, 4, {num_ranges}, 32]")
    lib = load()
    _check(lib.msa_top16_select_merge(
        scores.data_ptr(), T, cols, num_valid_pages.data_ptr(), init_blocks, local_blocks,
        num_ranges, partial.data_ptr() if partial is not None else None, out.data_ptr(),
        _errors_ptr(errors), _stream_handle(stream)))


# ---------------------------------------------------------------------------
# prefill chain ("prepare_msa_icp_indexer", prefill bullet)
# ---------------------------------------------------------------------------

def msa_prefill_plan_words(num_tokens: int, batch: int, cols: int) -> int:
    """int32 words of a plan that holds any prefill step of at most
    num_tokens query tokens over batch requests on a plane of cols columns."""
    n = load().msa_prefill_plan_words(int(num_tokens), int(batch), int(cols))
    _check(min(int(n), 0))
    return int(n)


def new_prefill_plan(num_tokens: int, batch: int, cols: int, device="cuda") -> torch.Tensor:
    """An int32 plan buffer sized by msa_prefill_plan_words."""
    return torch.empty(msa_prefill_plan_words(num_tokens, batch, cols), dtype=torch.int32,
                       device=device)


def msa_prefill_window_plan(qo_indptr: torch.Tensor, seq_lens: torch.Tensor,
                            plan: torch.Tensor, *, num_tokens: int, cols: int,
                            errors: torch.Tensor | None = None, stream=None) -> None:
    """Builds the plan of one prefill step: request b's chunk is rows
    [qo_indptr[b], qo_indptr[b+1]) of index_q ([num_tokens, 4, 128])."""
    _dev(qo_indptr, seq_lens, plan)
    B = seq_lens.numel()
    _need(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens: int32 [B]")
    _need(qo_indptr.dtype == torch.int32 and qo_indptr.shape == (B + 1,) and
          qo_indptr.is_contiguous(), f"qo_indptr: contiguous int32 [{B + 1}]")
    _need(plan.dtype == torch.int32 and plan.dim() == 1 and plan.is_contiguous(),
          "plan: contiguous int32 [words]")
    _check(load().msa_prefill_window_plan(qo_indptr.data_ptr(), seq_lens.data_ptr(), B,
                                          int(num_tokens), int(cols), plan.data_ptr(),
                                          plan.numel(), _errors_ptr(errors),
                                          _stream_handle(stream)))


def msa_prefill_local(index_q: torch.Tensor, index_k: torch.Tensor, block_table: torch.Tensor,
                      plan: torch.Tensor, score_scratch: torch.Tensor,
                      num_valid_pages: torch.Tensor, carrier: torch.Tensor, *, page_size: int,
                      init_blocks: int, local_blocks: int, num_ranges: int = 1,
                      errors: torch.Tensor | None = None, stream=None) -> None:
    """Scores one prefill step into score_scratch [Tq, 4, cols] and writes
    its Top16 carrier rows [Tq, 4, R, 32]."""
    q = _u8(index_q, "index_q")
    k = _u8(index_k, "index_k")
    _dev(q, k, block_table, plan, score_scratch, num_valid_pages, carrier)
    _need(q.dim() == 3 and q.shape[1:] == (NUM_HEADS, HEAD_DIM) and q.is_contiguous(),
          "index_q: contiguous [Tq, 4, 128]")
    Tq = q.shape[0]
    _need(k.dim() == 3 and k.shape[1] == page_size and k.shape[2] == HEAD_DIM and
          k.is_contiguous(), f"index_k: contiguous [pages, {page_size}, 128]")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and
          block_table.is_contiguous(), "block_table: contiguous int32 [B, width]")
    _need(plan.dtype == torch.int32 and plan.dim() == 1 and plan.is_contiguous(),
          "plan: contiguous int32 [words]")
    _need(score_scratch.dtype == torch.float32 and score_scratch.dim() == 3 and
          score_scratch.shape[:2] == (Tq, NUM_HEADS) and score_scratch.is_contiguous(),
          f"score_scratch: contiguous float32 [{Tq}, 4, cols]")
    cols = score_scratch.shape[2]
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (Tq,),
          f"num_valid_pages: int32 [{Tq}]")
    _need(carrier.dtype == torch.int32 and carrier.shape == (Tq, NUM_HEADS, num_ranges, ROW_WORDS)
          and carrier.is_contiguous(), f"carrier: contiguous int32 [{Tq}, 4, {num_ranges}, 32]")
    _check(load().msa_prefill_local(q.data_ptr(), k.data_ptr(), k.shape[0],
                                    block_table.data_ptr(), block_table.shape[1],
                                    block_table.shape[0], page_size,
                                    plan.data_ptr(), plan.numel(), score_scratch.data_ptr(), Tq,
                                    cols, num_valid_pages.data_ptr(), init_blocks, local_blocks,
                                    num_ranges, carrier.data_ptr(), _errors_ptr(errors),
                                    _stream_handle(stream)))


def msa_prefill_merge(received: torch.Tensor, num_valid_pages: torch.Tensor,
                      output: torch.Tensor, *, init_blocks: int, local_blocks: int,
                      errors: torch.Tensor | None = None, stream=None) -> None:
    """Merges the carrier rows [Tq, 4, R, 32] into output rows [Tq, 4, 32]."""
    _dev(received, num_valid_pages, output)
    _need(received.dtype == torch.int32 and received.dim() == 4 and
          received.shape[1] == NUM_HEADS and received.shape[3] == ROW_WORDS and
          received.is_contiguous(), "received: contiguous int32 [Tq, 4, R, 32]")
    Tq, _, R, _ = received.shape
    _need(num_valid_pages.dtype == torch.int32 and num_valid_pages.shape == (Tq,),
          "num_valid_pages: int32 [Tq]")
    _need(output.dtype == torch.int32 and output.shape == (Tq, NUM_HEADS, ROW_WORDS) and
          output.is_contiguous(), f"output: contiguous int32 [{Tq}, 4, 32]")
    _check(load().msa_prefill_merge(received.data_ptr(), Tq, R, num_valid_pages.data_ptr(),
                                    init_blocks, local_blocks, output.data_ptr(),
                                    _errors_ptr(errors), _stream_handle(stream)))
