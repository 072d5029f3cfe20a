"""Seeded synthetic inputs for the decode-time block indexer.

Both the HIP path (tests, bench) and the CPU oracle take their inputs from
here. This module holds no arithmetic of the method itself: it only draws
sequence lengths, page assignments and fp8 codes, and sizes buffers.

Shapes and dtypes follow the FlashInfer msa_ops pages
("flashinfer.msa_ops.msa_icp_decode_index_score_sharded": index_q
float8_e4m3fn [B*decode_query_len, 4, 128]; index_k [pages, page_size, 128]
(full page rows on one device); block_table int32 [B, >= pages per request];
seq_lens int32 [B]; "flashinfer.msa_ops.msa_icp_topk_select_publish":
num_valid_pages int32 [T] of B128 block counts).

Recipe (the same for every configuration; ``seed = 1000 + config number``):

1. ``torch.Generator`` on the CPU, seeded.
2. Draw order: sequence lengths, page permutation, outlier blocks, q, k.
3. Sequence lengths: fixed, integer-uniform inclusive ``randint(a, b + 1)``,
   or log-uniform ``floor(exp(U[ln a, ln b]))``.
4. Pages: a pool is permuted with ``randperm``; request b takes the next
   ``ceil(seq_len_b / page_size)`` pages of the permutation. One extra
   *poison page* (index = pool size) holds the code 0x7E (448.0) everywhere;
   every unused block_table slot points at it, and every row of a request's
   last page at or past seq_len is also set to 0x7E, so an over-read or a
   missing mask shows up as a large score.
5. Values: ``randn * scale`` cast with torch to float8_e4m3fn (round to
   nearest even), stored as raw uint8 codes. Outlier blocks (configuration 3)
   are whole B128 blocks of keys multiplied by 8 before the cast. With
   ``values="codes"`` every q and k byte is instead drawn uniformly from the
   254 finite e4m3fn codes (subnormals through +-448 in one dot product: the
   hardest case for fp32 accumulation).
6. ``num_valid_pages[t] = floor(pos_t / 128) + 1`` with
   ``pos_t = seq_len - decode_query_len + j`` (for one query token per
   request this is ``ceil(seq_len / 128)``).
7. ``cols`` = the smallest multiple of four that covers the longest
   request's B128 blocks (the score plane's width).

Prefill workloads (``q_lens`` given) score a chunk of query tokens per
request instead of decode_query_len tokens: request b's chunk holds
``q_len_b`` tokens (drawn right after the sequence lengths, clipped to
seq_len_b), rows ``[qo_indptr[b], qo_indptr[b+1])`` of index_q, token j at
position ``seq_len_b - q_len_b + j``; ``num_valid_pages`` follows step 6 for
every token. The rest of the recipe is unchanged.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEADS = 4
DIM = 128
BLOCK = 128
POISON_CODE = 0x7E  # e4m3fn 448.0, the largest finite value

# The five seeded workloads (B requests, sequence-length law, page size,
# decode_query_len, value scale, outlier fraction, forced blocks, ranges).
CONFIGS = {
    1: dict(name="tiny_b1_s4096_p128_q1", batch=1, seq=("fixed", 4096), page_size=128, dql=1,
            scale=1.0, outlier_frac=0.0, init=1, local=2, ranges=1, pool=("exact", 32)),
    2: dict(name="b8_s8k-32k_p128_q1", batch=8, seq=("uniform", 8192, 32768), page_size=128,
            dql=1, scale=0.5, outlier_frac=0.0, init=1, local=2, ranges=1, pool=("fixed", 2048)),
    3: dict(name="b32_s32k-128k_p256_q2_outliers", batch=32, seq=("uniform", 32768, 131072),
            page_size=256, dql=2, scale=1.0, outlier_frac=0.01, init=1, local=4, ranges=1,
            pool=("exact", None)),
    4: dict(name="b64_s1k-256k-log_p128_q4", batch=64, seq=("loguniform", 1024, 262144),
            page_size=128, dql=4, scale=1.0, outlier_frac=0.0, init=2, local=2, ranges=1,
            pool=("exact", None)),
    5: dict(name="long_b4_s1m_p256_q8_r8", batch=4, seq=("fixed", 1048576), page_size=256,
            dql=8, scale=1.0, outlier_frac=0.0, init=4, local=4, ranges=8,
            pool=("exact", 16384)),
}


@dataclass
class Workload:
    name: str
    index_q: torch.Tensor          # uint8 [T, 4, 128] (e4m3fn codes)
    index_k: torch.Tensor          # uint8 [num_pages, page_size, 128]
    block_table: torch.Tensor      # int32 [B, width]
    seq_lens: torch.Tensor         # int32 [B]
    num_valid_pages: torch.Tensor  # int32 [T]
    page_size: int
    dql: int
    cols: int
    init_blocks: int
    local_blocks: int
    num_ranges: int
    poison_page: int
    meta: dict = field(default_factory=dict)
    qo_indptr: torch.Tensor | None = None  # int32 [B + 1] for prefill chunks, else None

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        if self.qo_indptr is not None:
            return int(self.qo_indptr[-1])
        return self.batch * self.dql

    @property
    def q_lens(self) -> torch.Tensor:
        """Query tokens per request (decode_query_len each for decode)."""
        if self.qo_indptr is not None:
            return (self.qo_indptr[1:] - self.qo_indptr[:-1]).to(torch.int32)
        return torch.full((self.batch,), self.dql, dtype=torch.int32)

    @property
    def positions(self) -> torch.Tensor:
        """int64 [T]: the position of every query token."""
        ql = self.q_lens.to(torch.int64)
        sl = self.seq_lens.to(torch.int64)
        first = torch.repeat_interleave(sl - ql, ql)
        start = torch.repeat_interleave(torch.cumsum(ql, 0) - ql, ql)
        return first + torch.arange(int(ql.sum())) - start

    @property
    def total_keys(self) -> int:
        return int(self.seq_lens.clamp(min=0).sum())


def _draw_seq_lens(g: torch.Generator, batch: int, law) -> torch.Tensor:
    kind = law[0]
    if kind == "fixed":
        return torch.full((batch,), int(law[1]), dtype=torch.int64)
    if kind == "uniform":
        return torch.randint(int(law[1]), int(law[2]) + 1, (batch,), generator=g, dtype=torch.int64)
    if kind == "loguniform":
        lo, hi = math.log(law[1]), math.log(law[2])
        u = torch.rand((batch,), generator=g, dtype=torch.float64)
        return torch.floor(torch.exp(lo + (hi - lo) * u)).to(torch.int64)
    if kind == "list":
        return torch.tensor(list(law[1]), dtype=torch.int64)
    raise ValueError(f"unknown sequence-length law {law!r}")


def _to_e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    if bool(((codes & 0x7F) == 0x7F).any()):
        raise ValueError("fp8 cast produced a NaN code; value scale too large")
    return codes


FINITE_CODES = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8)


def _finite_codes(g: torch.Generator, shape) -> torch.Tensor:
    """Codes drawn uniformly from the 254 finite e4m3fn codes."""
    return FINITE_CODES[torch.randint(0, len(FINITE_CODES), shape, generator=g)]


def generate(*, batch: int, seq, page_size: int, dql: int, scale: float = 1.0,
             outlier_frac: float = 0.0, init: int = 1, local: int = 2, ranges: int = 1,
             pool=("exact", None), seed: int = 0, name: str = "custom", cols: int | None = None,
             table_width: int | None = None, chunk_pages: int = 1024,
             values: str = "normal", q_lens=None) -> Workload:
    """Draws one workload following the module recipe (a prefill workload
    when q_lens, a sequence-length law for the chunks, is given)."""
    if values not in ("normal", "codes"):
        raise ValueError(f"unknown value law {values!r}")
    g = torch.Generator().manual_seed(int(seed))
    seq_lens = _draw_seq_lens(g, batch, seq)
    if int(seq_lens.min()) < 0:
        raise ValueError("negative sequence length")
    qo_indptr = None
    if q_lens is not None:
        ql = torch.minimum(_draw_seq_lens(g, batch, q_lens), seq_lens)
        qo_indptr = torch.zeros(batch + 1, dtype=torch.int32)
        qo_indptr[1:] = torch.cumsum(ql, 0).to(torch.int32)
    pages_per_req = [(int(s) + page_size - 1) // page_size for s in seq_lens]
    need = sum(pages_per_req)
    pool_size = need if pool[0] == "exact" or pool[1] is None else int(pool[1])
    if pool[0] == "exact" and pool[1] is not None and int(pool[1]) != need:
        raise ValueError(f"pool {pool[1]} != pages needed {need}")
    if pool_size < need:
        raise ValueError(f"pool of {pool_size} pages cannot hold {need}")
    poison = pool_size
    num_pages = pool_size + 1

    blocks_max = max(((int(s) + BLOCK - 1) // BLOCK for s in seq_lens), default=0)
    if cols is None:
        cols = max(4, (blocks_max + 3) // 4 * 4)
    if table_width is None:
        table_width = max(1, max(max(pages_per_req, default=1), (cols * BLOCK + page_size - 1) // page_size))

    perm = torch.randperm(pool_size, generator=g) if pool_size > 0 else torch.zeros(0, dtype=torch.int64)
    block_table = torch.full((batch, table_width), poison, dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per_req):
        block_table[b, :npg] = perm[off:off + npg].to(torch.int32)
        off += npg

    # outlier B128 blocks (whole blocks of keys scaled x8 before the cast)
    halves = page_size // BLOCK
    outlier = torch.zeros((num_pages, halves), dtype=torch.bool)
    n_outlier_blocks = 0
    if outlier_frac > 0:
        for b in range(batch):
            nblk = (int(seq_lens[b]) + BLOCK - 1) // BLOCK
            if nblk == 0:
                continue
            cnt = max(1, int(round(outlier_frac * nblk)))
            chosen = torch.randperm(nblk, generator=g)[:cnt]
            for blk in chosen.tolist():
                p = int(block_table[b, (blk * BLOCK) // page_size])
                outlier[p, (blk * BLOCK % page_size) // BLOCK] = True
                n_outlier_blocks += 1

    T = batch * dql if qo_indptr is None else int(qo_indptr[-1])
    if values == "codes":
        index_q = _finite_codes(g, (T, HEADS, DIM))
    else:
        index_q = _to_e4m3_codes(torch.randn((T, HEADS, DIM), generator=g) * scale)

    index_k = torch.empty((num_pages, page_size, DIM), dtype=torch.uint8)
    for p0 in range(0, pool_size, chunk_pages):
        p1 = min(pool_size, p0 + chunk_pages)
        if values == "codes":
            index_k[p0:p1] = _finite_codes(g, (p1 - p0, page_size, DIM))
            continue
        x = torch.randn((p1 - p0, page_size, DIM), generator=g) * scale
        if outlier_frac > 0:
            mult = torch.where(outlier[p0:p1], 8.0, 1.0)                 # [n, halves]
            x = x * mult.repeat_interleave(BLOCK, dim=1).unsqueeze(-1)   # [n, ps, 1]
        index_k[p0:p1] = _to_e4m3_codes(x)
    index_k[poison] = POISON_CODE
    for b in range(batch):
        s, npg = int(seq_lens[b]), pages_per_req[b]
        if npg and s % page_size:
            index_k[int(block_table[b, npg - 1]), s % page_size:] = POISON_CODE

    if qo_indptr is None:
        j = torch.arange(dql, dtype=torch.int64)
        pos = (seq_lens[:, None] - dql + j[None, :]).reshape(-1)
    else:
        ql = (qo_indptr[1:] - qo_indptr[:-1]).to(torch.int64)
        start = torch.repeat_interleave(qo_indptr[:-1].to(torch.int64), ql)
        pos = torch.repeat_interleave(seq_lens - ql, ql) + torch.arange(T) - start
    nvp = torch.where(pos >= 0, pos // BLOCK + 1, torch.zeros_like(pos)).to(torch.int32)

    return Workload(name=name, index_q=index_q, index_k=index_k, block_table=block_table,
                    seq_lens=seq_lens.to(torch.int32), num_valid_pages=nvp, page_size=page_size,
                    dql=dql, cols=int(cols), init_blocks=init, local_blocks=local,
                    num_ranges=ranges, poison_page=poison,
                    meta=dict(seed=seed, pool=pool_size, outlier_blocks=n_outlier_blocks,
                              scale=scale, values=values),
                    qo_indptr=qo_indptr)


def config(n: int, **overrides) -> Workload:
    """The seeded workload of configuration n (1..5)."""
    spec = dict(CONFIGS[n])
    spec.update(overrides)
    return generate(seed=1000 + n, **spec)


def index_k_bytes(w: Workload) -> int:
    """Algorithmic index-K bytes of one pass: 128 bytes per key of every request."""
    return w.total_keys * DIM


def shard_rows(index_k, rank: int, world_size: int):
    """Rank `rank`'s shard of a cache whose pages are split by rows over
    world_size ranks: rows [rank * R, (rank + 1) * R) of every page,
    R = page_size / world_size, as a contiguous [pages, R, 128] tensor (the
    layout one rank holds). Pure data movement."""
    pages, page_size, dim = index_k.shape
    if page_size % world_size != 0 or not 0 <= rank < world_size:
        raise ValueError("world_size must divide page_size and 0 <= rank < world_size")
    r = page_size // world_size
    return index_k[:, rank * r:(rank + 1) * r, :].contiguous()

