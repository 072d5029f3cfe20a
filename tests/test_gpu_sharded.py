"""GPU parity of the row-sharded path, through the C ABI.

One rank's share of a cache whose pages are split by rows over world_size
ranks ("flashinfer.msa_ops.msa_icp_decode_index_score_sharded": index_k
shard, rank, world_size, the description's columns):

* msa_score_decode_sharded: each rank's plane within 1e-5 * A of the
  oracle's, -inf where the oracle has -inf, columns past roundup4(pages)
  untouched (canary), at both page sizes and world sizes 2 and 4;
* msa_top16_select_mapped on the oracle's planes: bit-exact rows, errors;
* msa_top16_merge_dedup on rows in any order with shared ids: bit-exact
  against the oracle's merge, missing forced ids counted;
* the whole sharded chain at the long-context, ragged and outlier workloads:
  every rank's plane, mapped select over R ranges, then the merge of all
  ranks' rows, equals the unsharded GPU chain bit for bit (a key's dot
  product does not depend on the rank that computes it, and max is exact).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS, shard_index_map
from parity import assert_rows_equal, compare_plane

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
ROW_FILL = 0x7BADBEEF


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sharded_cols(w) -> int:
    pages = -(-int(w.seq_lens.max()) // w.page_size)
    return max(4, -(-pages // 4) * 4)


def sharded_written(seq_lens, dql, page_size, cols):
    sl = np.asarray(seq_lens)
    out = np.zeros((sl.shape[0] * dql, 4, cols), dtype=bool)
    for b, s in enumerate(sl):
        w = oracle.written_columns_sharded(int(s), page_size)
        out[b * dql:(b + 1) * dql, :, :min(w, cols)] = True
    return out


def gpu_plane_sharded(w, rank, ws, cols, block_table=None):
    shard = workloads.shard_rows(w.index_k, rank, ws)
    out = torch.full((w.num_tokens, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                     device=DEV).view(torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bt = w.block_table if block_table is None else block_table
    msa.msa_score_decode_sharded(w.index_q.to(DEV), shard.to(DEV), bt.to(DEV),
                                 w.seq_lens.to(DEV), out, page_size=w.page_size,
                                 decode_query_len=w.dql, rank=rank, world_size=ws, errors=err)
    torch.cuda.synchronize()
    return out, int(err.item())


def check_rank_plane(w, rank, ws, got, cols, block_table=None):
    bt = (w.block_table if block_table is None else block_table).numpy()
    shard = workloads.shard_rows(w.index_k, rank, ws).numpy()
    ref, amax, _ = oracle.score_decode_sharded(
        w.index_q.numpy(), shard, bt, w.seq_lens.numpy(), page_size=w.page_size,
        decode_query_len=w.dql, rank=rank, world_size=ws, cols=cols, want_amax=True)
    written = sharded_written(w.seq_lens.numpy(), w.dql, w.page_size, cols)
    n_bad, ratio = compare_plane(got, ref, amax, written)
    assert n_bad == 0, f"rank {rank}/{ws}: {n_bad} elements out of tolerance (ratio {ratio})"
    assert np.all(got.view(np.uint32)[~written] == CANARY_BITS), "unwritten column touched"
    return ratio


# ---------------------------------------------------------------------------
# rank planes against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("page_size", [128, 256])
@pytest.mark.parametrize("ws", [2, 4])
@pytest.mark.parametrize("dql", [1, 3, 8])
def test_sharded_plane_ragged(page_size, ws, dql):
    seqs = [0, 1, dql - 1 if dql > 1 else 2, 63, 64, 65, 127, 128, 255, 256, 257, 777, 2048 + 5]
    w = workloads.generate(batch=len(seqs), seq=("list", seqs), page_size=page_size, dql=dql,
                           seed=500 + page_size + ws * 7 + dql)
    cols = sharded_cols(w) + 8  # spare columns that must stay untouched
    for rank in range(ws):
        got, err = gpu_plane_sharded(w, rank, ws, cols)
        assert err == 0
        check_rank_plane(w, rank, ws, got.cpu().numpy(), cols)


def test_sharded_plane_errors():
    """Out-of-range block_table entries a rank needs are counted (their
    columns score -inf); a plane narrower than a request is counted."""
    w = workloads.generate(batch=2, seq=("list", [3000, 600]), page_size=256, dql=2, seed=501)
    bt = w.block_table.clone()
    bt[0, 1] = w.index_k.shape[0]
    bt[1, 0] = -7
    got, err = gpu_plane_sharded(w, 1, 2, sharded_cols(w), block_table=bt)
    assert err == 2
    g = got.cpu().numpy()
    assert np.all(np.isneginf(g[0:2, :, 1])) and np.all(np.isneginf(g[2:4, :, 0]))
    _, err2 = gpu_plane_sharded(w, 0, 2, 8)  # request 0 needs 12 columns
    assert err2 == 1


# ---------------------------------------------------------------------------
# mapped select and duplicate-aware merge against the oracle
# ---------------------------------------------------------------------------

TIE_POOL = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.5, 2.0], dtype=np.float32)


@pytest.mark.parametrize("cols,R,scale,offset,init,local", [
    (64, 1, 1, 0, 1, 2), (64, 3, 2, 1, 4, 4), (300, 4, 2, 0, 2, 14), (1000, 1, 2, 1, 1, 4),
    (2047, 2, 2, 1, 16, 0), (4096, 8, 2, 0, 4, 4), (100, 5, 3, 2, 0, 0),
    (4096, 2, 2, 1, 4, 4), (12000, 3, 1, 0, 2, 2),  # ranges over 1024 columns: 4 waves
    # global ids at and above 2^30 through the filtered (more than 128
    # columns per range) and the four-wave paths
    (1000, 1, 1, (1 << 30) + 5, 2, 2), (1000, 2, 2, (1 << 30) + 3, 1, 4),
    (3000, 1, 1, (1 << 31) - 3011, 4, 4),
])
@pytest.mark.parametrize("ties", [False, True])
def test_select_mapped_bit_exact(cols, R, scale, offset, init, local, ties):
    rng = np.random.default_rng(cols + 31 * R + scale + offset)
    T = 6
    plane = (rng.choice(TIE_POOL, size=(T, 4, cols)) if ties
             else rng.standard_normal((T, 4, cols))).astype(np.float32)
    top = scale * cols + offset
    nvp = np.array([top, 0, 7, int(rng.integers(0, top + 1)), top + 5, -3], dtype=np.int32)
    out = msa.new_rows(T, 4, R, device=DEV)
    out.fill_(ROW_FILL)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_select_mapped(torch.from_numpy(plane).to(DEV), torch.from_numpy(nvp).to(DEV),
                                out, init_blocks=init, local_blocks=local, num_ranges=R,
                                index_scale=scale, index_offset=offset, errors=err)
    torch.cuda.synchronize()
    rs, ri, bad = oracle.top16_select_mapped(plane, nvp, init_blocks=init, local_blocks=local,
                                             num_ranges=R, index_scale=scale,
                                             index_offset=offset)
    assert int(err.item()) == bad == 2
    o = out.cpu()
    assert_rows_equal(msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), rs, ri,
                      f"mapped cols={cols} R={R} s={scale} o={offset}")


def _shuffled_rank_rows(rng, T, cols, ws, R, init, local, ties):
    """Rows of ws pseudo-ranks over one global row: rank r's plane holds the
    global scores of its ids with a random deficit on some entries (a partial
    maximum), at least one rank holding the true value; rows concatenated
    then shuffled per (token, head)."""
    plane = (rng.choice(TIE_POOL, size=(T, 4, cols)) if ties
             else rng.standard_normal((T, 4, cols))).astype(np.float32)
    nvp = rng.integers(0, cols + 1, size=T).astype(np.int32)
    nvp[0] = cols
    holder = rng.integers(0, ws, size=(T, 4, cols))
    s_all, i_all = [], []
    for r in range(ws):
        part = plane.copy()
        low = (holder != r) & (rng.random((T, 4, cols)) < 0.5)
        part[low] -= np.float32(0.25)
        ps, pi, _ = oracle.top16_select(part, nvp, init_blocks=init, local_blocks=local,
                                        num_ranges=R)
        s_all.append(ps)
        i_all.append(pi)
    s_cat = np.concatenate(s_all, axis=2)
    i_cat = np.concatenate(i_all, axis=2)
    for t in range(T):
        for h in range(4):
            perm = rng.permutation(s_cat.shape[2])
            s_cat[t, h] = s_cat[t, h, perm]
            i_cat[t, h] = i_cat[t, h, perm]
    return s_cat, i_cat, nvp


def rows_tensor(scores, ids):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).view(torch.int32)
    i = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32))
    return torch.cat([s, i], dim=-1).contiguous().to(DEV)


@pytest.mark.parametrize("ws,R,init,local", [(2, 1, 1, 2), (4, 1, 4, 4), (2, 8, 4, 4),
                                             (4, 16, 2, 14), (1, 64, 0, 0), (4, 3, 16, 0)])
@pytest.mark.parametrize("ties", [False, True])
def test_merge_dedup_bit_exact(ws, R, init, local, ties):
    rng = np.random.default_rng(ws * 100 + R + init)
    T, cols = 5, 300
    s_cat, i_cat, nvp = _shuffled_rank_rows(rng, T, cols, ws, R, init, local, ties)
    out = msa.new_rows(T, 4, device=DEV)
    out.fill_(ROW_FILL)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge_dedup(rows_tensor(s_cat, i_cat), torch.from_numpy(nvp).to(DEV), out,
                              init_blocks=init, local_blocks=local, errors=err)
    torch.cuda.synchronize()
    rs, ri, missing = oracle.top16_merge(s_cat, i_cat, nvp, init_blocks=init,
                                         local_blocks=local)
    assert int(err.item()) == missing == 0
    o = out.cpu()
    assert_rows_equal(msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), rs, ri,
                      f"dedup ws={ws} R={R}")


def test_merge_dedup_reports_missing_forced():
    rng = np.random.default_rng(77)
    s_cat, i_cat, nvp = _shuffled_rank_rows(rng, 2, 64, 2, 2, 2, 2, False)
    for r in range(i_cat.shape[2]):  # drop forced id 0 of (token 0, head 1) everywhere
        hit = i_cat[0, 1, r] == 0
        i_cat[0, 1, r][hit] = -1
        s_cat[0, 1, r][hit] = -np.inf
    out = msa.new_rows(2, 4, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge_dedup(rows_tensor(s_cat, i_cat), torch.from_numpy(nvp).to(DEV), out,
                              init_blocks=2, local_blocks=2, errors=err)
    torch.cuda.synchronize()
    rs, ri, missing = oracle.top16_merge(s_cat, i_cat, nvp, init_blocks=2, local_blocks=2)
    assert int(err.item()) == missing == 1
    o = out.cpu()
    assert_rows_equal(msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), rs, ri, "missing")


# ---------------------------------------------------------------------------
# the sharded chain at the workloads' shapes
# ---------------------------------------------------------------------------

def unsharded_chain(w, q, k, bt, sl, nvp):
    T, R = w.num_tokens, w.num_ranges
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    part = msa.new_rows(T, 4, R, device=DEV)
    final = msa.new_rows(T, 4, device=DEV)
    msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size, decode_query_len=w.dql)
    msa.msa_top16_select(plane, nvp, part, init_blocks=w.init_blocks,
                         local_blocks=w.local_blocks, num_ranges=R)
    if R > 1:
        msa.msa_top16_merge(part, nvp, final, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks)
    else:
        final.copy_(part[:, :, 0])
    torch.cuda.synchronize()
    return final.cpu()


@pytest.mark.parametrize("n", [3, 4, 5])
@pytest.mark.parametrize("ws", [2, 4])
def test_sharded_chain_equals_unsharded(n, ws):
    w = workloads.config(n)
    T, R = w.num_tokens, w.num_ranges
    say(f"[test] sharded chain config {n} ({w.name}) world_size {ws}")
    q, bt, sl = w.index_q.to(DEV), w.block_table.to(DEV), w.seq_lens.to(DEV)
    nvp = w.num_valid_pages.to(DEV)
    ref = unsharded_chain(w, q, w.index_k.to(DEV), bt, sl, nvp)
    cols = sharded_cols(w)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows = msa.new_rows(T, 4, ws * R, device=DEV)
    rows.fill_(ROW_FILL)
    for rank in range(ws):
        shard = workloads.shard_rows(w.index_k, rank, ws).to(DEV)
        plane = torch.full((T, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                           device=DEV).view(torch.float32)
        msa.msa_score_decode_sharded(q, shard, bt, sl, plane, page_size=w.page_size,
                                     decode_query_len=w.dql, rank=rank, world_size=ws,
                                     errors=err)
        scale, offset = shard_index_map(w.page_size, rank, ws)
        part = msa.new_rows(T, 4, R, device=DEV)
        msa.msa_top16_select_mapped(plane, nvp, part, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=R,
                                    index_scale=scale, index_offset=offset, errors=err)
        rows[:, :, rank * R:(rank + 1) * R] = part
        if n != 5 or rank == 0:  # the oracle plane of every rank, except config 5
            torch.cuda.synchronize()
            ratio = check_rank_plane(w, rank, ws, plane.cpu().numpy(), cols)
            say(f"   rank {rank}: plane worst |err|/tol = {ratio:.3g}")
        del shard
    final = msa.new_rows(T, 4, device=DEV)
    msa.msa_top16_merge_dedup(rows, nvp, final, init_blocks=w.init_blocks,
                              local_blocks=w.local_blocks, errors=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = final.cpu()
    assert_rows_equal(msa.row_scores(got).numpy(), msa.row_ids(got).numpy(),
                      msa.row_scores(ref).numpy(), msa.row_ids(ref).numpy(),
                      f"sharded chain config {n} ws {ws}")


def test_merge_dedup_equal_duplicates_keep_earliest():
    """Duplicates of an id with equal scores of either zero sign: the first
    occurrence in the concatenated rows is kept, as in the oracle."""
    T, R = 1, 3
    s = np.full((T, 4, R, 16), -np.inf, dtype=np.float32)
    i = np.full((T, 4, R, 16), -1, dtype=np.int32)
    for h in range(4):
        first, second = (np.float32(-0.0), np.float32(0.0)) if h % 2 == 0 else \
                        (np.float32(0.0), np.float32(-0.0))
        i[0, h, 0, :3] = [5, 9, 40]
        s[0, h, 0, :3] = [first, 1.0, 2.0]
        i[0, h, 2, :2] = [5, 40]
        s[0, h, 2, :2] = [second, 2.0]
        i[0, h, 1, :2] = [9, 11]
        s[0, h, 1, :2] = [0.5, -0.0]
    nvp = np.array([64], np.int32)
    out = msa.new_rows(T, 4, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge_dedup(rows_tensor(s, i), torch.from_numpy(nvp).to(DEV), out,
                              init_blocks=0, local_blocks=0, errors=err)
    torch.cuda.synchronize()
    rs, ri, missing = oracle.top16_merge(s, i, nvp, init_blocks=0, local_blocks=0)
    assert int(err.item()) == missing == 0
    o = out.cpu()
    assert_rows_equal(msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), rs, ri, "zeros")
    assert np.float32(rs[0, 0, 0]).view(np.uint32) == np.float32(-0.0).view(np.uint32)


@pytest.mark.parametrize("page_size,ws", [(128, 4), (256, 2)])
def test_sharded_plane_batch_above_64(page_size, ws):
    """Batches above 64 take the two-pass request search."""
    w = workloads.generate(batch=300, seq=("loguniform", 1, 9000), page_size=page_size, dql=3,
                           seed=502 + ws)
    cols = sharded_cols(w) + 4
    for rank in (0, ws - 1):
        got, err = gpu_plane_sharded(w, rank, ws, cols)
        assert err == 0
        check_rank_plane(w, rank, ws, got.cpu().numpy(), cols)
