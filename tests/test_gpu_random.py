"""Seeded random sweep of the whole chain through the C ABI.

Each case draws a small workload: batch, sequence lengths (zero, short,
exact block multiples and ragged ones, and in every third case one long
request), page size, decode_query_len, number of column ranges (up to 16, or
17 to 99) and forced blocks. It then runs
* msa_score_decode: the plane within the score bound of the oracle's, and the
  columns past the written range untouched;
* msa_top16_select over the ranges, then msa_top16_merge: bit for bit the
  oracle's select and merge on the GPU's own plane;
* msa_top16_select_merge (where the one-launch form applies): bit for bit the
  two-launch rows, with and without the range rows;
* msa_score_select with its merge: bit for bit the plane and rows of the
  separate launches, then the same without a plane (pool in the workspace) and
  as msa_score_select_noalloc (where the sizes fit its scratch array);
* the row-sharded chain over world size 2 or 4 (every rank's
  msa_score_decode_sharded and msa_top16_select_mapped, then
  msa_top16_merge_dedup of all ranks' rows): bit for bit the merged rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS, shard_index_map
from parity import assert_rows_equal, compare_plane, written_mask

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
ROW_FILL = 0x7BADBEEF


def say(*a):
    print(*a, flush=True)


def draw_case(seed):
    rng = np.random.default_rng(7000 + seed)
    batch = int(rng.integers(1, 40))
    page_size = int(rng.choice([128, 256]))
    dql = int(rng.integers(1, 9))
    kinds = rng.integers(0, 5, size=batch)
    seqs = []
    for k in kinds:
        if k == 0:
            seqs.append(0)
        elif k == 1:
            seqs.append(int(rng.integers(1, 200)))
        elif k == 2:
            seqs.append(128 * int(rng.integers(1, 40)))
        else:
            seqs.append(int(rng.integers(1, 6000)))
    if max(seqs) == 0:
        seqs[0] = 1
    if seed % 3 == 0:  # one long request: wide rows, several windows per wave
        seqs[int(rng.integers(0, batch))] = int(rng.integers(20000, 300000))
    init = int(rng.integers(0, 6))
    local = int(rng.integers(0, 6))
    w = workloads.generate(batch=batch, seq=("list", seqs), page_size=page_size, dql=dql,
                           seed=8000 + seed, scale=float(rng.choice([0.5, 1.0])),
                           init=init, local=local)
    R = int(rng.integers(1, min(17, w.cols + 1)))
    if seed % 6 == 3:  # more ranges than the one-launch forms take
        R = int(rng.integers(17, min(100, w.cols + 1)))
    ws = int(rng.choice([2, 4]))
    return w, R, ws


@pytest.mark.parametrize("seed", range(48))
def test_random_chain(seed):
    w, R, ws = draw_case(seed)
    T, cols = w.num_tokens, w.cols
    say(f"[test] random case {seed}: batch {w.batch} page {w.page_size} dql {w.dql} "
        f"cols {cols} R {R} init {w.init_blocks} local {w.local_blocks}")
    q, k = w.index_q.to(DEV), w.index_k.to(DEV)
    bt, sl, nvp = w.block_table.to(DEV), w.seq_lens.to(DEV), w.num_valid_pages.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kw = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks)

    plane = torch.full((T, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                       device=DEV).view(torch.float32)
    msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size, decode_query_len=w.dql,
                         errors=err)
    part = msa.new_rows(T, 4, R, device=DEV)
    part.fill_(ROW_FILL)
    msa.msa_top16_select(plane, nvp, part, num_ranges=R, errors=err, **kw)
    final = msa.new_rows(T, 4, device=DEV)
    final.fill_(ROW_FILL)
    msa.msa_top16_merge(part, nvp, final, errors=err, **kw)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    got = plane.cpu().numpy()
    ref, amax, _ = oracle.score_decode(w.index_q.numpy(), w.index_k.numpy(),
                                       w.block_table.numpy(), w.seq_lens.numpy(),
                                       page_size=w.page_size, decode_query_len=w.dql,
                                       cols=cols, want_amax=True)
    written = written_mask(w.seq_lens.numpy(), w.dql, cols)
    n_bad, ratio = compare_plane(got, ref, amax, written)
    assert n_bad == 0, (n_bad, ratio)
    assert np.all(got.view(np.uint32)[~written] == CANARY_BITS)

    # select and merge, bit for bit, on the GPU's plane; the unwritten
    # columns (canary NaNs) lie past num_valid_pages and are never ranked
    nvp_np = w.num_valid_pages.numpy()
    ps, pi, _ = oracle.top16_select(got, nvp_np, num_ranges=R, **kw)
    pc = part.cpu()
    assert_rows_equal(msa.row_scores(pc).numpy(), msa.row_ids(pc).numpy(), ps, pi,
                      f"select case {seed}")
    ms, mi, missing = oracle.top16_merge(ps, pi, nvp_np, **kw)
    assert missing == 0
    fc = final.cpu()
    assert_rows_equal(msa.row_scores(fc).numpy(), msa.row_ids(fc).numpy(), ms, mi,
                      f"merge case {seed}")

    if R <= 16 and -(-cols // R) <= 2048:
        for with_partial in (True, False):
            fused = msa.new_rows(T, 4, device=DEV)
            fused.fill_(ROW_FILL)
            fpart = msa.new_rows(T, 4, R, device=DEV) if with_partial else None
            if fpart is not None:
                fpart.fill_(ROW_FILL)
            msa.msa_top16_select_merge(plane, nvp, fused, num_ranges=R, partial=fpart,
                                       errors=err, **kw)
            torch.cuda.synchronize()
            assert torch.equal(fused, final)
            if fpart is not None:
                assert torch.equal(fpart, part)

        counters = msa.score_select_workspace(w.batch, w.dql, cols, R, device=DEV)
        plane2 = torch.full((T, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                            device=DEV).view(torch.float32)
        part2 = msa.new_rows(T, 4, R, device=DEV)
        part2.fill_(ROW_FILL)
        final2 = msa.new_rows(T, 4, device=DEV)
        final2.fill_(ROW_FILL)
        msa.msa_score_select(q, k, bt, sl, plane2, nvp, part2, counters, page_size=w.page_size,
                             decode_query_len=w.dql, num_ranges=R, merged=final2, errors=err,
                             **kw)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(plane2.view(torch.int32), plane.view(torch.int32))
        assert torch.equal(part2, part)
        assert torch.equal(final2, final)
        assert int(counters.count_nonzero()) == 0

        # the same launch without a plane (scores in the workspace's pool), and
        # its variant on the library's own scratch array: the same rows
        pool_ws = msa.score_select_workspace(w.batch, w.dql, cols, R, pool=True, device=DEV)
        head = msa.msa_score_select_workspace_words(w.batch, w.dql, cols, R, pool=False)
        fits = (msa.msa_score_select_workspace_words(w.batch, w.dql, cols, R, pool=True)
                <= msa.NOALLOC_SCRATCH_WORDS)
        for noalloc in ((False, True) if fits else (False,)):
            part3 = msa.new_rows(T, 4, R, device=DEV)
            part3.fill_(ROW_FILL)
            final3 = msa.new_rows(T, 4, device=DEV)
            final3.fill_(ROW_FILL)
            common = dict(page_size=w.page_size, decode_query_len=w.dql, num_ranges=R, cols=cols,
                          merged=final3, errors=err, **kw)
            if noalloc:
                msa.msa_score_select_noalloc(q, k, bt, sl, None, nvp, part3, **common)
            else:
                msa.msa_score_select(q, k, bt, sl, None, nvp, part3, pool_ws, **common)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert torch.equal(part3, part), f"noalloc={noalloc}: range rows differ"
            assert torch.equal(final3, final), f"noalloc={noalloc}: merged rows differ"
        assert int(pool_ws[:head].count_nonzero()) == 0

    # the row-sharded chain: every rank's share, then the owner's merge
    pages = -(-int(w.seq_lens.max()) // w.page_size)
    scols = max(4, -(-pages // 4) * 4)
    rs = min(R, scols)
    if ws * rs <= 64:
        rows = msa.new_rows(T, 4, ws * rs, device=DEV)
        rows.fill_(ROW_FILL)
        for rank in range(ws):
            shard = workloads.shard_rows(w.index_k, rank, ws).to(DEV)
            splane = torch.full((T, 4, scols), int(CANARY_BITS), dtype=torch.int32,
                                device=DEV).view(torch.float32)
            msa.msa_score_decode_sharded(q, shard, bt, sl, splane, page_size=w.page_size,
                                         decode_query_len=w.dql, rank=rank, world_size=ws,
                                         errors=err)
            scale, offset = shard_index_map(w.page_size, rank, ws)
            spart = msa.new_rows(T, 4, rs, device=DEV)
            msa.msa_top16_select_mapped(splane, nvp, spart, num_ranges=rs, index_scale=scale,
                                        index_offset=offset, errors=err, **kw)
            rows[:, :, rank * rs:(rank + 1) * rs] = spart
        merged = msa.new_rows(T, 4, device=DEV)
        merged.fill_(ROW_FILL)
        msa.msa_top16_merge_dedup(rows, nvp, merged, errors=err, **kw)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(merged, final), f"sharded chain ws {ws} case {seed}"
