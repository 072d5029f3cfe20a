"""GPU parity of msa_score_select (score plane and per-range Top16 rows in one
launch), through the C ABI.

Every case runs the fused launch twice with a plane and twice without one
(the scores then go to the workspace's pool), on one reused workspace, and
checks each time that
* the plane is bit-identical to msa_score_decode's, canary columns included;
* the range rows are bit-identical to msa_top16_select's on that plane, and
  the merged rows to msa_top16_merge's of those;
* the error count equals the two-call path's;
* the workspace (the pool excepted) holds zeros again after the launch.
The five workloads are also checked against the oracle: the rows equal the
oracle's select on the GPU's plane bit for bit, and, after the merge, the
oracle's chain on its own plane by the admissibility rule of tests/parity.py
(the rows must be the exact selection of some plane within tolerance).
Edge cases: every decode_query_len at both page sizes with empty and short
requests, range boundaries inside 4-column groups, one column per range,
batches above 64, num_valid_pages past the written columns or outside
[0, cols], bad block-table entries, a plane too narrow for a request.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS
from parity import assert_rows_equal, compare_e2e_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
FINITE_CANARY = 0xC0A00000  # -5.0: a canary the select may read as a score
ROW_FILL = 0x7BADBEEF


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_both(w, *, R=None, cols=None, nvp=None, block_table=None, canary=CANARY_BITS,
             repeat=2, pool=True):
    """Two-call path (msa_score_decode, msa_top16_select, msa_top16_merge),
    then the fused launch `repeat` times with a plane and, if `pool`, as many
    times without one (scores in the workspace's pool), all on one workspace;
    asserts they agree bit for bit and that the workspace (pool excepted) is
    zero after every launch. Returns (plane, rows, errors) of the fused launch
    with a plane (numpy, torch int32 on the device, int)."""
    T, B = w.num_tokens, w.batch
    R = R or w.num_ranges
    cols = cols or w.cols
    q, k, sl = w.index_q.to(DEV), w.index_k.to(DEV), w.seq_lens.to(DEV)
    bt = (w.block_table if block_table is None else block_table).to(DEV)
    nvp_t = (w.num_valid_pages if nvp is None else nvp).to(DEV)
    kw = dict(page_size=w.page_size, decode_query_len=w.dql)
    sel = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks, num_ranges=R)
    with_merged = R <= 64

    plane2 = torch.full((T, 4, cols), int(np.int32(np.uint32(canary))), dtype=torch.int32,
                        device=DEV).view(torch.float32)
    rows2 = msa.new_rows(T, 4, R, device=DEV)
    rows2.fill_(ROW_FILL)
    merged2 = msa.new_rows(T, 4, device=DEV)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(q, k, bt, sl, plane2, errors=err2, **kw)
    msa.msa_top16_select(plane2, nvp_t, rows2, errors=err2, **sel)
    if with_merged and R > 1:  # the fused launch counts what the merge counts
        msa.msa_top16_merge(rows2, nvp_t, merged2, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks, errors=err2)
    else:
        msa.msa_top16_merge(rows2, nvp_t, merged2, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks)
    torch.cuda.synchronize()
    ref_err = int(err2.item())
    ref_plane = plane2.view(torch.int32).cpu()
    ref_rows = rows2.cpu()
    ref_merged = merged2.cpu()

    ws = msa.score_select_workspace(B, w.dql, cols, R, pool=pool, device=DEV)
    head = msa.msa_score_select_workspace_words(B, w.dql, cols, R, pool=False)
    for mode in (["plane", "pool"] if pool else ["plane"]):
        for rep in range(repeat):
            plane1 = None
            if mode == "plane":
                plane1 = torch.full((T, 4, cols), int(np.int32(np.uint32(canary))),
                                    dtype=torch.int32, device=DEV).view(torch.float32)
            rows1 = msa.new_rows(T, 4, R, device=DEV)
            rows1.fill_(ROW_FILL)
            merged1 = msa.new_rows(T, 4, device=DEV) if with_merged else None
            if merged1 is not None:
                merged1.fill_(ROW_FILL)
            err1 = torch.zeros(1, dtype=torch.int32, device=DEV)
            msa.msa_score_select(q, k, bt, sl, plane1, nvp_t, rows1, ws, cols=cols,
                                 merged=merged1, errors=err1, **kw, **sel)
            torch.cuda.synchronize()
            what = f"{mode} launch {rep}"
            if plane1 is not None:
                got_plane = plane1.view(torch.int32).cpu()
                n_plane = int((got_plane != ref_plane).sum())
                assert n_plane == 0, f"{what}: {n_plane} plane words differ from msa_score_decode"
                rows_out = rows1
            got_rows = rows1.cpu()
            bad = (got_rows != ref_rows).any(dim=-1).nonzero()
            assert bad.numel() == 0, (f"{what}: {bad.shape[0]} rows differ from "
                                      f"msa_top16_select; first (t, h, r) {bad[:3].tolist()}")
            if merged1 is not None:
                badm = (merged1.cpu() != ref_merged).any(dim=-1).nonzero()
                assert badm.numel() == 0, (f"{what}: {badm.shape[0]} merged rows differ from "
                                           f"msa_top16_merge; first {badm[:3].tolist()}")
            assert int(err1.item()) == ref_err, (what, int(err1.item()), ref_err)
            assert int(ws[:head].count_nonzero()) == 0, f"{what} left the workspace non-zero"
    return got_plane.view(torch.float32).numpy(), rows_out, ref_err


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_score_select_workloads(n):
    w = workloads.config(n)
    T, R = w.num_tokens, w.num_ranges
    say(f"[test] score_select config {n} ({w.name}) R={R}")
    plane, rows, err = run_both(w)
    assert err == 0
    nvp = w.num_valid_pages.numpy()
    r = rows.cpu()
    g_s, g_i = msa.row_scores(r).numpy(), msa.row_ids(r).numpy()

    # the rows are the oracle's select on the GPU's own plane
    ps, pi, _ = oracle.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=R)
    assert_rows_equal(g_s, g_i, ps, pi, f"fused ranges config {n}")

    # merged, against the oracle's chain on its own plane (near-ties exempt)
    if R > 1:
        final = msa.new_rows(T, 4, device=DEV)
        msa.msa_top16_merge(rows, w.num_valid_pages.to(DEV), final, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks)
        torch.cuda.synchronize()
        f_i = msa.row_ids(final.cpu()).numpy()
    else:
        f_i = g_i[:, :, 0]
    ref, amax, bad = oracle.score_decode(
        w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(), w.seq_lens.numpy(),
        page_size=w.page_size, decode_query_len=w.dql, cols=w.cols, want_amax=True)
    assert bad == 0
    rs, ri, _ = oracle.top16_select(ref, nvp, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=1)
    n_exact, n_tie, failures = compare_e2e_rows(f_i, ri[:, :, 0], ref, amax, nvp, w.init_blocks,
                                                w.local_blocks)
    say(f"   rows exact={n_exact} near-tie={n_tie} failed={len(failures)}")
    assert not failures, failures[:3]


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dql", [1, 3, 4, 5, 8])
@pytest.mark.parametrize("page_size", [128, 256])
@pytest.mark.parametrize("R", [1, 3])
def test_score_select_ragged_small(dql, page_size, R):
    """Empty, one-token and shorter-than-dql requests, exact multiples of 128,
    odd block counts; with R = 3 the range boundaries fall inside 4-column
    groups."""
    seqs = [0, 1, dql - 1 if dql > 1 else 2, 127, 128, 129, 383, 512, 777, 2048 + 5]
    w = workloads.generate(batch=len(seqs), seq=("list", seqs), page_size=page_size, dql=dql,
                           seed=300 + dql * 3 + page_size + R, init=1, local=2, ranges=R)
    say(f"[test] ragged dql={dql} P{page_size} R={R} cols={w.cols}")
    _, _, err = run_both(w, R=R)
    assert err == 0


@pytest.mark.parametrize("R", [32, 64])
def test_score_select_one_column_per_range(R):
    w = workloads.generate(batch=3, seq=("list", [8192, 3000, 129]), page_size=128, dql=2,
                           seed=41 + R, init=2, local=2)
    assert w.cols == 64
    say(f"[test] one column per range R={R}")
    _, _, err = run_both(w, R=R)
    assert err == 0


def test_score_select_many_ranges_wide_plane():
    w = workloads.generate(batch=2, seq=("list", [1 << 20, 70000]), page_size=256, dql=8,
                           seed=43, init=4, local=4)
    assert w.cols == 8192
    say("[test] R=768 over 8192 columns")
    _, _, err = run_both(w, R=768, repeat=1)
    assert err == 0


def test_score_select_batch_above_64():
    """Batches above 64 take the two-pass request search in the scorer."""
    w = workloads.generate(batch=150, seq=("loguniform", 1, 40000), page_size=128, dql=2,
                           seed=44, init=1, local=2)
    say(f"[test] batch 150 cols={w.cols}")
    _, _, err = run_both(w, R=2)
    assert err == 0


def test_score_select_nvp_past_written_and_out_of_range():
    """num_valid_pages past a request's written columns makes the select read
    columns this launch never writes (here a finite canary), exactly as the
    separate select call would; values outside [0, cols] are counted once per
    token and clamped."""
    w = workloads.generate(batch=4, seq=("list", [5000, 300, 0, 2000]), page_size=128, dql=2,
                           seed=45, init=1, local=2)
    nvp = torch.full((w.num_tokens,), w.cols, dtype=torch.int32)
    nvp[1] = -2
    nvp[3] = w.cols + 9
    say(f"[test] nvp past written columns cols={w.cols}")
    _, _, err = run_both(w, R=2, nvp=nvp, canary=FINITE_CANARY, pool=False)
    # once per token from the select; the merge misses the forced ids past the
    # plane of token 3 in its four heads
    assert err == 2 + 4


def test_score_select_bad_block_table_and_narrow_plane():
    w = workloads.generate(batch=3, seq=("list", [3000, 600, 1000]), page_size=128, dql=1,
                           seed=46, init=1, local=2)
    bt = w.block_table.clone()
    bt[0, 2] = w.index_k.shape[0]
    bt[2, 0] = -1
    say("[test] bad block-table entries, plane narrower than request 0")
    _, _, err = run_both(w, R=2, block_table=bt, cols=16, canary=FINITE_CANARY)
    # two bad entries; request 0 is wider than the plane (scorer), and its
    # token's num_valid_pages (24) exceeds cols (select); the merge then misses
    # that token's forced ids past the plane in its four heads
    assert err == 4 + 4


# ---------------------------------------------------------------------------
# other work on the device at the same time
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 4, 5])
def test_score_select_beside_other_work(n):
    """The fused launch waits only in its helper waves (at most half of what
    the device holds), so its result does not depend on getting the whole
    device: here a second stream (default priority) keeps a long run of
    elementwise kernels in flight while the fused launch runs, and the rows,
    merged rows and error count must still equal the two-call path's, with
    the workspace zero afterwards."""
    w = workloads.config(n)
    T, R = w.num_tokens, w.num_ranges
    say(f"[test] score_select beside other work, config {n}")
    q, k, sl = w.index_q.to(DEV), w.index_k.to(DEV), w.seq_lens.to(DEV)
    bt, nvp = w.block_table.to(DEV), w.num_valid_pages.to(DEV)
    kw = dict(page_size=w.page_size, decode_query_len=w.dql)
    sel = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks)

    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    ref_rows = msa.new_rows(T, 4, R, device=DEV)
    ref_merged = msa.new_rows(T, 4, device=DEV)
    ref_err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(q, k, bt, sl, plane, errors=ref_err, **kw)
    msa.msa_top16_select(plane, nvp, ref_rows, num_ranges=R, errors=ref_err, **sel)
    msa.msa_top16_merge(ref_rows, nvp, ref_merged, errors=ref_err if R > 1 else None, **sel)
    torch.cuda.synchronize()

    busy = torch.ones(1 << 28, dtype=torch.float32, device=DEV)  # 1 GiB
    other = torch.cuda.Stream(device=DEV)
    ws = msa.score_select_workspace(w.batch, w.dql, w.cols, R, pool=True, device=DEV)
    head = msa.msa_score_select_workspace_words(w.batch, w.dql, w.cols, R, pool=False)
    main = torch.cuda.current_stream()
    for rep in range(3):
        rows = msa.new_rows(T, 4, R, device=DEV)
        merged = msa.new_rows(T, 4, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        with torch.cuda.stream(other):
            for _ in range(8):
                busy.mul_(1.0)
        msa.msa_score_select(q, k, bt, sl, None, nvp, rows, ws, cols=w.cols, merged=merged,
                             num_ranges=R, errors=err, stream=main, **kw, **sel)
        torch.cuda.synchronize()
        assert torch.equal(rows.cpu(), ref_rows.cpu()), f"rep {rep}: range rows differ"
        assert torch.equal(merged.cpu(), ref_merged.cpu()), f"rep {rep}: merged rows differ"
        assert int(err.item()) == int(ref_err.item()) == 0
        assert int(ws[:head].count_nonzero()) == 0, f"rep {rep}: workspace left non-zero"
