"""Back-to-back launches give the same bits every time.

The benchmark times the chain (msa_score_decode, msa_top16_select,
msa_top16_merge) many steps back to back with no synchronisation between
steps, over rotating copies of index_k, and times the one-launch forms
(msa_top16_select_merge, msa_score_select) beside it. These tests run the same
launches the same way, keep every step's outputs in buffers of their own, and
check after one synchronisation that
* every step's plane (canary columns past each request's written blocks
  included), range rows and merged rows equal the first step's bit for bit, and the first step's merged rows equal the oracle's select + merge
  on that plane (so the repeated value is the right one);
* the one-launch forms give the chain's rows bit for bit at every call;
* no launch counted an error, and msa_score_select's workspace (its pool
  excepted) is zero again after the last call.
Nothing here reads the clock: a race between a step's kernels (a select that
starts before the plane is complete, a merge that reads half-written rows, a
workspace counter left non-zero by one launch for the next) shows up as a
step whose bits differ.
"""
from __future__ import annotations

import sys

import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS
from parity import assert_rows_equal

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
STEPS = 24
ROW_FILL = 0x7BADBEEF


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def first_step_against_oracle(w, plane, final):
    """The oracle's select + merge on the GPU's own plane, bit for bit."""
    p = plane.cpu().numpy()
    nvp = w.num_valid_pages.numpy()
    os_, oi, bad = oracle.top16_select(p, nvp, init_blocks=w.init_blocks,
                                       local_blocks=w.local_blocks, num_ranges=w.num_ranges)
    assert bad == 0
    if w.num_ranges > 1:
        os_, oi, missing = oracle.top16_merge(os_, oi, nvp, init_blocks=w.init_blocks,
                                              local_blocks=w.local_blocks)
        assert missing == 0
    else:
        os_, oi = os_[:, :, 0], oi[:, :, 0]
    f = final.cpu()
    assert_rows_equal(msa.row_scores(f).numpy(), msa.row_ids(f).numpy(), os_, oi,
                      "first step vs oracle")


@pytest.mark.parametrize("n", [2, 4, 5])
def test_chain_back_to_back(n):
    w = workloads.config(n)
    say(f"[test] chain back to back, config {n}, {STEPS} steps")
    T, R = w.num_tokens, w.num_ranges
    q, bt, sl, nvp = (x.to(DEV) for x in (w.index_q, w.block_table, w.seq_lens,
                                          w.num_valid_pages))
    k0 = w.index_k.to(DEV)
    kcopies = [k0, k0.clone()]
    kw = dict(page_size=w.page_size, decode_query_len=w.dql)
    forced = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks)
    # columns past a request's written blocks keep the canary, so whole planes compare
    planes = [torch.full((T, 4, w.cols), int(CANARY_BITS), dtype=torch.int32,
                         device=DEV).view(torch.float32) for _ in range(STEPS)]
    parts = [msa.new_rows(T, 4, R, device=DEV) for _ in range(STEPS)]
    finals = [msa.new_rows(T, 4, device=DEV) for _ in range(STEPS)]
    ones = [msa.new_rows(T, 4, device=DEV) for _ in range(STEPS)]
    for t in parts + finals + ones:
        t.fill_(ROW_FILL)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    for i in range(STEPS):
        msa.msa_score_decode(q, kcopies[i % 2], bt, sl, planes[i], errors=errors, **kw)
        msa.msa_top16_select(planes[i], nvp, parts[i], num_ranges=R, errors=errors, **forced)
        if R > 1:
            msa.msa_top16_merge(parts[i], nvp, finals[i], errors=errors, **forced)
            msa.msa_top16_select_merge(planes[i], nvp, ones[i], num_ranges=R, errors=errors,
                                       **forced)
        else:
            finals[i].copy_(parts[i][:, :, 0])
            ones[i].copy_(parts[i][:, :, 0])
    torch.cuda.synchronize()
    assert int(errors.item()) == 0
    p0 = planes[0].view(torch.int32)
    for i in range(1, STEPS):
        assert torch.equal(planes[i].view(torch.int32), p0), f"step {i}: plane differs"
        assert torch.equal(parts[i], parts[0]), f"step {i}: range rows differ"
        assert torch.equal(finals[i], finals[0]), f"step {i}: merged rows differ"
    for i in range(STEPS):
        assert torch.equal(ones[i], finals[0]), f"step {i}: one-launch select + merge differs"
    first_step_against_oracle(w, planes[0], finals[0])


@pytest.mark.parametrize("n", [2, 5])
def test_score_select_back_to_back(n):
    """msa_score_select without a plane (scores in the workspace's pool),
    STEPS calls back to back on one workspace: every call's range and merged
    rows equal the chain's."""
    w = workloads.config(n)
    say(f"[test] score_select back to back, config {n}, {STEPS} calls")
    T, B, R = w.num_tokens, w.batch, w.num_ranges
    q, bt, sl, nvp = (x.to(DEV) for x in (w.index_q, w.block_table, w.seq_lens,
                                          w.num_valid_pages))
    k0 = w.index_k.to(DEV)
    kcopies = [k0, k0.clone()]
    kw = dict(page_size=w.page_size, decode_query_len=w.dql)
    forced = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks)

    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    ref_part = msa.new_rows(T, 4, R, device=DEV)
    ref_final = msa.new_rows(T, 4, device=DEV)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(q, k0, bt, sl, plane, errors=errors, **kw)
    msa.msa_top16_select(plane, nvp, ref_part, num_ranges=R, errors=errors, **forced)
    msa.msa_top16_merge(ref_part, nvp, ref_final, errors=errors, **forced)

    ws = msa.score_select_workspace(B, w.dql, w.cols, R, pool=True, device=DEV)
    head = msa.msa_score_select_workspace_words(B, w.dql, w.cols, R, pool=False)
    parts = [msa.new_rows(T, 4, R, device=DEV) for _ in range(STEPS)]
    finals = [msa.new_rows(T, 4, device=DEV) for _ in range(STEPS)]
    for t in parts + finals:
        t.fill_(ROW_FILL)
    torch.cuda.synchronize()
    for i in range(STEPS):
        msa.msa_score_select(q, kcopies[i % 2], bt, sl, None, nvp, parts[i], ws, cols=w.cols,
                             merged=finals[i], num_ranges=R, errors=errors, **kw, **forced)
    torch.cuda.synchronize()
    assert int(errors.item()) == 0
    assert int(ws[:head].count_nonzero()) == 0, "the last call left the workspace non-zero"
    for i in range(STEPS):
        assert torch.equal(parts[i], ref_part), f"call {i}: range rows differ from the chain"
        assert torch.equal(finals[i], ref_final), f"call {i}: merged rows differ from the chain"
    first_step_against_oracle(w, plane, ref_final)
