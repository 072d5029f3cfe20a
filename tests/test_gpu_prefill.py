"""GPU parity of the prefill chain (window plan -> local scoring and Top16
select -> merge) against the CPU oracle, through the C ABI.

* score scratch: every written element within 1e-5 * A of the oracle's
  prefill plane, -inf where the oracle has -inf, columns past each request's
  roundup4(blocks) left bit-identical (canary);
* carrier rows: bit-exact against the oracle's select on the GPU's own plane;
* merged rows: bit-exact against the oracle's merge of those rows, and end to
  end against the oracle's own plane within the admissibility rule of
  tests/parity.py;
* shapes: a short ragged chunk (1, 17 and 64 tokens), chunks crossing block
  and page boundaries at page_size 256 (with outlier blocks), empty chunks
  and an empty request, a ragged batch of six, 300 small requests (more than
  the plan kernel's threads), and a long window of 8192
  tokens at the end of a 65536-key request (sampled rows against the oracle,
  every row against the -inf pattern the causal rule fixes);
* errors: a plan made for another plane runs nothing; bad block-table
  entries are counted and their blocks score -inf.
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
from parity import assert_rows_equal, compare_e2e_rows, compare_plane

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    "short_ragged": dict(batch=3, seq=("list", [129, 300, 700]), q_lens=("list", [1, 17, 64]),
                         page_size=128, dql=1, init=1, local=2, ranges=2, seed=3101),
    "cross_p256": dict(batch=3, seq=("list", [515, 1000, 130]), q_lens=("list", [257, 300, 130]),
                       page_size=256, dql=1, init=2, local=3, ranges=3, seed=3102,
                       outlier_frac=0.05),
    "empty_chunks": dict(batch=4, seq=("list", [640, 0, 383, 900]),
                         q_lens=("list", [3, 0, 0, 40]), page_size=128, dql=1, init=1, local=1,
                         ranges=1, seed=3103, cols=12),
    "ragged_b6": dict(batch=6, seq=("uniform", 2000, 20000), q_lens=("uniform", 1, 700),
                      page_size=128, dql=1, init=2, local=2, ranges=4, seed=3104),
    # more requests than the plan kernel has threads: its scan runs in passes
    "many_requests_b300": dict(batch=300, seq=("uniform", 1, 700), q_lens=("uniform", 0, 24),
                               page_size=128, dql=1, init=1, local=2, ranges=2, seed=3106),
}

LONG = dict(batch=1, seq=("fixed", 65536), q_lens=("fixed", 8192), page_size=256, dql=1, init=4,
            local=4, ranges=4, seed=3105)


def written_mask_prefill(w, cols):
    """[Tq, 4, cols] bool: columns below min(roundup4(ceil(seq/128)), cols) of
    each token's request."""
    m = np.zeros((w.num_tokens, 4, cols), dtype=bool)
    qo = w.qo_indptr.numpy()
    for b, s in enumerate(w.seq_lens.tolist()):
        if s <= 0:
            continue
        wcols = min(-(-(-(-s // 128)) // 4) * 4, cols)
        m[qo[b]:qo[b + 1], :, :wcols] = True
    return m


def run_chain(w, cols=None, block_table=None, plan_cols=None):
    """Plan, local and merge on the device. Returns (plane, carrier, merged,
    errors) as CPU arrays/ints; the plane starts as canary."""
    cols = w.cols if cols is None else cols
    T, R = w.num_tokens, w.num_ranges
    q, k = w.index_q.to(DEV), w.index_k.to(DEV)
    bt = (w.block_table if block_table is None else block_table).to(DEV)
    qo, sl, nvp = w.qo_indptr.to(DEV), w.seq_lens.to(DEV), w.num_valid_pages.to(DEV)
    plane = torch.from_numpy(np.full((T, 4, cols), CANARY_BITS, dtype=np.uint32)
                             .view(np.float32)).to(DEV)
    plan = msa.new_prefill_plan(T, w.batch, cols, device=DEV)
    carrier = msa.new_rows(T, 4, R, device=DEV)
    merged = msa.new_rows(T, 4, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_prefill_window_plan(qo, sl, plan, num_tokens=T,
                                cols=cols if plan_cols is None else plan_cols, errors=err)
    msa.msa_prefill_local(q, k, bt, plan, plane, nvp, carrier, page_size=w.page_size,
                          init_blocks=w.init_blocks, local_blocks=w.local_blocks, num_ranges=R,
                          errors=err)
    msa.msa_prefill_merge(carrier, nvp, merged, init_blocks=w.init_blocks,
                          local_blocks=w.local_blocks, errors=err)
    torch.cuda.synchronize()
    return plane.cpu().numpy(), carrier.cpu(), merged.cpu(), int(err.item())


def oracle_plane(w, cols, tokens=None):
    plane, amax, bad = oracle.score_prefill(w.index_q.numpy(), w.index_k.numpy(),
                                            w.block_table.numpy(), w.qo_indptr.numpy(),
                                            w.seq_lens.numpy(), page_size=w.page_size, cols=cols,
                                            tokens=tokens, want_amax=True)
    assert bad == 0
    return plane, amax


def check_rows(w, got_plane, carrier, merged, ref_plane, amax):
    nvp = w.num_valid_pages.numpy()
    R = w.num_ranges
    ps, pi, sbad = oracle.top16_select(got_plane, nvp, init_blocks=w.init_blocks,
                                       local_blocks=w.local_blocks, num_ranges=R)
    assert sbad == 0
    assert_rows_equal(msa.row_scores(carrier).numpy(), msa.row_ids(carrier).numpy(), ps, pi,
                      f"{w.name} carrier")
    ms, mi, missing = oracle.top16_merge(ps, pi, nvp, init_blocks=w.init_blocks,
                                         local_blocks=w.local_blocks)
    assert missing == 0
    assert_rows_equal(msa.row_scores(merged).numpy(), msa.row_ids(merged).numpy(), ms, mi,
                      f"{w.name} merged")
    # end to end against the oracle's own plane
    _, ri, _ = oracle.top16_select(ref_plane, nvp, init_blocks=w.init_blocks,
                                   local_blocks=w.local_blocks, num_ranges=1)
    n_exact, n_tie, failures = compare_e2e_rows(msa.row_ids(merged).numpy(), ri[:, :, 0],
                                                ref_plane, amax, nvp, w.init_blocks,
                                                w.local_blocks)
    assert not failures, failures[:3]
    return n_exact, n_tie


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_chain(name):
    w = workloads.generate(name=name, **CASES[name])
    say(f"[prefill] {name}: {w.num_tokens} tokens over {w.batch} requests, cols {w.cols}")
    plane, carrier, merged, err = run_chain(w)
    assert err == 0
    ref, amax = oracle_plane(w, w.cols)
    written = written_mask_prefill(w, w.cols)
    assert np.all(plane.view(np.uint32)[~written] == CANARY_BITS), "wrote past the columns"
    n_bad, ratio = compare_plane(plane, ref, amax, written)
    say(f"[prefill] {name}: worst |err| / tol = {ratio:.3g}")
    assert n_bad == 0
    n_exact, n_tie = check_rows(w, plane, carrier, merged, ref, amax)
    say(f"[prefill] {name}: rows exact {n_exact}, near ties {n_tie}")


def test_prefill_long_window():
    """8192 query tokens at the end of a 65536-key request (P256): sampled
    rows against the oracle, every row against the causal -inf pattern, the
    carrier and merged rows against the oracle's select and merge of the GPU
    plane."""
    w = workloads.generate(name="long_q8192_s64k", **LONG)
    plane, carrier, merged, err = run_chain(w)
    assert err == 0
    T, cols = w.num_tokens, w.cols
    pos = w.positions.numpy()
    # causal pattern: column c holds a finite value iff its block has a key at
    # or before the token's position
    visible = np.arange(cols)[None, :] * 128 <= pos[:, None]
    fin = np.isfinite(plane)
    assert np.array_equal(fin, np.broadcast_to(visible[:, None, :], fin.shape)), "causal pattern"
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 4096, T - 65, T - 64,
                                      T - 2, T - 1], rng.integers(0, T, 36)])).astype(np.int64)
    ref, amax = oracle_plane(w, cols, tokens=toks)
    n_bad, ratio = compare_plane(plane[toks], ref, amax, np.ones(ref.shape, dtype=bool))
    say(f"[prefill] long window: {len(toks)} sampled tokens, worst |err| / tol = {ratio:.3g}")
    assert n_bad == 0
    nvp = w.num_valid_pages.numpy()
    ps, pi, _ = oracle.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=w.num_ranges)
    assert_rows_equal(msa.row_scores(carrier).numpy(), msa.row_ids(carrier).numpy(), ps, pi,
                      "long carrier")
    ms, mi, missing = oracle.top16_merge(ps, pi, nvp, init_blocks=w.init_blocks,
                                         local_blocks=w.local_blocks)
    assert missing == 0
    assert_rows_equal(msa.row_scores(merged).numpy(), msa.row_ids(merged).numpy(), ms, mi,
                      "long merged")


def test_prefill_plan_for_another_plane_runs_nothing():
    w = workloads.generate(name="short", **CASES["short_ragged"])
    # a plan made for a plane 4 columns wider: the scorer refuses it
    plane, _, _, err = run_chain(w, plan_cols=w.cols + 4)
    assert err >= 1
    assert np.all(plane.view(np.uint32) == CANARY_BITS)


def test_prefill_bad_block_table_entries():
    w = workloads.generate(name="bad_bt", **CASES["short_ragged"])
    bt = w.block_table.clone()
    bt[2, 1] = w.index_k.shape[0] + 3   # request 2, keys 128..255: block 1
    bt[1, 0] = -1                       # request 1, keys 0..127: block 0
    plane, _, _, err = run_chain(w, block_table=bt)
    assert err >= 2
    qo = w.qo_indptr.numpy()
    assert np.all(np.isneginf(plane[qo[2]:qo[3], :, 1]))
    assert np.all(np.isneginf(plane[qo[1]:qo[2], :, 0]))
    # the other blocks still match the oracle
    ref, amax = oracle_plane(w, w.cols)
    written = written_mask_prefill(w, w.cols)
    written[qo[2]:qo[3], :, 1] = False
    written[qo[1]:qo[2], :, 0] = False
    n_bad, _ = compare_plane(plane, ref, amax, written)
    assert n_bad == 0


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_plan_covers_every_window_once(name):
    """Plan items: every window of 64 tokens (or the chunk's tail) appears
    with column ranges tiling [0, needed) in order, its last item filling
    [needed, W_b); no item for an empty chunk or an empty request."""
    w = workloads.generate(name=name, **CASES[name])
    T = w.num_tokens
    plan = msa.new_prefill_plan(T, w.batch, w.cols, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_prefill_window_plan(w.qo_indptr.to(DEV), w.seq_lens.to(DEV), plan, num_tokens=T,
                                cols=w.cols, errors=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    p = plan.cpu().numpy()
    count = int(p[0])
    assert tuple(p[1:4]) == (w.batch, T, w.cols)
    items = p[msa.PREFILL_PLAN_HEADER_WORDS:].reshape(-1, msa.PREFILL_ITEM_WORDS)[:count]
    want = []
    qo = w.qo_indptr.numpy()
    for b, s in enumerate(w.seq_lens.tolist()):
        qlen = int(qo[b + 1] - qo[b])
        if s <= 0 or qlen <= 0:
            continue
        wb = min(-(-(-(-s // 128)) // 4) * 4, w.cols)
        for t0 in range(0, qlen, 64):
            n = min(64, qlen - t0)
            pos0 = s - qlen + t0
            last = pos0 + n - 1
            needed = 0 if last < 0 else min(wb, last // 128 + 1)
            ranges = [(c, min(32, needed - c)) for c in range(0, needed, 32)] or [(0, 0)]
            for i, (c0, nc) in enumerate(ranges):
                want.append((b, int(qo[b]) + t0, n, pos0, c0, nc,
                             wb if i == len(ranges) - 1 else 0, s))
    assert [tuple(int(x) for x in it) for it in items] == want
