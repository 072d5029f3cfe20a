"""msa_score_select_noalloc (no workspace argument, the library's own device
scratch array) against msa_score_select on a caller workspace: two calls in a
row on the same stream, the second with a smaller input, each compared bit for
bit (range rows, merged rows, and the plane where one is passed), with both
error counters zero. The first call leaves the scratch array full of a larger
problem's pool and counters; the second must not read any of it."""
from __future__ import annotations

import sys

import pytest
import torch

import sparse_attention_block_msa_amd as msa
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
FILL = 0x7BADBEEF

# (large, then smaller) pairs: sizes, mode of each call (pool: no plane)
SEQUENCES = {
    "pool_merged_then_plane": (
        dict(batch=16, seq=("uniform", 16384, 131072), page_size=256, dql=4, init=2, local=2,
             ranges=4, seed=7101),
        True,
        dict(batch=3, seq=("uniform", 1024, 8192), page_size=128, dql=1, init=1, local=2,
             ranges=2, seed=7102),
        False),
    "plane_then_pool_merged": (
        dict(batch=8, seq=("uniform", 8192, 65536), page_size=128, dql=2, init=1, local=4,
             ranges=8, seed=7103),
        False,
        dict(batch=2, seq=("uniform", 2048, 16384), page_size=256, dql=8, init=4, local=4,
             ranges=3, seed=7104),
        True),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_call(w, pool: bool, tag: str):
    """Runs msa_score_select (own zeroed workspace) and msa_score_select_noalloc
    on workload w and asserts identical outputs."""
    T, R, cols = w.num_tokens, w.num_ranges, w.cols
    say(f"[no_alloc] {tag}: B={w.batch} dql={w.dql} P{w.page_size} cols={cols} R={R} "
        f"pool={pool}")
    q, k, sl = w.index_q.to(DEV), w.index_k.to(DEV), w.seq_lens.to(DEV)
    bt, nvp = w.block_table.to(DEV), w.num_valid_pages.to(DEV)
    sel = dict(page_size=w.page_size, decode_query_len=w.dql, init_blocks=w.init_blocks,
               local_blocks=w.local_blocks, num_ranges=R, cols=cols)
    outs = []
    for noalloc in (False, True):
        plane = None
        if not pool:
            plane = torch.full((T, 4, cols), FILL, dtype=torch.int32, device=DEV).view(
                torch.float32)
        rows = msa.new_rows(T, 4, R, device=DEV)
        rows.fill_(FILL)
        merged = msa.new_rows(T, 4, device=DEV)
        merged.fill_(FILL)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        if noalloc:
            msa.msa_score_select_noalloc(q, k, bt, sl, plane, nvp, rows, merged=merged,
                                         errors=err, **sel)
        else:
            ws = msa.score_select_workspace(w.batch, w.dql, cols, R, pool=pool, device=DEV)
            msa.msa_score_select(q, k, bt, sl, plane, nvp, rows, ws, merged=merged, errors=err,
                                 **sel)
        torch.cuda.synchronize()
        outs.append((None if plane is None else plane.view(torch.int32).cpu(), rows.cpu(),
                     merged.cpu(), int(err.item())))
    (p0, r0, m0, e0), (p1, r1, m1, e1) = outs
    assert e0 == 0 and e1 == 0, (e0, e1)
    assert torch.equal(r0, r1), f"{tag}: range rows differ"
    assert torch.equal(m0, m1), f"{tag}: merged rows differ"
    if p0 is not None:
        assert torch.equal(p0, p1), f"{tag}: planes differ"
    # rows were written (no fill left) and merged rows hold ascending ids
    assert not (r1 == FILL).all(dim=-1).any()
    ids = m1[..., 16:]
    valid = ids >= 0
    assert bool(((ids[..., 1:] > ids[..., :-1]) | ~valid[..., 1:]).all())


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_matches_workspace_entry_point(name):
    big, big_pool, small, small_pool = SEQUENCES[name]
    wa = workloads.generate(name=name + "_first", **big)
    wb = workloads.generate(name=name + "_second", **small)
    assert wb.num_tokens * wb.cols < wa.num_tokens * wa.cols
    one_call(wa, big_pool, name + " call 1")
    one_call(wb, small_pool, name + " call 2 (smaller)")
