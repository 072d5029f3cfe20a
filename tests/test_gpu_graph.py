"""The chain under HIP graph capture, through the C ABI.

The library never allocates, synchronises or issues memsets, so a caller can
capture its launches in a graph. Each test captures the chain once, then
replays it several times with the program's own eager work and
synchronisations between replays, and checks every replay bit for bit
against the eager result of the same launches.
"""
from __future__ import annotations

import pytest
import torch

import sparse_attention_block_msa_amd as msa
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def _inputs(n):
    w = workloads.config(n)
    return (w, w.index_q.to(DEV), w.index_k.to(DEV), w.block_table.to(DEV), w.seq_lens.to(DEV),
            w.num_valid_pages.to(DEV))


@pytest.mark.parametrize("n", [2, 3])
def test_chain_graph_replays_match_eager(n):
    w, q, k, bt, sl, nvp = _inputs(n)
    T, R = w.num_tokens, w.num_ranges
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    part = msa.new_rows(T, 4, R, device=DEV)
    final = msa.new_rows(T, 4, device=DEV)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_warmup()

    def chain(stream):
        msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size, decode_query_len=w.dql,
                             errors=errors, stream=stream)
        msa.msa_top16_select(plane, nvp, part, init_blocks=w.init_blocks,
                             local_blocks=w.local_blocks, num_ranges=R, errors=errors,
                             stream=stream)
        msa.msa_top16_merge(part, nvp, final, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks, errors=errors, stream=stream)

    # the plane's unwritten columns are never touched, so every run starts
    # from the same fill
    plane.fill_(float("nan"))
    chain(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_plane, ref_part, ref_final = plane.clone(), part.clone(), final.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            chain(side)
    torch.cuda.synchronize()
    for rep in range(4):
        plane.fill_(float("nan"))  # eager work between replays
        part.fill_(-7)
        final.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plane.view(torch.int32), ref_plane.view(torch.int32)), rep
        assert torch.equal(part, ref_part), rep
        assert torch.equal(final, ref_final), rep
    assert int(errors.item()) == 0


def test_score_select_graph_replays_leave_workspace_zero():
    """The fused launch resets its counters itself, so replays need no memset
    between them."""
    w, q, k, bt, sl, nvp = _inputs(3)
    T, R = w.num_tokens, 4
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    rows = msa.new_rows(T, 4, R, device=DEV)
    merged = msa.new_rows(T, 4, device=DEV)
    ws = msa.score_select_workspace(w.batch, w.dql, w.cols, R, device=DEV)

    def launch(stream):
        msa.msa_score_select(q, k, bt, sl, plane, nvp, rows, ws, page_size=w.page_size,
                             decode_query_len=w.dql, init_blocks=w.init_blocks,
                             local_blocks=w.local_blocks, num_ranges=R, merged=merged,
                             stream=stream)

    plane.fill_(float("nan"))  # unwritten columns keep this fill
    launch(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_plane, ref_rows, ref_merged = plane.clone(), rows.clone(), merged.clone()
    assert int(ws.count_nonzero()) == 0

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            launch(side)
    torch.cuda.synchronize()
    for rep in range(4):
        plane.fill_(float("nan"))
        rows.fill_(-7)
        merged.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plane.view(torch.int32), ref_plane.view(torch.int32)), rep
        assert torch.equal(rows, ref_rows), rep
        assert torch.equal(merged, ref_merged), rep
        assert int(ws.count_nonzero()) == 0, rep
