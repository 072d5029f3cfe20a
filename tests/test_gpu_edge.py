"""GPU edge cases through the C ABI, checked against the CPU oracle.

Select / merge (bit-exact): ties, signed zeros and -inf (the ranking
treats -0 == +0, lower id wins), all-equal rows (more than 64 candidates at
the threshold), empty and short rows, forced blocks covering everything,
num_valid_pages outside [0, cols] (error counter, clamped), rows wide enough
for the four-wave path, and up to the maximum number of ranges. A plane of
more than 2^31 elements (scorer and select).

Scorer: empty and one-token requests, sequences shorter than the decode
length, exact multiples of 128, page_size 256 with odd block counts, every
decode_query_len, a plane exactly as wide as the written columns, a plane
too narrow (error counter, clamped), out-of-range block_table entries
(error counter, block scored -inf), 5000 requests, and pages past byte
offset 2^32 of a larger-than-4-GiB cache.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS
from parity import assert_rows_equal, compare_plane, written_mask

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


TIE_POOL = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.5, 2.0], dtype=np.float32)


def plane_of(rng, T, cols, kind):
    if kind == "normal":
        return rng.standard_normal((T, 4, cols)).astype(np.float32)
    if kind == "ties":
        return rng.choice(TIE_POOL, size=(T, 4, cols)).astype(np.float32)
    if kind == "equal":
        return np.full((T, 4, cols), 0.25, dtype=np.float32)
    if kind == "zeros":
        return rng.choice(np.array([0.0, -0.0], np.float32), size=(T, 4, cols))
    if kind == "neginf":
        p = np.full((T, 4, cols), -np.inf, dtype=np.float32)
        p[:, :, ::7] = 1.0
        return p
    raise ValueError(kind)


def gpu_select(plane, nvp, init, local, R):
    T = plane.shape[0]
    scores = torch.from_numpy(np.ascontiguousarray(plane)).to(DEV)
    nvp_t = torch.from_numpy(np.ascontiguousarray(nvp, dtype=np.int32)).to(DEV)
    out = msa.new_rows(T, 4, R, device=DEV)
    out.fill_(0x7BADBEEF)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_select(scores, nvp_t, out, init_blocks=init, local_blocks=local, num_ranges=R,
                         errors=err)
    torch.cuda.synchronize()
    o = out.cpu()
    return msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), int(err.item()), out, nvp_t


def gpu_merge(rows, nvp_t, init, local):
    T = rows.shape[0]
    out = msa.new_rows(T, 4, device=DEV)
    out.fill_(0x7BADBEEF)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge(rows, nvp_t, out, init_blocks=init, local_blocks=local, errors=err)
    torch.cuda.synchronize()
    o = out.cpu()
    return msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), int(err.item())


SELECT_CASES = [
    # (cols, R, init, local, kind)
    (1, 1, 1, 2, "normal"),
    (3, 1, 0, 0, "ties"),
    (4, 2, 1, 2, "ties"),
    (63, 1, 16, 0, "normal"),
    (64, 1, 0, 16, "ties"),
    (65, 3, 8, 8, "ties"),
    (200, 1, 1, 2, "equal"),
    (200, 4, 2, 2, "zeros"),
    (256, 1, 1, 2, "neginf"),
    (1000, 1, 1, 4, "ties"),
    (1024, 1, 4, 4, "equal"),
    (2048, 1, 2, 2, "normal"),
    (2048, 2, 2, 2, "ties"),
    (2049, 1, 1, 2, "normal"),
    (4096, 1, 4, 4, "ties"),
    (8192, 1, 4, 4, "normal"),
    (8192, 8, 4, 4, "equal"),
    (12287, 1, 1, 2, "ties"),
    (12287, 5, 0, 0, "normal"),
]


@pytest.mark.parametrize("cols,R,init,local,kind", SELECT_CASES)
def test_select_and_merge_edge(cols, R, init, local, kind):
    rng = np.random.default_rng(cols * 7 + R)
    T = 5
    plane = plane_of(rng, T, cols, kind)
    nvp = np.array([cols, 0, min(cols, 5), int(rng.integers(0, cols + 1)), max(0, cols - 1)],
                   dtype=np.int32)
    gs, gi, err, rows, nvp_t = gpu_select(plane, nvp, init, local, R)
    os_, oi, obad = oracle.top16_select(plane, nvp, init_blocks=init, local_blocks=local,
                                        num_ranges=R)
    assert err == 0 and obad == 0
    assert_rows_equal(gs, gi, os_, oi, f"select cols={cols} R={R} {kind}")
    ms, mi, merr = gpu_merge(rows, nvp_t, init, local)
    ws, wi, _ = oracle.top16_select(plane, nvp, init_blocks=init, local_blocks=local,
                                    num_ranges=1)
    assert merr == 0
    assert_rows_equal(ms, mi, ws[:, :, 0], wi[:, :, 0], f"merge cols={cols} R={R} {kind}")


@pytest.mark.parametrize("R", [4, 100])
def test_merge_repeated_rows_stays_in_its_row(R):
    """Partial rows that repeat one select row R times (not disjoint column
    ranges), so every forced id appears R times: the merge counts the
    malformed input in `errors`, writes a row of at most 16 valid entries
    and nothing past `out` (R = 100 takes the four-wave path)."""
    rng = np.random.default_rng(900 + R)
    T, cols, init, local = 3, 256, 4, 4
    plane = plane_of(rng, T, cols, "normal")
    nvp = np.array([cols, 100, 40], dtype=np.int32)
    _, _, err, rows1, nvp_t = gpu_select(plane, nvp, init, local, 1)
    assert err == 0
    rows = rows1.repeat(1, 1, R, 1).contiguous()
    guard = 4
    buf = msa.new_rows(T * 4 + guard, device=DEV)
    buf.fill_(0x7BADBEEF)
    out = buf[:T * 4].view(T, 4, msa.ROW_WORDS)
    errs = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge(rows, nvp_t, out, init_blocks=init, local_blocks=local, errors=errs)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[T * 4:] == 0x7BADBEEF), "merge wrote past its output rows"
    assert int(errs.item()) >= T * 4, "malformed rows not counted"
    ids = msa.row_ids(b[:T * 4]).numpy()
    for r, row in enumerate(ids):
        n = int(nvp[r // 4])
        assert np.all((row == -1) | ((row >= 0) & (row < n))), f"row {r}: bad ids {row}"


@pytest.mark.parametrize("R", [16, 100, 768])
def test_merge_many_ranges(R):
    """Merge of up to 768 partial rows (12288 entries: the four-wave path)."""
    rng = np.random.default_rng(R)
    cols = max(R * 16, 1024)
    cols = min(cols, 12287)
    T = 3
    plane = plane_of(rng, T, cols, "ties" if R == 100 else "normal")
    nvp = np.array([cols, cols // 2, 7], dtype=np.int32)
    init, local = 2, 3
    gs, gi, err, rows, nvp_t = gpu_select(plane, nvp, init, local, R)
    os_, oi, _ = oracle.top16_select(plane, nvp, init_blocks=init, local_blocks=local,
                                     num_ranges=R)
    assert err == 0
    assert_rows_equal(gs, gi, os_, oi, f"select R={R}")
    ms, mi, merr = gpu_merge(rows, nvp_t, init, local)
    rs, ri, missing = oracle.top16_merge(os_, oi, nvp, init_blocks=init, local_blocks=local)
    assert merr == 0 and missing == 0
    assert_rows_equal(ms, mi, rs, ri, f"merge R={R}")


def test_select_num_valid_pages_out_of_range():
    """nvp < 0 or > cols: counted once per token and clamped, like the oracle."""
    rng = np.random.default_rng(3)
    T, cols = 4, 300
    plane = plane_of(rng, T, cols, "normal")
    nvp = np.array([-5, cols + 10, 20, cols], dtype=np.int32)
    gs, gi, err, _, _ = gpu_select(plane, nvp, 1, 2, 2)
    os_, oi, obad = oracle.top16_select(plane, nvp, init_blocks=1, local_blocks=2, num_ranges=2)
    assert obad == 2 and err == 2
    assert_rows_equal(gs, gi, os_, oi, "clamped nvp")


def test_merge_reports_missing_forced_block():
    rng = np.random.default_rng(4)
    T, cols = 2, 128
    plane = plane_of(rng, T, cols, "normal")
    nvp = np.array([cols, cols], dtype=np.int32)
    os_, oi, _ = oracle.top16_select(plane, nvp, init_blocks=2, local_blocks=2, num_ranges=2)
    oi = oi.copy()
    oi[0, 1, 0, 0] = -1  # drop forced block 0 of (token 0, head 1)
    s = torch.from_numpy(np.ascontiguousarray(os_)).view(torch.int32)
    i = torch.from_numpy(np.ascontiguousarray(oi))
    rows = torch.cat([s, i], dim=-1).contiguous().to(DEV)
    nvp_t = torch.from_numpy(nvp).to(DEV)
    ms, mi, merr = gpu_merge(rows, nvp_t, 2, 2)
    rs, ri, missing = oracle.top16_merge(os_, oi, nvp, init_blocks=2, local_blocks=2)
    assert missing == 1 and merr >= 1
    assert_rows_equal(ms, mi, rs, ri, "merge with a missing forced block")


# ---------------------------------------------------------------------------
# scorer edge cases
# ---------------------------------------------------------------------------

def run_scorer(w, cols, *, block_table=None, extra=0):
    T = w.num_tokens
    out = torch.full((T, 4, cols + extra), int(CANARY_BITS), dtype=torch.int32,
                     device=DEV).view(torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bt = w.block_table if block_table is None else block_table
    msa.msa_score_decode(w.index_q.to(DEV), w.index_k.to(DEV), bt.to(DEV), w.seq_lens.to(DEV),
                         out, page_size=w.page_size, decode_query_len=w.dql, errors=err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def check_plane(w, got, cols_total, block_table=None):
    bt = (w.block_table if block_table is None else block_table).numpy()
    ref, amax, _ = oracle.score_decode(w.index_q.numpy(), w.index_k.numpy(), bt,
                                       w.seq_lens.numpy(), page_size=w.page_size,
                                       decode_query_len=w.dql, cols=cols_total, want_amax=True)
    written = written_mask(w.seq_lens.numpy(), w.dql, cols_total)
    n_bad, ratio = compare_plane(got, ref, amax, written)
    assert n_bad == 0, f"{n_bad} elements out of tolerance (ratio {ratio})"
    assert np.all(got.view(np.uint32)[~written] == CANARY_BITS), "unwritten column touched"


@pytest.mark.parametrize("dql", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("page_size", [128, 256])
def test_scorer_ragged_small(dql, page_size):
    seqs = [0, 1, dql - 1 if dql > 1 else 2, 127, 128, 129, 383, 512, 777, 2048 + 5]
    w = workloads.generate(batch=len(seqs), seq=("list", seqs), page_size=page_size, dql=dql,
                           seed=100 + dql * 3 + page_size, scale=1.0)
    got, err = run_scorer(w, w.cols, extra=8)
    assert err == 0
    check_plane(w, got, w.cols + 8)


def test_scorer_plane_exactly_as_wide_as_written():
    w = workloads.generate(batch=2, seq=("list", [4096, 4096 - 128 * 3]), page_size=128, dql=2,
                           seed=7)
    assert w.cols == 32
    got, err = run_scorer(w, w.cols)
    assert err == 0
    check_plane(w, got, w.cols)


def test_scorer_plane_too_narrow_is_counted_and_clamped():
    w = workloads.generate(batch=2, seq=("list", [3000, 200]), page_size=256, dql=1, seed=8)
    cols = 8  # request 0 needs 24 columns
    got, err = run_scorer(w, cols)
    assert err == 1
    check_plane(w, got, cols)


def test_scorer_bad_block_table_entries():
    """Entries outside [0, num_pages) are counted; their blocks score -inf and
    nothing outside index_k is read."""
    w = workloads.generate(batch=2, seq=("list", [1000, 600]), page_size=128, dql=2, seed=9)
    bt = w.block_table.clone()
    num_pages = w.index_k.shape[0]
    bt[0, 2] = num_pages          # one past the end
    bt[1, 0] = -3                 # negative
    got, err = run_scorer(w, w.cols, block_table=bt)
    assert err == 2
    # expected: the oracle's plane with those two blocks forced to -inf
    ref_bt = w.block_table.clone()
    ref, amax, _ = oracle.score_decode(w.index_q.numpy(), w.index_k.numpy(), ref_bt.numpy(),
                                       w.seq_lens.numpy(), page_size=128, decode_query_len=2,
                                       cols=w.cols, want_amax=True)
    ref[0:2, :, 2] = -np.inf
    ref[2:4, :, 0] = -np.inf
    written = written_mask(w.seq_lens.numpy(), 2, w.cols)
    n_bad, ratio = compare_plane(got, ref, amax, written)
    assert n_bad == 0, (n_bad, ratio)


FUSED_CASES = [
    # (cols, R, init, local, kind)
    (1, 1, 1, 2, "normal"),
    (64, 3, 8, 8, "ties"),
    (300, 4, 1, 4, "equal"),
    (1024, 1, 1, 4, "ties"),
    (2048, 1, 2, 2, "normal"),
    (2050, 2, 0, 0, "zeros"),
    (8192, 8, 4, 4, "normal"),
    (8192, 8, 4, 4, "ties"),
    (8192, 16, 2, 14, "neginf"),
    (12287, 16, 1, 2, "normal"),
]


@pytest.mark.parametrize("cols,R,init,local,kind", FUSED_CASES)
@pytest.mark.parametrize("with_partial", [True, False])
def test_select_merge_fused(cols, R, init, local, kind, with_partial):
    """One-launch select + merge == msa_top16_select then msa_top16_merge ==
    the oracle, bit for bit (merged rows and, when requested, range rows)."""
    rng = np.random.default_rng(cols * 13 + R)
    T = 5
    plane = plane_of(rng, T, cols, kind)
    nvp = np.array([cols, 0, min(cols, 5), int(rng.integers(0, cols + 1)), cols + 3],
                   dtype=np.int32)
    scores = torch.from_numpy(np.ascontiguousarray(plane)).to(DEV)
    nvp_t = torch.from_numpy(nvp).to(DEV)
    out = msa.new_rows(T, 4, device=DEV)
    out.fill_(0x7BADBEEF)
    part = msa.new_rows(T, 4, R, device=DEV) if with_partial else None
    if part is not None:
        part.fill_(0x7BADBEEF)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_select_merge(scores, nvp_t, out, init_blocks=init, local_blocks=local,
                               num_ranges=R, partial=part, errors=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1  # the token with num_valid_pages > cols
    os_, oi, obad = oracle.top16_select(plane, nvp, init_blocks=init, local_blocks=local,
                                        num_ranges=R)
    assert obad == 1
    clamped = np.minimum(np.maximum(nvp, 0), cols)
    rs, ri, missing = oracle.top16_merge(os_, oi, clamped, init_blocks=init, local_blocks=local)
    assert missing == 0
    o = out.cpu()
    assert_rows_equal(msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), rs, ri,
                      f"fused merge cols={cols} R={R} {kind}")
    if part is not None:
        pc = part.cpu()
        assert_rows_equal(msa.row_scores(pc).numpy(), msa.row_ids(pc).numpy(), os_, oi,
                          f"fused ranges cols={cols} R={R} {kind}")


def test_scorer_large_batch():
    """5000 short requests: the streaming grid's two-pass request search runs
    over 79 chunks of 64 requests; the plane matches the oracle everywhere."""
    w = workloads.generate(batch=5000, seq=("loguniform", 1, 3000), page_size=128, dql=2,
                           seed=91)
    got, err = run_scorer(w, w.cols, extra=4)
    assert err == 0
    check_plane(w, got, w.cols + 4)


def test_scorer_pages_beyond_4gib():
    """An index-K cache larger than 4 GiB whose used pages (poison page
    included) all sit above byte offset 2^32: 64-bit page addressing. The
    plane matches the oracle run on the compact copy of the same pages."""
    w = workloads.generate(batch=3, seq=("list", [3000, 700, 256]), page_size=256, dql=3,
                           seed=77)
    pages = w.index_k.shape[0]
    base = (1 << 32) // (256 * 128) + 5  # first page whose bytes start past 4 GiB
    say(f"[test] index-K of {(base + pages) * 256 * 128 / 2**30:.2f} GiB")
    big = torch.empty((base + pages, 256, 128), dtype=torch.uint8, device=DEV)
    big[base:] = w.index_k.to(DEV)
    bt = (w.block_table + base).to(DEV)  # every slot, the poison page's too
    cols = w.cols + 4
    out = torch.full((w.num_tokens, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                     device=DEV).view(torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(w.index_q.to(DEV), big, bt, w.seq_lens.to(DEV), out,
                         page_size=256, decode_query_len=w.dql, errors=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.cpu().numpy()
    del big
    torch.cuda.empty_cache()
    check_plane(w, got, cols)


def test_plane_beyond_2g_elements():
    """A plane of more than 2^31 float32 elements (8193 requests x 8 tokens x
    4 heads x 8192 columns, 8.6 GB): 64-bit plane offsets in the scorer and
    the select. The last requests' rows match the oracle (plane within the
    score bound, select bit for bit on the GPU's plane)."""
    batch, dql, cols = 8193, 8, 8192
    w = workloads.generate(batch=batch, seq=("uniform", 1, 300), page_size=128, dql=dql,
                           seed=78, cols=cols, table_width=4)
    T = w.num_tokens
    assert T * 4 * cols > 2**31
    say(f"[test] plane of {T * 4 * cols * 4 / 1e9:.1f} GB")
    plane = torch.full((T, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                       device=DEV).view(torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(w.index_q.to(DEV), w.index_k.to(DEV), w.block_table.to(DEV),
                         w.seq_lens.to(DEV), plane, page_size=128, decode_query_len=dql,
                         errors=err)
    rows = msa.new_rows(T, 4, 1, device=DEV)
    rows.fill_(0x7BADBEEF)
    nvp = w.num_valid_pages.to(DEV)
    msa.msa_top16_select(plane, nvp, rows, init_blocks=1, local_blocks=2, num_ranges=1,
                         errors=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    last = 3  # the last requests: their rows sit past element 2^31
    t0 = (batch - last) * dql
    got = plane[t0:].cpu().numpy()
    got_rows = rows[t0:, :, 0].cpu()
    del plane, rows
    torch.cuda.empty_cache()
    assert t0 * 4 * cols < 2**31 < T * 4 * cols  # the checked rows straddle element 2^31
    sub = slice(batch - last, batch)
    sl = w.seq_lens[sub].numpy()
    ref, amax, _ = oracle.score_decode(w.index_q[t0:].numpy(), w.index_k.numpy(),
                                       w.block_table[sub].numpy(), sl, page_size=128,
                                       decode_query_len=dql, cols=cols, want_amax=True)
    written = written_mask(sl, dql, cols)
    n_bad, ratio = compare_plane(got, ref, amax, written)
    assert n_bad == 0, (n_bad, ratio)
    assert np.all(got.view(np.uint32)[~written] == CANARY_BITS)
    nvp_sub = w.num_valid_pages[t0:].numpy()
    rs, ri, _ = oracle.top16_select(got, nvp_sub, init_blocks=1, local_blocks=2, num_ranges=1)
    assert_rows_equal(msa.row_scores(got_rows).numpy(), msa.row_ids(got_rows).numpy(),
                      rs[:, :, 0], ri[:, :, 0], "select past element 2^31")


@pytest.mark.parametrize("blocks", [1, 7, 3000])
@pytest.mark.parametrize("bpw", [msa.STREAM_PROBE_PERSISTENT, 2, 4, 8, 16])
def test_stream_read_probe_reads_every_byte(blocks, bpw):
    """The streaming-read probe (the benchmark's ceiling for the scorer) reads
    every byte once at every shape: its xor of all the buffer's dwords equals
    the host's, for a partial last workgroup and a partial last wave."""
    g = torch.Generator().manual_seed(blocks)
    host = torch.randint(0, 256, (blocks * 16384,), dtype=torch.uint8, generator=g)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    sink = torch.zeros(msa.STREAM_PROBE_SINK_WORDS, dtype=torch.int32, device=DEV)
    msa.msa_stream_read_probe(host.to(DEV), sink, blocks_per_wave=bpw)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want


def test_scorer_latency_mode_large_batch():
    """300 short requests on a 4-column plane: batch x cols = 1200 puts the
    scorer in its one-column-per-wave mode while the batch needs the
    two-pass request search (more than 64 requests); the fused score+select
    takes the same mode and must agree bit for bit."""
    w = workloads.generate(batch=300, seq=("loguniform", 1, 512), page_size=128, dql=2,
                           seed=93, cols=4)
    assert w.batch * w.cols <= 2048
    got, err = run_scorer(w, w.cols)
    assert err == 0
    check_plane(w, got, w.cols)
    T = w.num_tokens
    plane = torch.full((T, 4, w.cols), int(CANARY_BITS), dtype=torch.int32,
                       device=DEV).view(torch.float32)
    rows = msa.new_rows(T, 4, 2, device=DEV)
    ws = msa.score_select_workspace(w.batch, 2, w.cols, 2, device=DEV)
    e2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_select(w.index_q.to(DEV), w.index_k.to(DEV), w.block_table.to(DEV),
                         w.seq_lens.to(DEV), plane, w.num_valid_pages.to(DEV), rows, ws,
                         page_size=128, decode_query_len=2, init_blocks=1, local_blocks=1,
                         num_ranges=2, errors=e2)
    ref_rows = msa.new_rows(T, 4, 2, device=DEV)
    msa.msa_top16_select(torch.from_numpy(got).to(DEV), w.num_valid_pages.to(DEV), ref_rows,
                         init_blocks=1, local_blocks=1, num_ranges=2, errors=e2)
    torch.cuda.synchronize()
    assert int(e2.item()) == 0
    assert np.array_equal(plane.cpu().numpy().view(np.uint32), got.view(np.uint32))
    assert torch.equal(rows, ref_rows)
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("R", [1, 2])
def test_merge_many_rows_equals_row_per_group(R):
    """msa_top16_merge over more than 16 384 rows launches several rows per
    workgroup (one wave each): its rows and error count must equal those of
    launches over slices of fewer rows, which take one row per workgroup.
    With R = 1 some rows are malformed (swapped entries, a replaced forced
    id, a repeated id, non-canonical padding), so both the copy of a row that
    is already its own merge and the full selection run in the many-row
    shape."""
    rng = np.random.default_rng(4242 + R)
    T, cols, init, local = 4200, 48, 2, 3  # 16 800 rows
    plane = plane_of(rng, T, cols, "ties" if R == 2 else "normal")
    nvp = rng.integers(0, cols + 1, size=T).astype(np.int32)
    _, _, err, rows_d, nvp_t = gpu_select(plane, nvp, init, local, R)
    assert err == 0
    rows = rows_d.cpu().clone()
    if R == 1:
        sc = rows[:, :, 0, :16].view(torch.float32)
        ids = rows[:, :, 0, 16:]
        bad = rng.choice(T, size=300, replace=False)
        for i, t in enumerate(bad):
            h = i % 4
            m = int((ids[t, h] >= 0).sum())
            kind = i % 4
            if kind == 0 and m >= 3:
                sc[t, h, [1, 2]] = sc[t, h, [2, 1]].clone()
                ids[t, h, [1, 2]] = ids[t, h, [2, 1]].clone()
            elif kind == 1 and m >= 1:
                ids[t, h, 0] = cols - 1
                sc[t, h, 0] = 7.0
            elif kind == 2 and m >= 2:
                ids[t, h, 1] = ids[t, h, 0]
            elif m < 16:
                sc[t, h, m] = 0.25
    rows = rows.contiguous().to(DEV)
    ms, mi, err_all = gpu_merge(rows, nvp_t, init, local)
    pieces_s, pieces_i, err_pieces = [], [], 0
    for lo in range(0, T, 1500):  # 6000 rows per launch
        s_, i_, e_ = gpu_merge(rows[lo:lo + 1500].contiguous(), nvp_t[lo:lo + 1500].contiguous(),
                               init, local)
        pieces_s.append(s_)
        pieces_i.append(i_)
        err_pieces += e_
    assert np.array_equal(mi, np.concatenate(pieces_i))
    assert np.array_equal(ms.view(np.uint32), np.concatenate(pieces_s).view(np.uint32))
    assert err_all == err_pieces
    if R == 2:
        # well-formed input: the merge is the oracle's
        ps = msa.row_scores(rows.cpu()).numpy()
        pi = msa.row_ids(rows.cpu()).numpy()
        os_, oi, missing = oracle.top16_merge(ps, pi, nvp, init_blocks=init, local_blocks=local)
        assert missing == 0 and err_all == 0
        assert np.array_equal(mi, oi)
        assert np.array_equal(ms.view(np.uint32), os_.view(np.uint32))


def test_single_row_merge_equals_full_merge():
    """msa_top16_merge with R = 1 copies a row that is already its own merge
    (valid ids ascending in front, every forced id, canonical padding) and
    selects any other: its rows must equal the R = 2 merge of the same row
    and an all-padding row (the full selection over the same entries), for
    well-formed rows and for rows with swapped entries, a forced id replaced,
    non-canonical padding, a hole before the last entry and a repeated id."""
    rng = np.random.default_rng(2024)
    T, cols, init, local = 6, 300, 2, 3
    plane = plane_of(rng, T, cols, "normal")
    nvp = np.array([cols, 100, 40, 7, 0, cols], dtype=np.int32)
    _, _, err, rows1, nvp_t = gpu_select(plane, nvp, init, local, 1)
    assert err == 0
    rows = rows1.cpu().clone()  # [T, 4, 1, 32] int32: 16 scores then 16 ids
    sc = rows[:, :, 0, :16].view(torch.float32)
    ids = rows[:, :, 0, 16:]
    # token 1: swap two valid entries; token 2: replace the first forced id
    # (0) by a candidate id; token 3: padding with a finite score; token 5:
    # a hole (id -1) before the last valid entry, and a repeated id
    sc[1, 0, [1, 2]] = sc[1, 0, [2, 1]].clone()
    ids[1, 0, [1, 2]] = ids[1, 0, [2, 1]].clone()
    ids[2, 1, 0] = 30
    sc[2, 1, 0] = 9.0
    last = int((ids[3, 2] >= 0).sum())
    if last < 16:
        sc[3, 2, last] = 0.5
    ids[5, 3, 5] = -1
    ids[5, 0, 4] = ids[5, 0, 3]
    single = rows.to(DEV)
    ms1, mi1, _ = gpu_merge(single, nvp_t, init, local)
    pad = torch.empty_like(rows)
    pad[..., :16] = torch.tensor(float("-inf")).view(torch.int32)
    pad[..., 16:] = -1
    pair = torch.cat([rows, pad], dim=2).contiguous().to(DEV)
    ms2, mi2, _ = gpu_merge(pair, nvp_t, init, local)
    assert np.array_equal(mi1, mi2)
    assert np.array_equal(ms1.view(np.uint32), ms2.view(np.uint32))
