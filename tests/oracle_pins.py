"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:

* a library routine (torch's CPU float8_e4m3fn -> float cast; numpy float64
  matrix products, which are exact here: every partial sum of e4m3fn products
  is a multiple of 2^-18 below 2^43);
* a closed form (one-hot rows, monotone keys with a known block maximum);
* brute force written differently from the oracle (whole-request score
  matrices with explicit masks; O(n^2) rank counting for the Top16);
* an invariant (written-column range, merge of split lists == whole-row
  select);
* the stored column-count table in tests/golden.

The tests run them on the real oracle; the mutation test runs them on oracle
builds with planted mistakes and expects at least one to fail.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
CANARY_BITS = np.uint32(0x7FC0DEAD)
NEG_INF = np.float32(-np.inf)


# ----------------------------------------------------------------------------
# independent helpers (library routines, not the oracle)
# ----------------------------------------------------------------------------

def torch_decode(codes) -> np.ndarray:
    """float64 values of uint8 e4m3fn codes, decoded by torch's own cast."""
    t = torch.as_tensor(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_codes() -> np.ndarray:
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def canary_plane(T: int, cols: int) -> np.ndarray:
    return np.full((T, 4, cols), CANARY_BITS, dtype=np.uint32).view(np.float32)


def brute_force_plane(index_q, index_k, block_table, seq_lens, page_size, dql, cols):
    """Score plane by whole-request matrices: keys gathered in position order,
    S = Q @ K^T in float64 (exact), explicit causal mask, block max, one
    rounding to float32. Unwritten entries are NaN, amax alongside."""
    q = np.asarray(index_q, dtype=np.uint8)
    k = np.asarray(index_k, dtype=np.uint8)
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    B = sl.shape[0]
    out = np.full((B * dql, 4, cols), np.nan, dtype=np.float32)
    amax = np.zeros((B * dql, 4, cols), dtype=np.float64)
    for b in range(B):
        s = int(sl[b])
        if s <= 0:
            continue
        p = np.arange(s)
        keys = k[bt[b, p // page_size], p % page_size]          # [s, 128] codes
        kd = torch_decode(keys)                                  # [s, 128]
        qd = torch_decode(q[b * dql:(b + 1) * dql]).reshape(dql * 4, 128)
        S = qd @ kd.T                                            # [dql*4, s]
        A = np.abs(qd) @ np.abs(kd).T
        nblk = -(-s // 128)
        ncols = min(-(-nblk // 4) * 4, cols)
        for r in range(dql * 4):
            j = r // 4
            pos = s - dql + j
            vis = p <= pos
            for c in range(ncols):
                sel = vis & (p >= 128 * c) & (p < 128 * c + 128)
                if sel.any():
                    out[b * dql + j, r % 4, c] = np.float32(S[r, sel].max())
                    amax[b * dql + j, r % 4, c] = A[r, sel].max()
                else:
                    out[b * dql + j, r % 4, c] = NEG_INF
    return out, amax


def brute_select_row(srow, n, lo, hi, init, local):
    """Top16 row by rank counting: a candidate is taken iff fewer than
    (16 - |forced|) other candidates beat it (higher score, or equal score and
    lower id). Returns (ids ascending, scores)."""
    valid = list(range(lo, min(hi, n)))
    forced = [i for i in valid if i < init or i >= n - local]
    cand = [i for i in valid if i not in forced]
    budget = 16 - len(forced)
    taken = []
    for x in cand:
        beat = 0
        for y in cand:
            if y == x:
                continue
            if srow[y] > srow[x] or (srow[y] == srow[x] and y < x):
                beat += 1
        if beat < budget:
            taken.append(x)
    ids = sorted(forced + taken)
    return ids, [srow[i] for i in ids]


def _assert_row(ids_row, sc_row, exp_ids, srow):
    m = len(exp_ids)
    assert m <= 16
    got_ids = [int(x) for x in ids_row]
    assert got_ids[:m] == exp_ids, (got_ids, exp_ids)
    assert all(x == -1 for x in got_ids[m:]), got_ids
    for i, idx in enumerate(exp_ids):
        assert np.float32(sc_row[i]).view(np.uint32) == np.float32(srow[idx]).view(np.uint32)
    assert all(np.isneginf(sc_row[m:]))


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_e4m3_table(orc):
    """Decode table == torch's cast for all 256 codes; spot closed forms."""
    t = orc.e4m3fn_table()
    ref = torch_decode(np.arange(256, dtype=np.uint8))
    nan_codes = sorted(np.where(np.isnan(t))[0].tolist())
    assert nan_codes == [0x7F, 0xFF], nan_codes
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(ref[fin]))
    # closed forms of the OCP E4M3 definition
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x30] == 0.5
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])


def pin_dots_vs_float64(orc, seed=7):
    """Exact dots == float64 numpy products of torch-decoded rows."""
    rng = np.random.default_rng(seed)
    fc = finite_codes()
    parts = [
        rng.choice(fc, size=(1500, 128)),
        torch.randn(500, 128, generator=torch.Generator().manual_seed(seed)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy(),
        rng.integers(0, 8, size=(50, 128)),            # subnormals only
    ]
    q = np.concatenate([p.astype(np.uint8) for p in parts])
    k = np.concatenate([rng.permutation(p.astype(np.uint8)) for p in parts])
    # extremes: 448*448*128 and -448*448*128
    q = np.concatenate([q, np.full((2, 128), 0x7E, np.uint8)])
    k = np.concatenate([k, np.stack([np.full(128, 0x7E, np.uint8), np.full(128, 0xFE, np.uint8)])])
    f32, exact = orc.dots(q, k)
    ref = (torch_decode(q) * torch_decode(k)).sum(axis=1)
    assert np.array_equal(exact, ref)
    assert np.array_equal(f32, ref.astype(np.float32))
    assert exact[-2] == 448.0 * 448.0 * 128 and exact[-1] == -448.0 * 448.0 * 128


def pin_code_pairs(orc):
    """One-hot rows: q . k == dec(a) * dec(b) for every pair of finite codes."""
    fc = finite_codes()
    a, b = np.meshgrid(fc, fc, indexing="ij")
    a, b = a.ravel(), b.ravel()
    n = a.size
    dim = (a.astype(np.int64) * 7 + b) % 128
    q = np.zeros((n, 128), dtype=np.uint8)
    k = np.zeros((n, 128), dtype=np.uint8)
    q[np.arange(n), dim] = a
    k[np.arange(n), dim] = b
    f32, exact = orc.dots(q, k)
    prod = torch_decode(a) * torch_decode(b)
    assert np.array_equal(exact, prod)
    assert np.array_equal(f32, prod.astype(np.float32))
    # NaN codes propagate
    q1 = np.zeros((2, 128), np.uint8)
    k1 = np.zeros((2, 128), np.uint8)
    q1[0, 3] = 0x7F
    k1[1, 5] = 0xFF
    f, _ = orc.dots(q1, k1)
    assert np.isnan(f).all()


def _tiny_workloads():
    yield workloads.generate(batch=3, seq=("list", [300, 1000, 129]), page_size=128, dql=1,
                             seed=11, pool=("exact", None))
    yield workloads.generate(batch=4, seq=("list", [700, 256, 513, 1]), page_size=256, dql=2,
                             seed=12, outlier_frac=0.05)
    yield workloads.generate(batch=6, seq=("list", [1, 7, 8, 9, 383, 640]), page_size=128,
                             dql=8, seed=13, scale=0.5)
    yield workloads.generate(batch=3, seq=("list", [0, 3, 1030]), page_size=256, dql=5, seed=14,
                             cols=12)


def pin_plane_brute_force(orc):
    """Oracle plane == whole-request brute force, bit for bit, incl. amax."""
    for w in _tiny_workloads():
        args = (w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(), w.seq_lens.numpy())
        plane, amax, bad = orc.score_decode(*args, page_size=w.page_size,
                                            decode_query_len=w.dql, cols=w.cols, want_amax=True)
        ref, ref_amax = brute_force_plane(*args, w.page_size, w.dql, w.cols)
        assert bad == 0
        written = ~np.isnan(ref)
        assert np.array_equal(np.isnan(plane), np.isnan(ref)), w.name
        assert np.array_equal(plane[written], ref[written]), w.name
        assert np.array_equal(amax[written], ref_amax[written]), w.name
        # sampled interface agrees with the plane
        T = w.num_tokens
        rows, cols = np.nonzero(written.reshape(T * 4, w.cols))
        s, a, bad2 = orc.score_sampled(*args, rows, cols, page_size=w.page_size,
                                       decode_query_len=w.dql)
        assert bad2 == 0
        assert np.array_equal(s, ref.reshape(T * 4, w.cols)[rows, cols])
        assert np.array_equal(a, ref_amax.reshape(T * 4, w.cols)[rows, cols])


def pin_plane_closed_form(orc):
    """q = 1.0 at dim 0; key p carries code min(p % 128, 126) at dim 0, so the
    block maximum is the value of the last visible key's code (codes 0x00..0x7E
    increase in value): tests the inclusive causal bound exactly."""
    dql = 8
    seqs = [1, 2, 127, 128, 129, 200, 256, 300]
    B = len(seqs)
    ps = 128
    npages = [-(-s // ps) for s in seqs]
    total = sum(npages)
    k = np.zeros((total + 1, ps, 128), dtype=np.uint8)
    k[:, :, 0] = np.minimum(np.arange(ps), 126).astype(np.uint8)[None, :]
    bt = np.full((B, 4), total, dtype=np.int32)
    perm = np.random.default_rng(3).permutation(total)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        off += n
    q = np.zeros((B * dql, 4, 128), dtype=np.uint8)
    q[:, :, 0] = 0x38  # 1.0
    cols = 4
    plane, _, bad = orc.score_decode(q, k, bt, np.array(seqs, np.int32), page_size=ps,
                                     decode_query_len=dql, cols=cols)
    assert bad == 0
    val = torch_decode(np.arange(256, dtype=np.uint8))
    for b, s in enumerate(seqs):
        nblk = -(-s // 128)
        for j in range(dql):
            pos = s - dql + j
            for c in range(cols):
                got = plane[b * dql + j, :, c]
                if c >= nblk:
                    want = -np.inf
                elif pos < 128 * c:
                    want = -np.inf
                else:
                    last = min(pos, s - 1, 128 * c + 127)
                    want = val[min(last % 128, 126)]
                assert np.all(got == np.float32(want)), (s, j, c, got, want)


def pin_written_range(orc):
    """Canary columns past roundup4(blocks) stay bit-identical; columns in
    [blocks, roundup4(blocks)) hold -inf; the rest are written."""
    for w in _tiny_workloads():
        T = w.num_tokens
        cols = w.cols + 8
        base = canary_plane(T, cols)
        plane, _, _ = orc.score_decode(w.index_q.numpy(), w.index_k.numpy(),
                                       w.block_table.numpy(), w.seq_lens.numpy(),
                                       page_size=w.page_size, decode_query_len=w.dql, cols=cols,
                                       plane=base)
        bits = plane.view(np.uint32)
        for b in range(w.batch):
            s = int(w.seq_lens[b])
            nblk = -(-s // 128) if s > 0 else 0
            wcols = -(-nblk // 4) * 4
            rows = slice(b * w.dql, (b + 1) * w.dql)
            assert np.all(bits[rows, :, wcols:] == CANARY_BITS), (w.name, b)
            assert np.all(np.isneginf(plane[rows, :, nblk:wcols])), (w.name, b)
            assert not np.any(bits[rows, :, :nblk] == CANARY_BITS), (w.name, b)


def pin_column_counts_golden(orc):
    """Written-column counts of the stored table (derived by hand from the
    column rule of the msa_icp_decode_index_score_sharded page)."""
    path = os.path.join(HERE, "golden", "column_counts.txt")
    n = 0
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            seq_len, page_size, want = (int(x) for x in line.split())
            assert orc.written_columns(seq_len) == want, (seq_len, page_size, want)
            n += 1
    assert n >= 10


def _random_plane(rng, T, cols, ties):
    if ties:
        pool = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.5, 2.0], dtype=np.float32)
        return rng.choice(pool, size=(T, 4, cols)).astype(np.float32)
    return rng.standard_normal((T, 4, cols)).astype(np.float32)


def pin_select_brute_force(orc, seed=5):
    """Oracle select == rank-counting brute force (ids and raw scores)."""
    rng = np.random.default_rng(seed)
    cases = [(1, 2, 1), (0, 0, 1), (16, 0, 1), (0, 16, 2), (8, 8, 3), (4, 4, 5), (2, 2, 4),
             (1, 4, 1)]
    for ci, (init, local, R) in enumerate(cases):
        for ties in (False, True):
            T, cols = 3, int(rng.integers(1, 90))
            s = _random_plane(rng, T, cols, ties)
            nvp = rng.integers(0, cols + 1, size=T).astype(np.int32)
            nvp[0] = cols
            if T > 1:
                nvp[1] = min(cols, int(rng.integers(0, 20)))
            sc, ids, bad = orc.top16_select(s, nvp, init_blocks=init, local_blocks=local,
                                            num_ranges=R)
            assert bad == 0
            w = -(-cols // R)
            for t in range(T):
                for h in range(4):
                    for r in range(R):
                        lo, hi = r * w, min(r * w + w, cols)
                        exp_ids, _ = brute_select_row(s[t, h], int(nvp[t]), lo, hi, init, local)
                        _assert_row(ids[t, h, r], sc[t, h, r], exp_ids, s[t, h])


def pin_select_invariants(orc, seed=6):
    """ids ascending, unique, valid; forced present; count = min(16, |valid|)."""
    rng = np.random.default_rng(seed)
    for init, local in [(1, 2), (4, 4), (2, 2), (1, 4), (0, 0), (16, 0)]:
        T, cols = 8, 700
        s = _random_plane(rng, T, cols, ties=bool(rng.integers(0, 2)))
        nvp = rng.integers(0, cols + 1, size=T).astype(np.int32)
        sc, ids, _ = orc.top16_select(s, nvp, init_blocks=init, local_blocks=local)
        for t in range(T):
            n = int(nvp[t])
            forced = set(range(min(init, n))) | set(range(max(0, n - local), n))
            for h in range(4):
                row = [int(x) for x in ids[t, h, 0] if x >= 0]
                assert row == sorted(set(row))
                assert all(0 <= x < n for x in row)
                assert forced <= set(row)
                assert len(row) == min(16, n)


def pin_merge_split_equivalence(orc, seed=8):
    """merge(select over R ranges) == select over the whole row, bit for bit;
    merge of one full row is the identity."""
    rng = np.random.default_rng(seed)
    for init, local in [(1, 2), (4, 4), (0, 0), (2, 14)]:
        for ties in (False, True):
            T, cols = 4, 256
            s = _random_plane(rng, T, cols, ties)
            nvp = rng.integers(0, cols + 1, size=T).astype(np.int32)
            nvp[0] = cols
            nvp[1] = 5
            whole_s, whole_i, _ = orc.top16_select(s, nvp, init_blocks=init, local_blocks=local)
            for R in (1, 2, 3, 8, cols // 4):
                ps, pi, _ = orc.top16_select(s, nvp, init_blocks=init, local_blocks=local,
                                             num_ranges=R)
                ms, mi, missing = orc.top16_merge(ps, pi, nvp, init_blocks=init,
                                                  local_blocks=local)
                assert missing == 0
                assert np.array_equal(mi, whole_i[:, :, 0]), (init, local, R)
                assert np.array_equal(ms.view(np.uint32), whole_s[:, :, 0].view(np.uint32))


def pin_merge_missing_forced(orc):
    """A merge input that lacks a forced id is reported."""
    T, cols = 1, 64
    s = np.arange(T * 4 * cols, dtype=np.float32).reshape(T, 4, cols)
    nvp = np.array([cols], np.int32)
    ps, pi, _ = orc.top16_select(s, nvp, init_blocks=2, local_blocks=2, num_ranges=2)
    pi = pi.copy()
    ps = ps.copy()
    pi[0, 0, 0, 0] = -1  # drop forced id 0 from head 0
    _, _, missing = orc.top16_merge(ps, pi, nvp, init_blocks=2, local_blocks=2)
    assert missing == 1


# ----------------------------------------------------------------------------
# row-sharded scoring and the column -> global id mapping
# ----------------------------------------------------------------------------

def shard_index_map(page_size: int, rank: int, world_size: int):
    """(index_scale, index_offset) taking rank `rank`'s plane column c to its
    global B128 block id: c itself at page_size 128, 2c + rank*2//world_size
    at page_size 256, where a column is a local page ("flashinfer.msa_ops.
    msa_icp_decode_index_score_sharded", description)."""
    if page_size == 128:
        return 1, 0
    return 2, rank * 2 // world_size


def brute_force_plane_sharded(index_q, index_k, block_table, seq_lens, page_size, dql, cols,
                              rank, world_size):
    """One rank's plane by whole-request matrices over the FULL cache: the
    rank owns rows [rank*R, rank*R + R) of every page (R = page_size /
    world_size); column c is the request's page c, so its keys are the
    positions p with p // page_size == c and rank*R <= p % page_size < rank*R + R.
    Written columns: the request's pages rounded up to four. float64 products
    (exact), explicit mask, one rounding. Unwritten entries are NaN."""
    q = np.asarray(index_q, dtype=np.uint8)
    k = np.asarray(index_k, dtype=np.uint8)
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    R = page_size // world_size
    B = sl.shape[0]
    out = np.full((B * dql, 4, cols), np.nan, dtype=np.float32)
    amax = np.zeros((B * dql, 4, cols), dtype=np.float64)
    for b in range(B):
        s = int(sl[b])
        if s <= 0:
            continue
        p = np.arange(s)
        kd = torch_decode(k[bt[b, p // page_size], p % page_size])
        qd = torch_decode(q[b * dql:(b + 1) * dql]).reshape(dql * 4, 128)
        S = qd @ kd.T
        A = np.abs(qd) @ np.abs(kd).T
        mine = (p % page_size >= rank * R) & (p % page_size < rank * R + R)
        ncols = min(-(-(-(-s // page_size)) // 4) * 4, cols)
        for r in range(dql * 4):
            j = r // 4
            vis = mine & (p <= s - dql + j)
            for c in range(ncols):
                sel = vis & (p // page_size == c)
                if sel.any():
                    out[b * dql + j, r % 4, c] = np.float32(S[r, sel].max())
                    amax[b * dql + j, r % 4, c] = A[r, sel].max()
                else:
                    out[b * dql + j, r % 4, c] = NEG_INF
    return out, amax


def _sharded_cases():
    # (workload, world_size)
    yield workloads.generate(batch=3, seq=("list", [300, 1000, 129]), page_size=128, dql=1,
                             seed=21), 2
    yield workloads.generate(batch=3, seq=("list", [700, 64, 1025]), page_size=128, dql=3,
                             seed=22, scale=0.5), 4
    yield workloads.generate(batch=4, seq=("list", [700, 256, 513, 1]), page_size=256, dql=2,
                             seed=23, outlier_frac=0.05), 2
    yield workloads.generate(batch=3, seq=("list", [0, 200, 1100]), page_size=256, dql=5,
                             seed=24), 4


def pin_sharded_plane_brute_force(orc):
    """A rank's plane == brute force over the full cache, bit for bit
    (values, amax and the written range, with spare columns that must stay
    unwritten)."""
    for w, ws in _sharded_cases():
        # 8 spare columns past the widest request's written range
        cols = max(4, -(-(-(-int(w.seq_lens.max()) // w.page_size)) // 4) * 4) + 8
        for rank in range(ws):
            shard = workloads.shard_rows(w.index_k, rank, ws).numpy()
            args = (w.index_q.numpy(), shard, w.block_table.numpy(), w.seq_lens.numpy())
            plane, amax, bad = orc.score_decode_sharded(
                *args, page_size=w.page_size, decode_query_len=w.dql, rank=rank,
                world_size=ws, cols=cols, want_amax=True)
            ref, ref_amax = brute_force_plane_sharded(
                w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(),
                w.seq_lens.numpy(), w.page_size, w.dql, cols, rank, ws)
            assert bad == 0
            written = ~np.isnan(ref)
            assert np.array_equal(np.isnan(plane), np.isnan(ref)), (w.name, rank)
            assert np.array_equal(plane[written], ref[written]), (w.name, rank)
            assert np.array_equal(amax[written], ref_amax[written]), (w.name, rank)


def pin_sharded_rows_partition(orc):
    """The ranks' rows partition every page, so per global B128 block the max
    over the ranks that hold its rows equals the unsharded plane's column
    (page_size 128: every rank holds part of block c; 256: rank r holds part
    of block 2c + r*2//world_size)."""
    for w, ws in _sharded_cases():
        args = (w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(),
                w.seq_lens.numpy())
        full, _, _ = orc.score_decode(*args, page_size=w.page_size, decode_query_len=w.dql,
                                      cols=w.cols)
        scols = max(4, -(-(-(-int(w.seq_lens.max()) // w.page_size)) // 4) * 4)
        combined = np.full(full.shape, -np.inf, dtype=np.float32)
        for rank in range(ws):
            shard = workloads.shard_rows(w.index_k, rank, ws).numpy()
            plane, _, _ = orc.score_decode_sharded(
                args[0], shard, args[2], args[3], page_size=w.page_size,
                decode_query_len=w.dql, rank=rank, world_size=ws, cols=scols)
            scale, offset = shard_index_map(w.page_size, rank, ws)
            for c in range(scols):
                gid = scale * c + offset
                if gid >= w.cols:
                    continue
                col = np.where(np.isnan(plane[:, :, c]), -np.inf, plane[:, :, c])
                combined[:, :, gid] = np.maximum(combined[:, :, gid], col)
        written = ~np.isnan(full)
        assert np.array_equal(combined[written], full[written]), w.name


def brute_select_row_mapped(srow, n, lo, hi, init, local, scale, offset):
    """Top16 row of columns [lo, hi) whose global ids are scale*c + offset, by
    rank counting on global ids (valid: id < n). Returns (ids, columns)."""
    cols = [c for c in range(lo, hi) if scale * c + offset < n]
    gid = {c: scale * c + offset for c in cols}
    forced = [c for c in cols if gid[c] < init or gid[c] >= n - local]
    cand = [c for c in cols if c not in forced]
    budget = 16 - len(forced)
    taken = []
    for x in cand:
        beat = sum(1 for y in cand if y != x and (srow[y] > srow[x] or
                                                  (srow[y] == srow[x] and gid[y] < gid[x])))
        if beat < budget:
            taken.append(x)
    chosen = sorted(forced + taken, key=lambda c: gid[c])
    return [gid[c] for c in chosen], chosen


def pin_mapped_select(orc, seed=25):
    """Mapped select: identity mapping == plain select; other mappings ==
    rank counting on global ids (ids, raw scores, padding)."""
    rng = np.random.default_rng(seed)
    for ties in (False, True):
        T, cols = 3, 70
        s = _random_plane(rng, T, cols, ties)
        nvp = np.array([cols, 9, int(rng.integers(0, cols + 1))], np.int32)
        a = orc.top16_select(s, nvp, init_blocks=2, local_blocks=3, num_ranges=3)
        b = orc.top16_select_mapped(s, nvp, init_blocks=2, local_blocks=3, num_ranges=3)
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[0].view(np.uint32),
                                                             b[0].view(np.uint32))
        for scale, offset, init, local, R in [(2, 0, 1, 2, 1), (2, 1, 4, 4, 3),
                                              (1, 0, 0, 16, 2), (2, 1, 16, 0, 1)]:
            nvp2 = np.array([scale * cols + offset, 17, int(rng.integers(0, 2 * cols))],
                            np.int32)
            sc, ids, bad = orc.top16_select_mapped(s, nvp2, init_blocks=init,
                                                   local_blocks=local, num_ranges=R,
                                                   index_scale=scale, index_offset=offset)
            assert bad == 0
            w = -(-cols // R)
            for t in range(T):
                for h in range(4):
                    for r in range(R):
                        exp_ids, exp_cols = brute_select_row_mapped(
                            s[t, h], int(nvp2[t]), r * w, min(r * w + w, cols), init, local,
                            scale, offset)
                        m = len(exp_ids)
                        got = [int(x) for x in ids[t, h, r]]
                        assert got[:m] == exp_ids and all(x == -1 for x in got[m:])
                        assert np.array_equal(sc[t, h, r, :m].view(np.uint32),
                                              s[t, h, exp_cols].view(np.uint32))
                        assert np.all(np.isneginf(sc[t, h, r, m:]))


def pin_sharded_chain_exact(orc):
    """Each rank's plane, mapped select over R ranges, then the merge of all
    ranks' rows == select over the unsharded plane, bit for bit (the merge
    keeps an id's highest score, and a block's max over its row shards is
    its unsharded max)."""
    for w, ws in _sharded_cases():
        args = (w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(),
                w.seq_lens.numpy())
        nvp = w.num_valid_pages.numpy()
        full, _, _ = orc.score_decode(*args, page_size=w.page_size, decode_query_len=w.dql,
                                      cols=w.cols)
        full = np.where(np.isnan(full), np.float32(-np.inf), full)
        ref_s, ref_i, _ = orc.top16_select(full, nvp, init_blocks=w.init_blocks,
                                           local_blocks=w.local_blocks)
        scols = max(4, -(-(-(-int(w.seq_lens.max()) // w.page_size)) // 4) * 4)
        R = 2
        rows_s, rows_i = [], []
        for rank in range(ws):
            shard = workloads.shard_rows(w.index_k, rank, ws).numpy()
            plane, _, _ = orc.score_decode_sharded(
                args[0], shard, args[2], args[3], page_size=w.page_size,
                decode_query_len=w.dql, rank=rank, world_size=ws, cols=scols)
            plane = np.where(np.isnan(plane), np.float32(-np.inf), plane)
            scale, offset = shard_index_map(w.page_size, rank, ws)
            ps, pi, bad = orc.top16_select_mapped(plane, nvp, init_blocks=w.init_blocks,
                                                  local_blocks=w.local_blocks, num_ranges=R,
                                                  index_scale=scale, index_offset=offset)
            assert bad == 0
            rows_s.append(ps)
            rows_i.append(pi)
        ms, mi, missing = orc.top16_merge(np.concatenate(rows_s, axis=2),
                                          np.concatenate(rows_i, axis=2), nvp,
                                          init_blocks=w.init_blocks,
                                          local_blocks=w.local_blocks)
        assert missing == 0, w.name
        assert np.array_equal(mi, ref_i[:, :, 0]), w.name
        assert np.array_equal(ms.view(np.uint32), ref_s[:, :, 0].view(np.uint32)), w.name


# ----------------------------------------------------------------------------
# prefill chunks ("prepare_msa_icp_indexer", the prefill chain)
# ----------------------------------------------------------------------------

def brute_force_plane_prefill(index_q, index_k, block_table, qo_indptr, seq_lens, page_size,
                              cols):
    """Prefill plane by whole-request matrices: the chunk's Q rows against all
    the request's keys in position order (float64, exact), an explicit
    position mask per query token, block max, one rounding to float32.
    Unwritten entries are NaN, amax alongside."""
    q = np.asarray(index_q, dtype=np.uint8)
    k = np.asarray(index_k, dtype=np.uint8)
    bt = np.asarray(block_table)
    qo = np.asarray(qo_indptr, dtype=np.int64)
    sl = np.asarray(seq_lens)
    T = int(qo[-1])
    out = np.full((T, 4, cols), np.nan, dtype=np.float32)
    amax = np.zeros((T, 4, cols), dtype=np.float64)
    for b in range(sl.shape[0]):
        s, t0, t1 = int(sl[b]), int(qo[b]), int(qo[b + 1])
        if s <= 0 or t1 == t0:
            continue
        p = np.arange(s)
        kd = torch_decode(k[bt[b, p // page_size], p % page_size])       # [s, 128]
        qd = torch_decode(q[t0:t1]).reshape((t1 - t0) * 4, 128)
        S = qd @ kd.T
        A = np.abs(qd) @ np.abs(kd).T
        nblk = -(-s // 128)
        ncols = min(-(-nblk // 4) * 4, cols)
        qlen = t1 - t0
        for r in range((t1 - t0) * 4):
            j = r // 4
            pos = s - qlen + j
            for c in range(ncols):
                sel = (p <= pos) & (p >= 128 * c) & (p < 128 * c + 128)
                if sel.any():
                    out[t0 + j, r % 4, c] = np.float32(S[r, sel].max())
                    amax[t0 + j, r % 4, c] = A[r, sel].max()
                else:
                    out[t0 + j, r % 4, c] = NEG_INF
    return out, amax


def _tiny_prefill_workloads():
    # short ragged chunks, one of a single token, one at the very start
    yield workloads.generate(batch=3, seq=("list", [129, 300, 700]), q_lens=("list", [1, 17, 64]),
                             page_size=128, dql=1, seed=31)
    # chunks crossing block and page boundaries at P256, one chunk = whole request
    yield workloads.generate(batch=3, seq=("list", [515, 1000, 130]),
                             q_lens=("list", [257, 300, 130]), page_size=256, dql=1, seed=32,
                             outlier_frac=0.05)
    # an empty chunk and an empty request between non-empty ones, narrow plane
    yield workloads.generate(batch=4, seq=("list", [640, 0, 383, 900]),
                             q_lens=("list", [3, 0, 0, 40]), page_size=128, dql=1, seed=33,
                             cols=12)


def _prefill_args(w):
    return (w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(), w.qo_indptr.numpy(),
            w.seq_lens.numpy())


def pin_prefill_brute_force(orc):
    """Prefill oracle plane == whole-request brute force, bit for bit, incl.
    amax; a token subset returns those tokens' rows."""
    for w in _tiny_prefill_workloads():
        args = _prefill_args(w)
        plane, amax, bad = orc.score_prefill(*args, page_size=w.page_size, cols=w.cols,
                                             want_amax=True)
        ref, ref_amax = brute_force_plane_prefill(*args, w.page_size, w.cols)
        assert bad == 0
        written = ~np.isnan(ref)
        assert np.array_equal(np.isnan(plane), np.isnan(ref)), w.name
        assert np.array_equal(plane[written], ref[written]), w.name
        assert np.array_equal(amax[written], ref_amax[written]), w.name
        toks = np.array([w.num_tokens - 1, 0, w.num_tokens // 2], dtype=np.int64)
        sub, sub_a, bad2 = orc.score_prefill(*args, page_size=w.page_size, cols=w.cols,
                                             tokens=toks, want_amax=True)
        assert bad2 == 0
        assert np.array_equal(sub, ref[toks], equal_nan=True), w.name
        assert np.array_equal(sub_a[~np.isnan(sub)], ref_amax[toks][~np.isnan(sub)]), w.name


def pin_prefill_closed_form(orc):
    """q = 1.0 at dim 0, key p carries code min(p % 128, 126) at dim 0: each
    block's maximum is the value of its last visible key, for every token of
    a chunk of 300 tokens (the inclusive causal bound per token)."""
    ps, s, qlen = 256, 700, 300
    npg = -(-s // ps)
    k = np.zeros((npg + 1, ps, 128), dtype=np.uint8)
    k[:, :, 0] = np.minimum(np.arange(ps) % 128, 126).astype(np.uint8)[None, :]
    bt = np.full((1, 4), npg, dtype=np.int32)
    bt[0, :npg] = np.random.default_rng(4).permutation(npg)
    q = np.zeros((qlen, 4, 128), dtype=np.uint8)
    q[:, :, 0] = 0x38  # 1.0
    cols = 8
    plane, _, bad = orc.score_prefill(q, k, bt, np.array([0, qlen], np.int32),
                                      np.array([s], np.int32), page_size=ps, cols=cols)
    assert bad == 0
    val = torch_decode(np.arange(256, dtype=np.uint8))
    nblk = -(-s // 128)
    for j in range(qlen):
        pos = s - qlen + j
        for c in range(cols):
            if c >= nblk or pos < 128 * c:
                want = -np.inf
            else:
                want = val[min(min(pos, 128 * c + 127) % 128, 126)]
            assert np.all(plane[j, :, c] == np.float32(want)), (j, c, plane[j, :, c], want)


def pin_prefill_uniform_chunks_are_decode(orc):
    """With every chunk decode_query_len tokens long the prefill plane is the
    decode plane (the decode plane is pinned by its own brute force)."""
    for w in _tiny_workloads():
        B = w.batch
        qo = (np.arange(B + 1) * w.dql).astype(np.int32)
        args = (w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy())
        dec, _, b1 = orc.score_decode(*args, w.seq_lens.numpy(), page_size=w.page_size,
                                      decode_query_len=w.dql, cols=w.cols)
        pre, _, b2 = orc.score_prefill(*args, qo, w.seq_lens.numpy(), page_size=w.page_size,
                                       cols=w.cols)
        assert b1 == b2 == 0
        assert np.array_equal(dec, pre, equal_nan=True), w.name


ALL_PINS = [
    pin_e4m3_table, pin_dots_vs_float64, pin_code_pairs, pin_plane_brute_force,
    pin_plane_closed_form, pin_written_range, pin_column_counts_golden, pin_select_brute_force,
    pin_select_invariants, pin_merge_split_equivalence, pin_merge_missing_forced,
    pin_sharded_plane_brute_force, pin_sharded_rows_partition, pin_mapped_select,
    pin_sharded_chain_exact, pin_prefill_brute_force, pin_prefill_closed_form,
    pin_prefill_uniform_chunks_are_decode,
]
