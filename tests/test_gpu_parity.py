"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* score plane: every written element within 1e-5 * A of the oracle, -inf
  where the oracle has -inf, and every column past roundup4(blocks) left
  bit-identical (canary);
* Top16 select run on the oracle's plane: bit-exact rows;
* select + merge on the GPU's own plane vs the oracle on the same plane:
  bit-exact rows (all five workloads at full size);
* end to end (GPU plane -> GPU Top16 vs oracle plane -> oracle Top16): equal
  ids except near-ties within the tolerance band;
* fp8 decode: every pair of finite e4m3fn codes through the scorer equals
  the exact product.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_msa_amd as msa
import workloads
from oracle_pins import CANARY_BITS, torch_decode
from parity import assert_rows_equal, compare_e2e_rows, compare_plane, written_mask

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Case:
    """A workload on the device plus its oracle plane (computed once)."""

    def __init__(self, w: workloads.Workload):
        self.w = w
        self.q = w.index_q.to(DEV)
        self.k = w.index_k.to(DEV)
        self.bt = w.block_table.to(DEV)
        self.sl = w.seq_lens.to(DEV)
        self.nvp = w.num_valid_pages.to(DEV)
        self._oracle = None

    @property
    def oracle_plane(self):
        if self._oracle is None:
            w = self.w
            plane, amax, bad = oracle.score_decode(
                w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(), w.seq_lens.numpy(),
                page_size=w.page_size, decode_query_len=w.dql, cols=w.cols, want_amax=True)
            assert bad == 0
            self._oracle = (plane, amax)
        return self._oracle

    def gpu_plane(self, cols=None, canary=True):
        w = self.w
        cols = cols or w.cols
        if canary:
            out = torch.full((w.num_tokens, 4, cols), int(CANARY_BITS), dtype=torch.int32,
                             device=DEV).view(torch.float32)
        else:
            out = torch.empty((w.num_tokens, 4, cols), dtype=torch.float32, device=DEV)
        errors = torch.zeros(1, dtype=torch.int32, device=DEV)
        msa.msa_score_decode(self.q, self.k, self.bt, self.sl, out, page_size=w.page_size,
                             decode_query_len=w.dql, errors=errors)
        torch.cuda.synchronize()
        return out.cpu().numpy(), int(errors.item())


_CASES: dict = {}


def config_case(n: int) -> Case:
    if n not in _CASES:
        say(f"[gen] config {n}")
        _CASES[n] = Case(workloads.config(n))
    return _CASES[n]


def gpu_select(plane_np_or_t, nvp_t, init, local, R):
    scores = plane_np_or_t if torch.is_tensor(plane_np_or_t) else torch.from_numpy(
        np.ascontiguousarray(plane_np_or_t)).to(DEV)
    T = scores.shape[0]
    out = msa.new_rows(T, 4, R, device=DEV)
    out.fill_(0x7BADBEEF)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_select(scores, nvp_t, out, init_blocks=init, local_blocks=local, num_ranges=R,
                         errors=errors)
    torch.cuda.synchronize()
    o = out.cpu()
    return msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), int(errors.item())


def gpu_merge(part_rows_t, nvp_t, init, local):
    T = part_rows_t.shape[0]
    out = msa.new_rows(T, 4, device=DEV)
    out.fill_(0x7BADBEEF)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_top16_merge(part_rows_t, nvp_t, out, init_blocks=init, local_blocks=local,
                        errors=errors)
    torch.cuda.synchronize()
    o = out.cpu()
    return msa.row_scores(o).numpy(), msa.row_ids(o).numpy(), int(errors.item())


def rows_tensor(scores, ids):
    """[..., 16] scores + ids -> int32 rows [..., 32] on the device."""
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).view(torch.int32)
    i = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32))
    return torch.cat([s, i], dim=-1).contiguous().to(DEV)


# ---------------------------------------------------------------------------
# fp8 decode through the scorer
# ---------------------------------------------------------------------------

def test_e4m3_code_pairs_through_scorer():
    """Query row a holds code a at one dim; every key of block b holds code b
    in all dims; so plane[a, b] = dec(a) * dec(b) exactly (an 8-bit product
    of two 4-bit significands is exact in fp32)."""
    say("[test] e4m3 code pairs")
    c = np.arange(256, dtype=np.uint8)
    fc = c[(c & 0x7F) != 0x7F]                    # 254 finite codes
    nb = fc.size + 2                              # blocks per request: codes + 2 filler blocks
    dql = 8
    rows_per_req = 4 * dql                        # 32 query rows per request
    B = -(-fc.size // rows_per_req)               # 8 requests
    seq = nb * 128
    pages = nb                                    # page_size 128, one block per page
    k = np.zeros((pages + 1, 128, 128), dtype=np.uint8)
    k[:fc.size] = fc[:, None, None]
    bt = np.tile(np.arange(pages, dtype=np.int32), (B, 1))
    q = np.zeros((B * dql, 4, 128), dtype=np.uint8)
    qa = np.zeros(B * rows_per_req, dtype=np.uint8)
    qa[:fc.size] = fc
    qflat = q.reshape(B * rows_per_req, 128)
    qflat[np.arange(B * rows_per_req), np.arange(B * rows_per_req) % 128] = qa
    cols = -(-nb // 4) * 4
    out = torch.zeros((B * dql, 4, cols), dtype=torch.float32, device=DEV)
    msa.msa_score_decode(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                         torch.from_numpy(bt).to(DEV),
                         torch.full((B,), seq, dtype=torch.int32, device=DEV), out,
                         page_size=128, decode_query_len=dql)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B * rows_per_req, cols)[:fc.size, :fc.size]
    dec = torch_decode(fc)
    want = (dec[:, None] * dec[None, :]).astype(np.float32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} code pairs differ; first (a, b) codes "
                           f"{[(int(fc[i]), int(fc[j])) for i, j in bad[:5]]} got "
                           f"{[float(got[i, j]) for i, j in bad[:5]]} want "
                           f"{[float(want[i, j]) for i, j in bad[:5]]}")


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_score_plane_parity(n):
    case = config_case(n)
    w = case.w
    say(f"[test] score plane config {n} ({w.name}) keys={w.total_keys}")
    extra = min(8, 8192 - w.cols)  # canary columns past the plane's own width
    got, errs = case.gpu_plane(cols=w.cols + extra)
    assert errs == 0
    ref, amax = case.oracle_plane
    T = w.num_tokens
    written = written_mask(w.seq_lens.numpy(), w.dql, w.cols + extra)
    ref_full = np.full((T, 4, w.cols + extra), np.nan, np.float32)
    ref_full[:, :, :w.cols] = ref
    amax_full = np.zeros((T, 4, w.cols + extra))
    amax_full[:, :, :w.cols] = amax
    n_bad, ratio = compare_plane(got, ref_full, amax_full, written)
    say(f"   worst |err| / tol = {ratio:.3g}")
    assert n_bad == 0, f"{n_bad} plane elements outside tolerance (worst ratio {ratio})"
    bits = got.view(np.uint32)
    assert np.all(bits[~written] == CANARY_BITS), "a column past roundup4(blocks) was written"


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_select_on_oracle_plane_bit_exact(n):
    case = config_case(n)
    w = case.w
    say(f"[test] select on oracle plane config {n} R={w.num_ranges}")
    ref, _ = case.oracle_plane
    plane = np.where(np.isnan(ref), np.float32(-np.inf), ref).astype(np.float32)
    nvp = w.num_valid_pages.numpy()
    gs, gi, errs = gpu_select(plane, case.nvp, w.init_blocks, w.local_blocks, w.num_ranges)
    os_, oi, obad = oracle.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                        local_blocks=w.local_blocks, num_ranges=w.num_ranges)
    assert errs == 0 and obad == 0
    assert_rows_equal(gs, gi, os_, oi, f"select config {n}")
    if w.num_ranges > 1:
        ms, mi, merrs = gpu_merge(rows_tensor(gs, gi), case.nvp, w.init_blocks, w.local_blocks)
        rs, ri, missing = oracle.top16_merge(os_, oi, nvp, init_blocks=w.init_blocks,
                                             local_blocks=w.local_blocks)
        assert merrs == 0 and missing == 0
        assert_rows_equal(ms, mi, rs, ri, f"merge config {n}")
        ws, wi, _ = oracle.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                        local_blocks=w.local_blocks, num_ranges=1)
        assert_rows_equal(ms, mi, ws[:, :, 0], wi[:, :, 0], f"merge == whole-row select {n}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_end_to_end(n):
    """The chain as the benchmark runs it: plane, select over R ranges,
    merge when R > 1, all on the GPU; checked against the oracle chain and,
    bit-exactly, against the oracle's select/merge on the GPU's own plane."""
    case = config_case(n)
    w = case.w
    say(f"[test] end to end config {n}")
    T, R = w.num_tokens, w.num_ranges
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=DEV)
    part = msa.new_rows(T, 4, R, device=DEV)
    final = msa.new_rows(T, 4, device=DEV)
    errors = torch.zeros(1, dtype=torch.int32, device=DEV)
    msa.msa_score_decode(case.q, case.k, case.bt, case.sl, plane, page_size=w.page_size,
                         decode_query_len=w.dql, errors=errors)
    msa.msa_top16_select(plane, case.nvp, part, init_blocks=w.init_blocks,
                         local_blocks=w.local_blocks, num_ranges=R, errors=errors)
    if R > 1:
        msa.msa_top16_merge(part, case.nvp, final, init_blocks=w.init_blocks,
                            local_blocks=w.local_blocks, errors=errors)
    else:
        final.copy_(part[:, :, 0])
    torch.cuda.synchronize()
    assert int(errors.item()) == 0
    if 1 < R <= 16 and -(-w.cols // R) <= 2048:
        # the one-launch select + merge on the same plane: bit-identical
        # merged rows and range rows, then merged rows alone (the form the
        # benchmark times beside its step)
        fused = msa.new_rows(T, 4, device=DEV)
        fused_part = msa.new_rows(T, 4, R, device=DEV)
        fused.fill_(0x7BADBEEF)
        fused_part.fill_(0x7BADBEEF)
        msa.msa_top16_select_merge(plane, case.nvp, fused, init_blocks=w.init_blocks,
                                   local_blocks=w.local_blocks, num_ranges=R,
                                   partial=fused_part, errors=errors)
        torch.cuda.synchronize()
        assert int(errors.item()) == 0
        assert torch.equal(fused, final)
        assert torch.equal(fused_part, part)
        fused.fill_(0x7BADBEEF)  # the benchmark's form: merged rows only
        msa.msa_top16_select_merge(plane, case.nvp, fused, init_blocks=w.init_blocks,
                                   local_blocks=w.local_blocks, num_ranges=R, errors=errors)
        torch.cuda.synchronize()
        assert int(errors.item()) == 0
        assert torch.equal(fused, final)
    gplane = plane.cpu().numpy()
    fin = final.cpu()
    g_s, g_i = msa.row_scores(fin).numpy(), msa.row_ids(fin).numpy()
    nvp = w.num_valid_pages.numpy()

    # select/merge exactness on the GPU's own plane
    ps, pi, _ = oracle.top16_select(gplane, nvp, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=R)
    if R > 1:
        os_, oi, _ = oracle.top16_merge(ps, pi, nvp, init_blocks=w.init_blocks,
                                        local_blocks=w.local_blocks)
    else:
        os_, oi = ps[:, :, 0], pi[:, :, 0]
    assert_rows_equal(g_s, g_i, os_, oi, f"GPU-plane chain config {n}")

    # against the oracle's own chain, near-ties exempt
    ref, amax = case.oracle_plane
    rs, ri, _ = oracle.top16_select(ref, nvp, init_blocks=w.init_blocks,
                                    local_blocks=w.local_blocks, num_ranges=1)
    n_exact, n_tie, failures = compare_e2e_rows(g_i, ri[:, :, 0], ref, amax, nvp, w.init_blocks,
                                                w.local_blocks)
    say(f"   rows exact={n_exact} near-tie={n_tie} failed={len(failures)}")
    assert not failures, failures[:3]
