"""Host checks of the end-to-end comparison rule in tests/parity.py: a GPU
row that differs from the oracle's is accepted only when some plane within
1e-5 * A of the oracle's, block by block, selects it exactly."""
from __future__ import annotations

import numpy as np

from parity import compare_e2e_rows


def _case(scores, amax, n, init=0, local=0):
    plane = np.full((1, 4, len(scores)), -np.inf, dtype=np.float32)
    a = np.zeros((1, 4, len(scores)), dtype=np.float64)
    plane[0, :, :] = scores
    a[0, :, :] = amax
    return plane, a, np.array([n], dtype=np.int32)


def _row(ids):
    r = np.full((1, 4, 16), -1, dtype=np.int32)
    r[0, :, :len(ids)] = ids
    return r


def test_swap_within_own_tolerances_is_accepted():
    # 17 valid blocks; block 16 (dropped) sits 1.5e-5 below block 15 (kept);
    # A = 1 for both, so tol = 1e-5 each and the swap is admissible
    s = np.arange(17, 0, -1, dtype=np.float64)
    s[15], s[16] = 1.0, 1.0 - 1.5e-5
    amax = np.ones(17)
    plane, a, nvp = _case(s.astype(np.float32), amax, 17)
    oracle_ids = _row(list(range(16)))
    gpu_ids = _row(list(range(15)) + [16])
    ex, tie, fails = compare_e2e_rows(gpu_ids, oracle_ids, plane, a, nvp, 0, 0)
    assert (ex, tie, fails) == (0, 4, [])


def test_swap_beyond_boundary_tolerances_is_rejected_even_if_row_max_a_is_large():
    # the same gap, but the two boundary blocks have A = 0.5 (tol 5e-6 each)
    # while another block of the row has a huge A: the row maximum must not
    # widen the band
    s = np.arange(17, 0, -1, dtype=np.float64)
    s[15], s[16] = 1.0, 1.0 - 1.5e-5
    amax = np.full(17, 0.5)
    amax[0] = 1e4
    plane, a, nvp = _case(s.astype(np.float32), amax, 17)
    gpu_ids = _row(list(range(15)) + [16])
    ex, tie, fails = compare_e2e_rows(gpu_ids, _row(list(range(16))), plane, a, nvp, 0, 0)
    assert ex == 0 and tie == 0 and len(fails) == 4


def test_dropping_a_forced_block_is_rejected():
    s = np.linspace(5, 1, 20)
    plane, a, nvp = _case(s.astype(np.float32), np.ones(20), 20)
    oracle_ids = _row(list(range(15)) + [19])  # init 0, local 1: block 19 forced
    gpu_ids = _row(list(range(16)))
    _, tie, fails = compare_e2e_rows(gpu_ids, oracle_ids, plane, a, nvp, 0, 1)
    assert tie == 0 and len(fails) == 4


def test_picking_a_far_block_is_rejected():
    # the GPU keeps block 19 (score 0.1) over block 15 (score 1.0)
    s = np.arange(20, 0, -1, dtype=np.float64) / 20
    plane, a, nvp = _case(s.astype(np.float32), np.ones(20), 20)
    gpu_ids = _row(list(range(15)) + [19])
    _, tie, fails = compare_e2e_rows(gpu_ids, _row(list(range(16))), plane, a, nvp, 0, 0)
    assert tie == 0 and len(fails) == 4


def test_identical_rows_count_as_exact():
    s = np.linspace(3, 1, 10)
    plane, a, nvp = _case(s.astype(np.float32), np.ones(10), 10)
    ids = _row(list(range(10)))
    assert compare_e2e_rows(ids, ids, plane, a, nvp, 1, 2) == (4, 0, [])
