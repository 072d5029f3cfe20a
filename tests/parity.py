"""Comparison helpers for GPU-vs-oracle parity.

Tolerances:

* Score plane: |S_gpu - S_oracle| <= 1e-5 * A, where A is the largest
  sum_i |q_i k_i| over the block's visible keys. fp32 recursive summation of
  128 products errs by at most gamma_127 * sum|p_i| ~= 7.6e-6 * sum|p_i|
  (Higham, Accuracy and Stability of Numerical Algorithms, sec. 4.2), the
  oracle's single rounding adds at most 2^-24 * |S| <= 6e-8 * A, and a max of
  perturbed values moves by at most the largest perturbation. Empty columns
  are -inf on both sides.
* Top16 select on a given plane: bit-exact (ids and raw score bits).
* End-to-end ids (GPU plane -> GPU select/merge vs oracle plane -> oracle
  select/merge): equal, except in rows where the GPU's own rounding can
  change the choice. With tol(i) = 1e-5 * A(t, h, i) for block i, a GPU row
  is accepted only if it is the exact selection of some plane whose every
  value lies within tol of the oracle's: the lists are as long, every
  forced id is kept, every kept id is a valid block, and
      max over dropped non-forced valid x of (S(x) - tol(x))
          <= min over kept non-forced y of (S(y) + tol(y)).
  The condition is necessary (otherwise some dropped block beats some kept
  one under every admissible perturbation) and sufficient (raise the kept,
  lower the dropped). It uses each block's own A, not the row's largest.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-5


def compare_plane(gpu: np.ndarray, ref: np.ndarray, amax: np.ndarray, written: np.ndarray):
    """Returns (n_bad, worst_ratio) over the written elements."""
    g = gpu[written].astype(np.float64)
    r = ref[written].astype(np.float64)
    a = amax[written]
    ninf_g, ninf_r = np.isneginf(g), np.isneginf(r)
    bad_inf = int(np.count_nonzero(ninf_g != ninf_r))
    fin = ~ninf_g & ~ninf_r
    err = np.abs(g[fin] - r[fin])
    tol = REL_TOL * a[fin]
    over = err > tol
    ratio = float(np.max(err / np.maximum(tol, 1e-30))) if err.size else 0.0
    return bad_inf + int(np.count_nonzero(over)) + int(np.count_nonzero(np.isnan(g))), ratio


def written_mask(seq_lens: np.ndarray, dql: int, cols: int) -> np.ndarray:
    """[T, 4, cols] bool: columns below roundup4(ceil(seq/128)) per request."""
    B = len(seq_lens)
    m = np.zeros((B * dql, 4, cols), dtype=bool)
    for b, s in enumerate(seq_lens):
        s = int(s)
        if s <= 0:
            continue
        nblk = -(-s // 128)
        w = min(-(-nblk // 4) * 4, cols)
        m[b * dql:(b + 1) * dql, :, :w] = True
    return m


def forced_set(n: int, init: int, local: int):
    return set(range(min(init, n))) | set(range(max(0, n - local), n))


def compare_e2e_rows(gpu_ids, oracle_ids, oracle_plane, amax, nvp, init, local):
    """Checks final rows [T, 4, 16]; returns (n_exact, n_near_tie, failures list)."""
    T = gpu_ids.shape[0]
    n_exact = n_tie = 0
    failures = []
    for t in range(T):
        n = int(nvp[t])
        forced = forced_set(n, init, local)
        for h in range(4):
            g = [int(x) for x in gpu_ids[t, h] if x >= 0]
            o = [int(x) for x in oracle_ids[t, h] if x >= 0]
            if g == o:
                n_exact += 1
                continue
            srow = oracle_plane[t, h, :n].astype(np.float64)
            tol = REL_TOL * amax[t, h, :n].astype(np.float64)
            gset = set(g)
            kept = [i for i in g if i not in forced]
            dropped = [i for i in range(n) if i not in forced and i not in gset]
            ok = (len(g) == len(o) and forced <= gset and
                  all(0 <= i < n for i in g) and len(gset) == len(g))
            if ok and kept and dropped:
                worst_dropped = max(srow[x] - tol[x] for x in dropped)
                best_floor = min(srow[y] + tol[y] for y in kept)
                ok = worst_dropped <= best_floor
                margin = best_floor - worst_dropped
            else:
                margin = float("nan")
            band = margin
            if ok:
                n_tie += 1
            else:
                failures.append((t, h, f"inadmissible (margin {band:.3g})", g, o))
    return n_exact, n_tie, failures


def assert_rows_equal(gpu_scores, gpu_ids, ref_scores, ref_ids, what=""):
    """Bit-exact comparison of Top16 rows (ids and score bits)."""
    gi = np.asarray(gpu_ids)
    ri = np.asarray(ref_ids)
    bad = np.argwhere(gi != ri)
    assert bad.size == 0, f"{what}: {len(bad)} id mismatches, first at {bad[:3].tolist()}: " \
                          f"gpu {gi[tuple(bad[0][:-1])].tolist()} ref {ri[tuple(bad[0][:-1])].tolist()}"
    gs = np.ascontiguousarray(gpu_scores, dtype=np.float32).view(np.uint32)
    rs = np.ascontiguousarray(ref_scores, dtype=np.float32).view(np.uint32)
    bad = np.argwhere(gs != rs)
    assert bad.size == 0, f"{what}: {len(bad)} score-bit mismatches, first at {bad[:3].tolist()}"
