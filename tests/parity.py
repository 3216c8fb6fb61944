"""Comparison rules between the GPU path and the oracle.

Selection (block_idx): bit-exact wherever the oracle's (k-1)-th and k-th best
non-local block scores differ by more than 1e-3 relative.  Closer than that,
several selections are correct: the GPU set must hold the local block, every
block clearly above the boundary, and only blocks within tolerance of it; its
attention is then compared with the oracle's attention on the GPU's own set.

Attention (o, lse): o max-abs <= 2e-2 and mean-abs <= 1e-3, lse max-abs <= 1e-3.
"""
from __future__ import annotations

import numpy as np

REL_GAP = 1e-3
O_MAX_ABS = 2e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def check_block_idx(gpu_bi: np.ndarray, M: np.ndarray, rows, k: int, B_k: int):
    """gpu_bi [n, H_kv, k] int; M [n, H_kv, B] oracle scores (float64); rows = query positions.

    Returns a boolean mask [n, H_kv] of rows whose selection may legally differ from
    the oracle's (near ties).  Raises AssertionError on any violation.
    """
    gpu_bi = np.asarray(gpu_bi)
    n, H_kv, kk = gpu_bi.shape
    assert kk == k
    rows = np.asarray(rows)
    tie = np.zeros((n, H_kv), dtype=bool)
    for a in range(n):
        i = int(rows[a])
        bl = i // B_k
        for r in range(H_kv):
            g = gpu_bi[a, r]
            valid = g[g >= 0]
            where = f"row {i} group {r}: gpu {g.tolist()}"
            assert np.all(g[len(valid):] == -1), "padding must follow the chosen blocks: " + where
            assert np.all(np.diff(valid) > 0), "chosen blocks must be ascending and distinct: " + where
            assert bl in valid, "local block missing: " + where
            if bl + 1 <= k:
                assert valid.tolist() == list(range(bl + 1)), "all causal blocks expected: " + where
                continue
            assert len(valid) == k, "k blocks expected: " + where
            m = M[a, r, :bl]
            order = np.lexsort((np.arange(bl), -m))  # score desc, index asc
            t, t2 = m[order[k - 2]], m[order[k - 1]]
            tol = REL_GAP * max(abs(t), abs(t2))
            expect = np.sort(np.append(order[:k - 1], bl))
            if t - t2 > tol:
                assert valid.tolist() == expect.tolist(), f"selection differs (gap {t - t2:.3g}): {where}, " \
                                                          f"oracle {expect.tolist()}"
            else:
                tie[a, r] = True
                others = valid[valid != bl]
                assert np.all(m[others] >= t2 - tol), "chose a block clearly below the boundary: " + where
                must = np.nonzero(m > t + tol)[0]
                assert set(must.tolist()) <= set(others.tolist()), "missed a clearly better block: " + where
    return tie


def check_exact_twin_ties(gpu_bi: np.ndarray, M: np.ndarray, rows, k: int, B_k: int) -> int:
    """Rows whose selection boundary is an exact tie between two blocks with equal
    scores (duplicated index keys), with every other block clearly (> 1e-3 relative)
    above or below the tied value: the only freedom left is which of the two tied
    blocks takes the last slot, and the lower block index must win.  On such rows the
    GPU set must equal the oracle's bit for bit.  Returns the number of rows checked.

    The caller makes the tied blocks exact copies, so the GPU's fp32 scores of the
    two are equal too (same bf16 products in the same order); it checks that on the
    GPU's own block scores where an entry point exposes them."""
    gpu_bi = np.asarray(gpu_bi)
    n, H_kv, _ = gpu_bi.shape
    rows = np.asarray(rows)
    checked = 0
    for a in range(n):
        bl = int(rows[a]) // B_k
        if bl + 1 <= k:
            continue
        for r in range(H_kv):
            m = M[a, r, :bl]
            order = np.lexsort((np.arange(bl), -m))
            t, t2 = m[order[k - 2]], m[order[k - 1]]
            if t != t2:
                continue
            tol = REL_GAP * max(abs(t), 1e-30)
            above_ok = k < 3 or m[order[k - 3]] - t > tol
            below_ok = bl <= k or t - m[order[k]] > tol
            if not (above_ok and below_ok):
                continue
            expect = np.sort(np.append(order[:k - 1], bl))
            assert order[k - 2] < order[k - 1]
            g = gpu_bi[a, r]
            assert g.tolist() == expect.tolist(), \
                f"row {int(rows[a])} group {r}: exact tie between blocks {order[k - 2]} and {order[k - 1]} " \
                f"must go to the lower one; gpu {g.tolist()}, oracle {expect.tolist()}"
            checked += 1
    return checked


def check_attn(o, lse, o_ref, lse_ref, what: str = ""):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape
    inf_ref = np.isinf(lse_ref)
    assert np.array_equal(np.isinf(lse), inf_ref), f"{what}: empty rows differ"
    if inf_ref.any():
        assert np.all(o[inf_ref] == 0), f"{what}: empty rows must have o = 0"
    d = np.abs(o - o_ref)
    dl = np.abs(lse[~inf_ref] - lse_ref[~inf_ref])
    stats = dict(o_max=float(d.max()) if d.size else 0.0, o_mean=float(d.mean()) if d.size else 0.0,
                 lse_max=float(dl.max()) if dl.size else 0.0)
    assert stats["o_max"] <= O_MAX_ABS, f"{what}: o max-abs {stats}"
    assert stats["o_mean"] <= O_MEAN_ABS, f"{what}: o mean-abs {stats}"
    assert stats["lse_max"] <= LSE_MAX_ABS, f"{what}: lse max-abs {stats}"
    return stats
