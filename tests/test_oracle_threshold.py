"""Pins of the oracle's threshold sparsification with error feedback.

* brute force on tiny vectors: the sent set is every index with |acc| >= tau when at most
  k_cap reach it, else the k_cap largest (lower index first among equal magnitudes);
* numpy: mask |acc| >= tau, then lexsort among the masked;
* special cases: tau = 0 (Top-k of everything), tau above every magnitude (nothing sent,
  e = acc), an entry exactly at tau is sent, cap 0.
"""
import numpy as np
import pytest

from tests.test_oracle_select import brute_force_topk


@pytest.mark.parametrize("seed", range(8))
def test_brute_force(orc, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    g = rng.integers(-3, 4, n).astype(np.float32)
    e = (rng.integers(-2, 3, n) * 0.5).astype(np.float32)
    acc = (g.astype(np.float64) + e.astype(np.float64)).astype(np.float32)
    for tau in (0.0, 0.5, 1.0, 2.5, 9.0):
        for k_cap in range(n + 1):
            ee = e.copy()
            vals, idx = orc.threshold_ef_segment(g.copy(), ee, k_cap, tau)
            reach = [i for i in range(n) if abs(float(acc[i])) >= tau]
            if len(reach) <= k_cap:
                want = reach
            else:
                want = brute_force_topk(acc, k_cap)
            assert idx.tolist() == want
            assert vals.tobytes() == acc[want].tobytes()
            exp = acc.copy()
            exp[want] = 0.0
            assert ee.tobytes() == exp.tobytes()


def test_numpy_mask_then_lexsort(orc):
    rng = np.random.default_rng(7)
    n = 50000
    g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    acc = np.add(g, e, dtype=np.float32)
    for tau, k_cap in ((5e-3, 1000), (5e-3, 100), (1.0, 50), (0.0, 77)):
        m = np.flatnonzero(np.abs(acc) >= np.float32(tau))
        if m.size > k_cap:
            order = np.lexsort((m, -np.abs(acc[m].astype(np.float64))))
            m = np.sort(m[order[:k_cap]])
        ee = e.copy()
        vals, idx = orc.threshold_ef_segment(g.copy(), ee, k_cap, tau)
        assert np.array_equal(idx, m)
        assert vals.tobytes() == acc[m].tobytes()


def test_edges(orc):
    g = np.array([0.5, -1.0, 0.25, 1.0], np.float32)
    e = np.zeros(4, np.float32)
    vals, idx = orc.threshold_ef_segment(g.copy(), e.copy(), 4, 1.0)
    assert idx.tolist() == [1, 3]                      # exactly at the threshold: sent
    ee = e.copy()
    vals, idx = orc.threshold_ef_segment(g.copy(), ee, 4, 2.0)
    assert idx.size == 0 and ee.tolist() == g.tolist()  # nothing reaches: e = acc
    vals, idx = orc.threshold_ef_segment(g.copy(), e.copy(), 0, 0.0)
    assert idx.size == 0
    vals, idx = orc.threshold_ef_segment(g.copy(), e.copy(), 2, -1.0)   # |tau| is used
    assert idx.tolist() == [1, 3]
