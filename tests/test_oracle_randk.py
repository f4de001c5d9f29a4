"""Pins of the oracle's Random-k (a uniformly random k-subset per step, by the k largest
Philox keys; error feedback, or values scaled by n/k without it).

* exactly k distinct positions, ascending, values acc at those positions; with error
  feedback sent + residual == acc bit for bit (conservation);
* uniformity: each position is kept with frequency k/n, each pair with k(k-1)/(n(n-1)),
  each of the C(5,2) subsets with frequency 1/10 (chi-square), over many steps;
* unbiasedness without error feedback: the mean of the scaled sparse vector over steps is
  acc, within the estimator's own standard deviation; the scale is fl32(n/k);
* the mask does not depend on the values, changes with the step and with the segment;
* the counter mapping (a definition, not a fact): keys recomputed from the Philox
  known-answer-pinned generator and sorted by (key desc, position asc) give the same mask.
"""
import itertools
import math

import numpy as np
import pytest


def _acc(g, e):
    return np.add(e, g, dtype=np.float32)


@pytest.mark.parametrize("n,k", [(1, 0), (1, 1), (7, 3), (100, 1), (1000, 37), (4096, 4096)])
def test_exact_k_and_conservation(orc, n, k):
    rng = np.random.default_rng(n * 31 + k)
    g = rng.standard_normal(n).astype(np.float32)
    e = (rng.standard_normal(n) * 0.1).astype(np.float32)
    acc = _acc(g, e)
    ee = e.copy()
    vals, idx = orc.randk_segment(g, k, e=ee, seed=5, step=2)
    assert idx.size == k
    assert np.all(np.diff(idx) > 0) and (k == 0 or (idx[0] >= 0 and idx[-1] < n))
    assert vals.tobytes() == acc[idx].tobytes()
    dense = ee.copy()
    assert np.all(dense[idx] == 0) and not np.any(np.signbit(dense[idx]))
    dense[idx] = vals
    assert dense.tobytes() == acc.tobytes()


def _masks(orc, n, k, steps, seed=11, seg_base=0):
    g = np.ones(n, np.float32)
    out = np.zeros((steps, n), bool)
    for t in range(steps):
        _, idx = orc.randk_segment(g, k, e=np.zeros(n, np.float32), seed=seed, step=t,
                                   seg_base=seg_base)
        out[t, idx] = True
    return out


def test_marginal_and_pairwise_uniform(orc):
    n, k, steps = 20, 5, 4000
    m = _masks(orc, n, k, steps)
    assert np.all(m.sum(1) == k)
    p = k / n
    sd = math.sqrt(steps * p * (1 - p))
    cnt = m.sum(0)
    assert np.all(np.abs(cnt - steps * p) < 6 * sd), cnt
    pp = k * (k - 1) / (n * (n - 1))
    sdp = math.sqrt(steps * pp * (1 - pp))
    both = m.astype(np.int64).T @ m.astype(np.int64)
    off = both[~np.eye(n, dtype=bool)]
    assert np.all(np.abs(off - steps * pp) < 6 * sdp), (off.min(), off.max())


def test_every_subset_equally_likely(orc):
    n, k, steps = 5, 2, 5000
    m = _masks(orc, n, k, steps, seed=3)
    subsets = {c: 0 for c in itertools.combinations(range(n), k)}
    for row in m:
        subsets[tuple(np.flatnonzero(row))] += 1
    exp = steps / len(subsets)
    chi2 = sum((c - exp) ** 2 / exp for c in subsets.values())
    assert chi2 < 40.0, subsets   # 9 degrees of freedom: P(chi2 > 40) ~ 7e-6


def test_unbiased_without_error_feedback(orc):
    n, k, steps = 16, 4, 20000
    rng = np.random.default_rng(9)
    g = rng.standard_normal(n).astype(np.float32)
    mean = np.zeros(n)
    for t in range(steps):
        vals, idx = orc.randk_segment(g, k, seed=21, step=t)
        assert vals.tobytes() == (g[idx] * np.float32(4.0)).tobytes()
        mean[idx] += vals
    mean /= steps
    sd = np.abs(g) * math.sqrt((n / k - 1) / steps)
    assert np.all(np.abs(mean - g) < 6 * sd + 1e-12)
    vals, idx = orc.randk_segment(np.ones(10, np.float32), 3, seed=1, step=0)
    assert np.all(vals == np.float32(10 / 3))        # fl32 of n/k


def test_mask_depends_on_step_and_segment_not_values(orc):
    n, k = 1000, 10
    g1 = np.random.default_rng(0).standard_normal(n).astype(np.float32)
    g2 = np.random.default_rng(1).standard_normal(n).astype(np.float32) * 100
    _, i1 = orc.randk_segment(g1, k, e=np.zeros(n, np.float32), seed=4, step=7)
    _, i2 = orc.randk_segment(g2, k, e=np.zeros(n, np.float32), seed=4, step=7)
    assert np.array_equal(i1, i2)
    masks = [tuple(orc.randk_segment(g1, k, seed=4, step=t)[1]) for t in range(8)]
    assert len(set(masks)) == 8
    _, i3 = orc.randk_segment(g1, k, seed=4, step=7, seg_base=1000)
    _, i4 = orc.randk_segment(g1, k, seed=5, step=7)
    assert not np.array_equal(i1, i3) and not np.array_equal(i1, i4)


def test_momentum_and_mask(orc):
    n, k = 300, 17
    rng = np.random.default_rng(2)
    g = rng.standard_normal(n).astype(np.float32)
    e = rng.standard_normal(n).astype(np.float32)
    u = rng.standard_normal(n).astype(np.float32)
    m = np.float32(0.9)
    u_new = np.add(np.multiply(m, u, dtype=np.float32), g, dtype=np.float32)
    acc = np.add(e, u_new, dtype=np.float32)
    uu, ee = u.copy(), e.copy()
    vals, idx = orc.randk_segment(g, k, e=ee, u=uu, momentum=0.9, mask_u=True, seed=8, step=1)
    assert vals.tobytes() == acc[idx].tobytes()
    want_u = u_new.copy()
    want_u[idx] = 0
    assert uu.tobytes() == want_u.tobytes()


@pytest.mark.parametrize("seg_base", [0, 3, 1 << 33])
def test_counter_mapping(orc, seg_base):
    n, k, seed, step = 23, 6, 0x123456789ABC, 77
    keys = []
    for i in range(n):
        gi = seg_base + i
        ctr = [(gi >> 2) & 0xFFFFFFFF, (gi >> 34) & 0xFFFFFFFF, step & 0xFFFFFFFF, 0x53]
        w = orc.philox4x32_10(ctr, [seed & 0xFFFFFFFF, seed >> 32])
        keys.append(int(w[gi & 3]) >> 1)
    order = sorted(range(n), key=lambda i: (-keys[i], i))
    _, idx = orc.randk_segment(np.ones(n, np.float32), k, seed=seed, step=step,
                               seg_base=seg_base)
    assert idx.tolist() == sorted(order[:k])
