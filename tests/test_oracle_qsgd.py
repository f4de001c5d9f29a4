"""Pins of the oracle's QSGD codec ("Communication Optimization > Gradient Compression",
QSGD paragraph; the 1/s factor its formula lacks is restored so that E[Q] = g holds).

* hand cases with integer levels (no randomness involved);
* unbiasedness E[Q_s(v)] = v over many independent draws (the page's key property), and the
  toy example's 0.3 -> 1 with probability 0.3 at one level;
* the variance bound of Alistarh et al. (NeurIPS 2017, Lemma 3.1):
  E||Q_s(v) - v||^2 <= min(n/s^2, sqrt(n)/s) ||v||^2;
* the norm against the exactly rounded sqrt of the exact sum of squares (within 1 ulp);
* codes within {floor(a), ceil(a)}, |code| <= s, s = 1 ternary; error feedback exact and
  conserving; decompression.
"""
import math

import numpy as np
import pytest


def test_hand_integer_levels(orc):
    codes, norm = orc.qsgd_segment(np.array([3, -4, 0, -0.0], np.float32), levels=5)
    assert norm == 5.0 and codes.tolist() == [3, -4, 0, 0]
    codes, norm = orc.qsgd_segment(np.array([0.6, 0.8], np.float32), levels=1)
    # norm 1, step 1: a = 0.6 and 0.8, each rounds to 0 or 1
    assert norm == np.float32(1.0) and set(codes.tolist()) <= {0, 1}
    codes, norm = orc.qsgd_segment(np.zeros(5, np.float32), levels=7)
    assert norm == 0 and not codes.any()


def test_unbiased_and_toy(orc):
    v = np.array([0.3, -0.25, 0.9, 0.0, -0.05, 0.2], np.float32)
    n, s, D = v.size, 3, 20000
    norm = np.float32(math.sqrt(float(np.sum(v.astype(np.float64) ** 2))))
    step = np.float32(norm / np.float32(s))
    acc = np.zeros(n)
    acc2 = np.zeros(n)
    for d in range(D):
        codes, nn = orc.qsgd_segment(v, levels=s, seed=d // 100, step=d % 100)
        assert nn == norm
        q = orc.qsgd_decompress_segment(codes, nn, s).astype(np.float64)
        acc += q
        acc2 += q * q
    mean = acc / D
    sd = np.sqrt(np.maximum(acc2 / D - mean ** 2, 1e-30) / D)
    assert np.all(np.abs(mean - v) <= 4 * sd + 1e-7)
    # the page's toy example (0.3 between levels 0 and 1 is sent as 1 with probability 0.3):
    # 10000 entries of 0.3 plus one large entry chosen so that norm / s is about 1
    M, s2 = 10000, 100
    x = np.full(M + 1, np.float32(0.3), np.float32)
    x[0] = np.float32(math.sqrt(s2 * s2 - M * 0.09))
    codes, nn = orc.qsgd_segment(x, levels=s2, seed=5)
    a = float(np.float32(0.3) / np.float32(nn / np.float32(s2)))
    assert abs(a - 0.3) < 1e-5
    p = (codes[1:] == 1).mean()
    assert set(np.unique(codes[1:]).tolist()) <= {0, 1}
    assert abs(p - a) < 4 * math.sqrt(a * (1 - a) / M)


@pytest.mark.parametrize("s", [1, 3, 15, 127])
def test_variance_bound(orc, s):
    rng = np.random.default_rng(s)
    n = 512
    v = (rng.standard_t(3, n)).astype(np.float32)
    vv = float(np.sum(v.astype(np.float64) ** 2))
    D = 400
    err = 0.0
    for d in range(D):
        codes, nn = orc.qsgd_segment(v, levels=s, seed=1, step=d)
        q = orc.qsgd_decompress_segment(codes, nn, s).astype(np.float64)
        err += float(np.sum((q - v) ** 2))
    bound = min(n / s ** 2, math.sqrt(n) / s) * vv
    assert err / D <= bound * 1.05


def test_norm_codes_and_error_feedback(orc):
    rng = np.random.default_rng(9)
    n, s = 20000, 15
    g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    e0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = e0.copy()
    codes, norm = orc.qsgd_segment(g, e=e, levels=s, seed=3, step=4, seg_base=777)
    acc = np.add(e0, g, dtype=np.float32)
    exact = math.sqrt(math.fsum(float(a) * float(a) for a in acc))
    assert abs(float(norm) - exact) <= float(np.spacing(np.float32(exact)))
    step = np.float32(norm / np.float32(s))
    a = np.minimum(np.divide(np.abs(acc), step, dtype=np.float32), np.float32(s))
    q = np.abs(codes.astype(np.int32))
    assert np.all((q == np.floor(a)) | (q == np.ceil(a))) and q.max() <= s
    assert np.all(np.sign(codes[codes != 0]) == np.sign(acc[codes != 0]))
    deq = np.multiply(codes.astype(np.float32), step, dtype=np.float32)
    assert e.tobytes() == np.subtract(acc, deq, dtype=np.float32).tobytes()
    c1, _ = orc.qsgd_segment(np.float32([0.5, -0.25, 1.0]), levels=1, seed=1)
    assert set(c1.tolist()) <= {-1, 0, 1}


def test_conservation_and_decompress(orc):
    rng = np.random.default_rng(10)
    n, T, s = 4000, 6, 7
    e = np.zeros(n, np.float32)
    sum_g, sum_q = np.zeros(n), np.zeros(n)
    for t in range(T):
        g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        sum_g += g
        codes, norm = orc.qsgd_segment(g, e=e, levels=s, seed=2, step=t)
        sum_q += orc.qsgd_decompress_segment(codes, norm, s).astype(np.float64)
    assert np.linalg.norm(sum_q + e - sum_g) <= 1e-6 * np.linalg.norm(sum_g)
    base = np.ones(3, np.float32)
    d = orc.qsgd_decompress_segment(np.int8([2, -1, 0]), 4.0, 2, dense=base.copy(),
                                    accumulate=True)
    assert d.tolist() == [5.0, -1.0, 1.0]


def test_rejects_bad_levels(orc):
    with pytest.raises(ValueError):
        orc.qsgd_segment(np.zeros(3, np.float32), levels=128)
    with pytest.raises(ValueError):
        orc.qsgd_segment(np.zeros(3, np.float32), levels=0)
