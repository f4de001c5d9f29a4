"""Pins of the oracle's local gradient clipping (l2 norm per segment brought down to c).

* the 3-4-5 triangle: norm 5, clipped to c = 1 gives (0.6, 0.8) within an ulp;
* the norm against numpy's float64 norm (one fp32 rounding: within one ulp);
* after clipping the norm is c within a few fp32 roundings and every element is scaled by
  the same factor (direction kept); below the bound the segment is untouched bit for bit;
* c = 0 clears a non-zero segment.
"""
import numpy as np
import pytest


def test_three_four_five(orc):
    g = np.array([3.0, 4.0], np.float32)
    assert orc.clip_by_norm_segment(g, 1.0) == np.float32(5.0)
    assert abs(float(g[0]) - 0.6) <= float(np.spacing(np.float32(0.6)))
    assert abs(float(g[1]) - 0.8) <= float(np.spacing(np.float32(0.8)))


@pytest.mark.parametrize("seed", range(4))
def test_norm_direction_and_bound(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 200000))
    g = (rng.standard_t(3, n) * 10 ** rng.uniform(-4, 2)).astype(np.float32)
    want = np.linalg.norm(g.astype(np.float64))
    for c in (want * 0.3, want * 2.0):
        h = g.copy()
        norm = orc.clip_by_norm_segment(h, c)
        assert abs(float(norm) - want) <= float(np.spacing(np.float32(want)))
        if c > want:
            assert h.tobytes() == g.tobytes()
        else:
            got = np.linalg.norm(h.astype(np.float64))
            assert abs(got - c) <= 4 * 2.0 ** -24 * c
            ratio = h[g != 0].astype(np.float64) / g[g != 0]
            f = np.float32(np.float32(c) / norm)
            assert np.all(np.abs(ratio - float(f)) <= 2.0 ** -23 * float(f))


def test_zero_bound_and_equal_norm(orc):
    g = np.array([1.0, -2.0, 2.0], np.float32)        # norm exactly 3
    h = g.copy()
    orc.clip_by_norm_segment(h, 3.0)
    assert h.tobytes() == g.tobytes()
    h = g.copy()
    orc.clip_by_norm_segment(h, 0.0)
    assert np.all(h == 0)
