"""Pins of the oracle's int8 stage, its Philox stream and decompression.

* Philox4x32-10 against the published known-answer vectors (tests/golden);
* chi-square uniformity of the 24-bit draws (scipy);
* unbiased stochastic rounding: the pages' toy example (0.3 between levels 0 and 1 is
  sent as 1 with probability 0.3) and the mean error over 10^6 draws within 3 sigma;
* closed forms: scale = absmax / 127 rounded once, the absmax entry codes to +-127,
  codes lie in {floor(a), ceil(a)}, integer a rounds deterministically, |code| <= 127;
* error feedback of the quantisation error: e = acc - code*scale exactly;
* decompression reconstructs acc = residual + dense(sent).
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers(orc):
    with open(os.path.join(GOLD, "philox4x32_10_kat.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        out = orc.philox4x32_10(w[0:4], w[4:6])
        assert out.tolist() == w[6:10]


def _codes_for(orc, vals, seed=0, step=0, seg_base=0):
    vals = np.asarray(vals, np.float32)
    idx = np.arange(vals.size, dtype=np.int32)
    return orc.quant_int8_segment(vals, idx, seg_base, None, seed, step)


def test_draws_uniform(orc):
    # the code of a value with frac = j/64 rounds up iff u24 < j * 2^18: the round-up rate
    # at each level recovers the draw's distribution function at that level
    j = np.tile(np.arange(64), 4096)
    vals = np.concatenate([[np.float32(127.0)], (j / 64.0).astype(np.float32)])
    codes, scale = _codes_for(orc, vals, seed=1234, step=3)
    assert scale == np.float32(1.0)
    up = codes[1:].astype(np.int64)
    # P(up | j) = j/64 exactly (frac * 2^24 is a multiple of 2^18); check per level
    for jj in (1, 16, 32, 63):
        p = up[j == jj].mean()
        sd = np.sqrt((jj / 64) * (1 - jj / 64) / 4096)
        assert abs(p - jj / 64) < 4 * sd
    # chi-square over the 64 cells of P(u24 in [j, j+1) * 2^18) from differences of levels
    draws = []
    for seed in range(2):
        for step in range(8):
            ctrs = np.arange(20000, dtype=np.uint64)
            w = np.array([orc.philox4x32_10([c & 0xFFFFFFFF, c >> 32, step, 0x51],
                                            [seed, 0])[0] for c in ctrs[:2000]], np.uint64)
            draws.append(w >> np.uint64(8))
    d = np.concatenate(draws)
    hist = np.bincount((d >> np.uint64(18)).astype(np.int64), minlength=64)
    chi = stats.chisquare(hist)
    assert chi.pvalue > 1e-4


def test_sr_toy_from_pages(orc):
    with open(os.path.join(GOLD, "pages_figures.json")) as f:
        toy = json.load(f)["stochastic_rounding_toy"]
    x = np.float32(toy["value"])
    n = 1_000_000
    # scale = absmax / 127 = 1 exactly, so a = 0.3f: levels 0 and 1 as in the toy example
    vals = np.full(n + 1, x, np.float32)
    vals[0] = np.float32(127.0)
    codes, scale = _codes_for(orc, vals, seed=0, step=0)
    assert scale == np.float32(1.0)
    c = codes[1:].astype(np.float64)
    assert set(np.unique(c)) <= set(toy["levels"])
    p = c.mean()
    sigma = np.sqrt(toy["p_up"] * (1 - toy["p_up"]) / n)
    assert abs(p - float(x)) < 3 * sigma                  # mean error within 3 sigma
    assert abs(p - toy["p_up"]) < 3 * sigma + 1e-7


def test_sr_unbiased_mean_error(orc):
    rng = np.random.default_rng(5)
    n = 1_000_000
    vals = (rng.standard_t(3, n) * 1e-2).astype(np.float32)
    codes, scale = _codes_for(orc, vals, seed=99, step=7, seg_base=12345)
    deq = codes.astype(np.float64) * np.float64(scale)
    err = deq - vals.astype(np.float64)
    sigma = np.sqrt(np.sum(err ** 2)) / n                 # std of the mean (per-draw var <= 1/4 step^2)
    assert abs(err.mean()) < 3 * sigma


def test_int8_closed_forms(orc):
    rng = np.random.default_rng(6)
    vals = (rng.standard_normal(50000) * 3e-3).astype(np.float32)
    vals[17] = np.float32(-0.25)                          # the absmax entry
    codes, scale = _codes_for(orc, vals, seed=3, step=1)
    absmax = np.abs(vals).max()
    assert absmax == np.float32(0.25)
    assert scale == np.float32(np.float64(absmax) / 127.0)   # one rounding of the quotient
    assert codes[17] == -127
    a = np.minimum(np.divide(np.abs(vals), scale, dtype=np.float32), np.float32(127))
    q = np.abs(codes.astype(np.int32))
    assert np.all((q == np.floor(a)) | (q == np.ceil(a)))
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    assert np.all(np.sign(codes[codes != 0]) == np.sign(vals[codes != 0]))
    # integer a never moves
    ints = np.array([127.0, 3.0, -5.0, 0.0, 126.0, -1.0], np.float32)
    for s in range(5):
        c, sc = _codes_for(orc, ints, seed=s, step=s)
        assert sc == np.float32(1.0) and c.tolist() == [127, 3, -5, 0, 126, -1]


def test_int8_zero_segment_and_error_feedback(orc):
    vals = np.zeros(5, np.float32)
    codes, scale = _codes_for(orc, vals)
    assert scale == 0 and not codes.any()
    rng = np.random.default_rng(8)
    vals = (rng.standard_normal(1000)).astype(np.float32)
    idx = np.sort(rng.choice(100000, 1000, replace=False)).astype(np.int32)
    e_seg = np.full(100000, np.float32(7.0))
    codes, scale = orc.quant_int8_segment(vals, idx, 5_000_000, e_seg, seed=1, step=2)
    deq = np.multiply(codes.astype(np.float32), scale, dtype=np.float32)
    assert e_seg[idx].tobytes() == np.subtract(vals, deq, dtype=np.float32).tobytes()
    keep = np.ones(100000, bool)
    keep[idx] = False
    assert np.all(e_seg[keep] == 7.0)


def test_counter_layout_is_global_index(orc):
    # the draw depends on (seed, step, global index) only: splitting a segment's base
    # and local index differently gives the same codes
    vals = np.linspace(-1, 1, 999).astype(np.float32)
    idx = np.arange(999, dtype=np.int32)
    c1, _ = orc.quant_int8_segment(vals, idx, 1000, None, 5, 9)
    c2, _ = orc.quant_int8_segment(vals, idx + 10, 990, None, 5, 9)
    assert np.array_equal(c1, c2)
    c3, _ = orc.quant_int8_segment(vals, idx, 1000, None, 5, 10)
    assert not np.array_equal(c1, c3)


@pytest.mark.parametrize("accumulate", [False, True])
def test_decompress_reconstructs(orc, accumulate):
    rng = np.random.default_rng(9)
    sizes = [1000, 3, 5000]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ks = np.array([orc.k_from_ratio(n, 0.05) for n in sizes], np.int64)
    g = rng.standard_normal(off[-1]).astype(np.float32)
    e = np.zeros(off[-1], np.float32)
    acc = g.copy()
    vals, idx = orc.topk_ef(g, e, off, ks)
    base = np.full(off[-1], np.float32(0.5)) if accumulate else None
    dense = orc.decompress(off, ks, idx, vals=vals,
                           dense=None if base is None else base.copy(), accumulate=accumulate)
    sent = np.zeros(off[-1], np.float32)
    pos = 0
    for s in range(len(sizes)):
        sent[off[s] + idx[pos:pos + ks[s]]] = vals[pos:pos + ks[s]]
        pos += ks[s]
    assert np.add(e, sent, dtype=np.float32).tobytes() == acc.tobytes()
    want = np.add(base, sent, dtype=np.float32) if accumulate else sent
    assert dense.tobytes() == want.tobytes()
    codes, scales = orc.quant_int8(vals, idx, off, ks)
    dq = orc.decompress(off, ks, idx, codes=codes, scales=scales)
    pos = 0
    for s in range(len(sizes)):
        sel = slice(pos, pos + ks[s])
        want = np.multiply(codes[sel].astype(np.float32), scales[s], dtype=np.float32)
        assert dq[off[s] + idx[sel]].tobytes() == want.tobytes()
        pos += ks[s]
