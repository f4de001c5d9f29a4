"""Pins of the oracle's 1-bit sign compression with error feedback.

* hand-worked cases from the 1-bit SGD formula Q(g) = sign(g)*||g||_1/d
  ("Communication Optimization > Gradient Compression", 1-bit SGD section);
* the scale against the exactly rounded sum (math.fsum) within 1 ulp;
* the bits against numpy's comparison and its bit packing (LSB first);
* the residual equals acc - sign*scale in IEEE fp32 (numpy);
* error feedback conserves the signal: sum of sent + final residual = sum of gradients;
* the pages' 32x ratio; decompression; momentum 0 reduces to plain.
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_cases(orc):
    with open(os.path.join(GOLD, "hand_examples.json")) as f:
        gold = json.load(f)
    for name in ("sign_case", "sign_zero_case"):
        c = gold[name]
        e = np.asarray(c["e"], np.float32)
        bits, scale = orc.sign_ef_segment(np.asarray(c["g"], np.float32), e)
        assert bits.tolist() == c["bits"], name
        assert scale == np.float32(c["scale"]), name
        assert e.tolist() == c["e_out"], name


@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000, 65536 + 7])
def test_scale_bits_residual(orc, n):
    rng = np.random.default_rng(n)
    g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    e0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = e0.copy()
    bits, scale = orc.sign_ef_segment(g, e)
    acc = np.add(e0, g, dtype=np.float32)
    exact = math.fsum(abs(float(a)) for a in acc) / n
    assert abs(float(scale) - exact) <= float(np.spacing(np.float32(exact)))
    neg = acc < 0
    want_bits = np.packbits(np.concatenate([neg, np.zeros((-n) % 32, bool)]),
                            bitorder="little").view("<u4")
    assert np.array_equal(bits, want_bits)
    q = np.where(neg, -scale, scale).astype(np.float32)
    assert e.tobytes() == np.subtract(acc, q, dtype=np.float32).tobytes()


def test_conservation_and_ratio(orc):
    with open(os.path.join(GOLD, "pages_figures.json")) as f:
        fig = json.load(f)["one_bit_ratio"]
    rng = np.random.default_rng(3)
    n, T = 10016, 8                       # a multiple of 32: no padding bits
    e = np.zeros(n, np.float32)
    sum_g = np.zeros(n)
    sum_sent = np.zeros(n)
    for _ in range(T):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        sum_g += g
        bits, scale = orc.sign_ef_segment(g, e)
        sum_sent += orc.sign_decompress_segment(bits, scale, n).astype(np.float64)
    assert (4 * n) / bits.nbytes == fig["compression_ratio"]
    assert np.linalg.norm(sum_sent + e - sum_g) <= 1e-6 * np.linalg.norm(sum_g)


def test_decompress_and_accumulate(orc):
    bits = np.array([0b1010], np.uint32)
    d = orc.sign_decompress_segment(bits, 1.5, 4)
    assert d.tolist() == [1.5, -1.5, 1.5, -1.5]
    base = np.array([1.0, 1.0, 0.25, 0.0], np.float32)
    d = orc.sign_decompress_segment(bits, 1.5, 4, dense=base.copy(), accumulate=True)
    assert d.tolist() == [2.5, -0.5, 1.75, -1.5]


def test_momentum_zero_is_plain(orc):
    rng = np.random.default_rng(4)
    n = 777
    g = (rng.standard_normal(n) + 0.1).astype(np.float32)
    e1 = (rng.standard_normal(n) * 0.1).astype(np.float32)
    e2 = e1.copy()
    b1, s1 = orc.sign_ef_segment(g, e1)
    b2, s2 = orc.sign_ef_segment(g, e2, u=np.zeros(n, np.float32), momentum=0.0)
    assert np.array_equal(b1, b2) and s1 == s2 and e1.tobytes() == e2.tobytes()


def test_empty_segment(orc):
    bits, scale = orc.sign_ef_segment(np.zeros(0, np.float32), np.zeros(0, np.float32))
    assert bits.size == 0 and scale == 0
