"""k from a ratio, and the pages' ratio arithmetic reproduced from the oracle's output.

k = min(n, ceil(n * ratio)): the workload with 2^20 elements at 0.1% keeps 1049 entries,
so the rounding is upward; ratios are taken in exact parts per billion.
"""
import json
import os

import numpy as np

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_k_from_ratio(orc):
    assert orc.k_from_ratio(1 << 20, 0.001) == 1049
    assert orc.k_from_ratio(6400, 0.01) == 64            # exact, although 0.01 is inexact in binary
    assert orc.k_from_ratio(1 << 24, 0.01) == 167773
    assert orc.k_from_ratio(4096, 0.001) == 5
    assert orc.k_from_ratio(131072000, 0.001) == 131072
    assert orc.k_from_ratio(64, 0.01) == 1
    assert orc.k_from_ratio(10, 0.0) == 0
    assert orc.k_from_ratio(10, 1.0) == 10
    assert orc.k_from_ratio(0, 0.5) == 0
    assert orc.k_from_ratio(10, 1.5) == -1
    assert orc.k_from_ratio(10, -0.1) == -1
    assert orc.k_from_ratio(10, float("nan")) == -1
    rng = np.random.default_rng(0)
    for _ in range(2000):
        n = int(rng.integers(1, 1 << 31))
        ppb = int(rng.integers(0, 10 ** 9 + 1))
        k = orc.k_from_ratio(n, ppb / 1e9)
        assert k == min(n, -(-n * ppb // 10 ** 9))       # Python big-int ceiling


def test_pages_ratio_figures(orc):
    with open(os.path.join(GOLD, "pages_figures.json")) as f:
        fig = json.load(f)
    n = 10 ** 6
    g = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    e = np.zeros(n, np.float32)
    a = fig["topk_ratio_at_0p1pct"]
    k = orc.k_from_ratio(n, a["density"])
    vals, idx = orc.topk_ef_segment(g, e, k)
    assert n / vals.size == a["compression_ratio"]
    b = fig["wire_ratio_with_int32_index_at_0p1pct"]
    wire = vals.nbytes + idx.nbytes
    assert wire / vals.size == b["bytes_per_entry"]
    assert n * b["dense_bytes_per_entry"] / wire == b["compression_ratio"]
    c = fig["int8_ratio"]
    codes, _ = orc.quant_int8_segment(vals, idx, 0)
    assert vals.nbytes / codes.nbytes == c["compression_ratio"]
