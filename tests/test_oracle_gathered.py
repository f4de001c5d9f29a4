"""Pins of the oracle's receiver side: payloads of several workers added in worker order.

* fp32 addition is not associative: three workers sending 1e8, 1 and -1e8 to one position
  sum to 0 in worker order (1e8 + 1 rounds back to 1e8), to 1 in another;
* against numpy: zeros, then per worker np.add.at in fp32 (indices unique within a payload);
* threshold payloads: the (+0, -1) padding carries nothing;
* int8 payloads: fl(code * scale) per worker's own scales; accumulate adds onto dense.
"""
import numpy as np

import oracle


def test_worker_order_is_the_summation_order(orc):
    seg_off = np.array([0, 4], np.int64)
    k = np.array([1], np.int64)
    idx = np.array([2, 2, 2], np.int32)
    vals = np.array([1e8, 1.0, -1e8], np.float32)
    d = orc.decompress_gathered(seg_off, k, 3, idx, vals=vals)
    assert d.tolist() == [0.0, 0.0, 0.0, 0.0]
    d = orc.decompress_gathered(seg_off, k, 3, idx, vals=vals[[0, 2, 1]].copy())
    assert d.tolist() == [0.0, 0.0, 1.0, 0.0]


def _payloads(orc, sizes, P, ratio, seed):
    seg_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(seg_off[-1])
    k = np.array([orc.k_from_ratio(s, ratio) for s in sizes], np.int64)
    rng = np.random.default_rng(seed)
    vals, idx = [], []
    for _ in range(P):
        g = rng.standard_t(3, n).astype(np.float32)
        v, i = orc.topk_ef(g, np.zeros(n, np.float32), seg_off, k)
        vals.append(v)
        idx.append(i)
    return seg_off, k, np.concatenate(vals), np.concatenate(idx)


def test_numpy_worker_by_worker(orc):
    sizes = [1000, 37, 5000, 1]
    P = 5
    seg_off, k, vals, idx = _payloads(orc, sizes, P, 0.1, 3)
    K = int(k.sum())
    want = np.zeros(int(seg_off[-1]), np.float32)
    seg_of_entry = np.repeat(np.arange(len(sizes)), k)
    for w in range(P):
        pos = seg_off[seg_of_entry] + idx[w * K:(w + 1) * K]
        np.add.at(want, pos, vals[w * K:(w + 1) * K])
    got = orc.decompress_gathered(seg_off, k, P, idx, vals=vals)
    assert got.tobytes() == want.tobytes()
    base = np.random.default_rng(4).standard_normal(int(seg_off[-1])).astype(np.float32)
    got = orc.decompress_gathered(seg_off, k, P, idx, vals=vals, dense=base.copy(),
                                  accumulate=True)
    want2 = base.copy()
    for w in range(P):
        np.add.at(want2, seg_off[seg_of_entry] + idx[w * K:(w + 1) * K], vals[w * K:(w + 1) * K])
    assert got.tobytes() == want2.tobytes()


def test_padding_carries_nothing(orc):
    seg_off = np.array([0, 6, 10], np.int64)
    k = np.array([3, 2], np.int64)
    idx = np.array([1, 4, -1, 0, -1,     2, -1, -1, 3, 1], np.int32)
    vals = np.array([1, 2, 0, 3, 0,      4, 0, 0, 5, 6], np.float32)
    d = orc.decompress_gathered(seg_off, k, 2, idx, vals=vals)
    assert d.tolist() == [0, 1, 4, 0, 2, 0, 3, 6, 0, 5]


def test_int8_payloads(orc):
    seg_off = np.array([0, 3, 5], np.int64)
    k = np.array([2, 1], np.int64)
    idx = np.array([0, 2, 1, 0, 1, 1], np.int32)
    codes = np.array([2, -3, 127, 1, 1, -1], np.int8)
    scales = np.array([0.5, 0.25, 2.0, 4.0], np.float32)
    d = orc.decompress_gathered(seg_off, k, 2, idx, codes=codes, scales=scales)
    # worker 0: 1.0 @0, -1.5 @2, 31.75 @4; worker 1: 2.0 @0, 2.0 @1, -4.0 @4
    assert d.tolist() == [3.0, 2.0, -1.5, 0.0, 27.75]
