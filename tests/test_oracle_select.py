"""Pins of the oracle's Top-k selection against things other than itself.

* brute-force enumeration of every k-subset on tiny vectors (a different algorithm:
  the selected set is the lexicographically smallest index set whose smallest |acc| is
  not below the largest dropped |acc|), with plain Python float comparisons of |acc|;
* numpy's lexsort of (|acc| desc, index asc) on larger vectors (a library routine);
* hand-worked cases derived from the two Top-K / error-feedback equations
  ("Communication Optimization > Gradient Compression", Top-K section);
* special cases: k = 0, k = n, all-equal, +-0, infinities, denormals.
"""
import itertools
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_topk(acc, k):
    """Smallest-index k-subset among those that keep k entries of largest |acc|."""
    n = len(acc)
    mags = [abs(float(a)) for a in acc]
    best = None
    for subset in itertools.combinations(range(n), k):     # lexicographic order
        chosen = set(subset)
        kept_min = min((mags[i] for i in subset), default=float("inf"))
        dropped_max = max((mags[i] for i in range(n) if i not in chosen), default=-1.0)
        if kept_min >= dropped_max:
            best = subset
            break
    assert best is not None
    return list(best)


def run_oracle(orc, g, e, k):
    g = np.asarray(g, np.float32).copy()
    e = np.asarray(e, np.float32).copy()
    vals, idx = orc.topk_ef_segment(g, e, k)
    return vals, idx, e


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    # integer-valued data so ties straddle the threshold often; signs mixed
    g = rng.integers(-3, 4, n).astype(np.float32)
    e = (rng.integers(-2, 3, n) * 0.5).astype(np.float32)
    if seed % 3 == 0:
        g[rng.integers(0, n)] = -0.0
    acc = (g.astype(np.float64) + e.astype(np.float64)).astype(np.float32)
    for k in range(n + 1):
        vals, idx, e_out = run_oracle(orc, g, e, k)
        want = brute_force_topk(acc, k)
        assert idx.tolist() == want
        assert vals.tobytes() == acc[want].tobytes()
        expect_e = acc.copy()
        expect_e[want] = 0.0
        assert e_out.tobytes() == expect_e.tobytes()


@pytest.mark.parametrize("seed,n,k", [(0, 1000, 1), (1, 5000, 37), (2, 100000, 100),
                                      (3, 4096, 4096), (4, 777, 0), (5, 20000, 19999)])
def test_numpy_lexsort(orc, seed, n, k):
    rng = np.random.default_rng(seed)
    g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    acc = np.add(g, e, dtype=np.float32)           # numpy's IEEE fp32 add
    order = np.lexsort((np.arange(n), -np.abs(acc.astype(np.float64))))
    want = np.sort(order[:k])
    vals, idx, e_out = run_oracle(orc, g, e, k)
    assert np.array_equal(idx, want)
    assert vals.tobytes() == acc[want].tobytes()
    expect_e = acc.copy()
    expect_e[want] = 0.0
    assert e_out.tobytes() == expect_e.tobytes()


def test_hand_examples(orc):
    with open(os.path.join(GOLD, "hand_examples.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        vals, idx, e_out = run_oracle(orc, case["g"], case["e"], case["k"])
        assert vals.tolist() == case["vals"], case["name"]
        assert idx.tolist() == case["idx"], case["name"]
        assert e_out.tolist() == case["e_out"], case["name"]
        # the residual's sign of zero: x - x = +0 under round-to-nearest
        assert not np.any(np.signbit(e_out[idx])), case["name"]
    mc = gold["momentum_case"]
    g = np.asarray(mc["g"], np.float32)
    e = np.asarray(mc["e"], np.float32)
    for mask in (False, True):
        u = np.asarray(mc["u"], np.float32).copy()
        ee = e.copy()
        vals, idx = orc.topk_ef_segment(g, ee, mc["k"], u=u, momentum=mc["m"], mask_u=mask)
        assert vals.tolist() == mc["vals"] and idx.tolist() == mc["idx"]
        assert ee.tolist() == mc["e_out"]
        want_u = list(mc["u_out"])
        if mask:
            for i in mc["idx"]:
                want_u[i] = 0.0
        assert u.tolist() == want_u


def test_all_equal_segment(orc):
    n = 1000
    for v in (0.0, -0.0, 1.5, -1.5):
        g = np.full(n, v, np.float32)
        e = np.zeros(n, np.float32)
        vals, idx, e_out = run_oracle(orc, g, e, 37)
        assert idx.tolist() == list(range(37))
        assert np.all(e_out[37:] == np.float32(v))


def test_signed_zero_and_inf_order(orc):
    # -0 and +0 tie; +-inf are the largest magnitudes; denormals order by magnitude
    den = np.float32(1e-44)
    g = np.array([-0.0, 0.0, den, -2 * den, np.inf, -np.inf, 1.0, -0.0], np.float32)
    e = np.zeros_like(g)
    vals, idx, _ = run_oracle(orc, g, e, 5)
    assert idx.tolist() == [2, 3, 4, 5, 6]
    vals, idx, _ = run_oracle(orc, g, e, 6)     # one of the zeros: the lowest index
    assert idx.tolist() == [0, 2, 3, 4, 5, 6]
    # denormal arithmetic is kept (no flush to zero): 1e-44 + 1e-44
    g = np.array([den], np.float32)
    e = np.array([den], np.float32)
    vals, idx, _ = run_oracle(orc, g, e, 1)
    assert vals[0] == np.float32(2 * den) and vals[0] != 0


def test_multi_segment_matches_per_segment(orc):
    rng = np.random.default_rng(7)
    sizes = [5, 64, 1, 0, 300, 17]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ks = np.array([orc.k_from_ratio(n, 0.1) for n in sizes], np.int64)
    g = rng.standard_normal(off[-1]).astype(np.float32)
    e = rng.standard_normal(off[-1]).astype(np.float32)
    e1 = e.copy()
    vals, idx = orc.topk_ef(g, e1, off, ks)
    pos = 0
    for s, n in enumerate(sizes):
        ee = e[off[s]:off[s + 1]].copy()
        v, i = orc.topk_ef_segment(g[off[s]:off[s + 1]].copy(), ee, int(ks[s]))
        assert np.array_equal(vals[pos:pos + ks[s]], v) and np.array_equal(idx[pos:pos + ks[s]], i)
        assert ee.tobytes() == e1[off[s]:off[s + 1]].tobytes()
        pos += ks[s]


def test_rejects_bad_k(orc):
    g = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        orc.topk_ef_segment(g, g.copy(), 5)
