"""Pins of the oracle's error-feedback and momentum arithmetic.

* every fp32 result equals numpy's IEEE float32 operation, and equals the double result
  rounded once to fp32 (exact for +, x, / since 53 >= 2*24 + 2: Figueroa 1995);
* the split is exact: residual + scatter(sent) == acc bit for bit, one side zero;
* conservation over iterations (the algebra of e_t = (g_t + e_{t-1}) - g^_t from
  "Communication Optimization > Gradient Compression", Top-K section):
  sum_t g^_t + e_T == sum_t g_t within 1e-6 relative;
* momentum correction ("Gradient Sparsification" glossary, momentum sections):
  m = 0 reduces to plain EF bit for bit; u_t against its closed form sum m^(t-s) g_s.
"""
import numpy as np
import pytest


def _rng_grad(rng, n, scale=1e-3):
    return (rng.standard_t(3, n) * scale).astype(np.float32)


def test_ef_add_is_ieee_fp32(orc):
    rng = np.random.default_rng(11)
    n = 20000
    g = _rng_grad(rng, n)
    e = (rng.standard_normal(n) * np.exp(rng.uniform(-30, 5, n))).astype(np.float32)
    e[:50] = np.float32(1e-41) * rng.integers(-5, 5, 50)   # denormals
    ee = e.copy()
    orc.topk_ef_segment(g, ee, 0)                            # k = 0: e becomes acc
    want = np.add(e, g, dtype=np.float32)
    assert ee.tobytes() == want.tobytes()
    via_double = (e.astype(np.float64) + g.astype(np.float64)).astype(np.float32)
    assert ee.tobytes() == via_double.tobytes()


def test_momentum_is_two_roundings(orc):
    rng = np.random.default_rng(12)
    n = 20000
    g = _rng_grad(rng, n)
    u = _rng_grad(rng, n, 1e-2)
    e = _rng_grad(rng, n, 1e-3)
    m = np.float32(0.9)
    uu, ee = u.copy(), e.copy()
    orc.topk_ef_segment(g, ee, 0, u=uu, momentum=float(m))
    mu = np.multiply(m, u, dtype=np.float32)
    want_u = np.add(mu, g, dtype=np.float32)
    assert uu.tobytes() == want_u.tobytes()
    # a fused multiply-add would round once: check the data can tell the two apart
    fused = (m.astype(np.float64) * u.astype(np.float64) + g.astype(np.float64)).astype(np.float32)
    assert np.any(fused != want_u)
    assert ee.tobytes() == np.add(e, want_u, dtype=np.float32).tobytes()


@pytest.mark.parametrize("k", [0, 1, 57, 1000])
def test_split_is_exact(orc, k):
    rng = np.random.default_rng(k)
    n = 1000
    g = _rng_grad(rng, n)
    e = _rng_grad(rng, n, 1e-4)
    acc = np.add(e, g, dtype=np.float32)
    ee = e.copy()
    vals, idx = orc.topk_ef_segment(g, ee, k)
    assert vals.size == k and idx.size == k                 # nnz = k
    assert np.all(np.diff(idx) > 0)                         # ascending, distinct
    sent = np.zeros(n, np.float32)
    sent[idx] = vals
    assert np.all((sent == 0) | (ee == 0))                  # one side is zero everywhere
    assert np.add(ee, sent, dtype=np.float32).tobytes() == acc.tobytes()
    if 0 < k < n:                                           # kept magnitudes dominate
        kept = np.abs(vals).min()
        mask = np.ones(n, bool)
        mask[idx] = False
        assert kept >= np.abs(acc[mask]).max()


@pytest.mark.parametrize("ratio,T", [(0.001, 8), (0.01, 8), (0.1, 5)])
def test_ef_conservation(orc, ratio, T):
    rng = np.random.default_rng(int(ratio * 1e4) + T)
    sizes = [4096, 100, 30000, 1]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ks = np.array([orc.k_from_ratio(n, ratio) for n in sizes], np.int64)
    N = int(off[-1])
    e = np.zeros(N, np.float32)
    sum_g = np.zeros(N)
    sum_sent = np.zeros(N)
    out_off = np.concatenate([[0], np.cumsum(ks)])
    for t in range(T):
        g = _rng_grad(rng, N)
        sum_g += g
        vals, idx = orc.topk_ef(g, e, off, ks)
        for s in range(len(sizes)):
            sel = slice(out_off[s], out_off[s + 1])
            np.add.at(sum_sent, off[s] + idx[sel], vals[sel].astype(np.float64))
    for s in range(len(sizes)):
        a, b = off[s], off[s + 1]
        lhs = sum_sent[a:b] + e[a:b]
        ref = sum_g[a:b]
        assert np.linalg.norm(lhs - ref) <= 1e-6 * np.linalg.norm(ref)


def test_momentum_zero_is_plain_ef(orc):
    rng = np.random.default_rng(21)
    n = 5000
    e0 = _rng_grad(rng, n)
    u = np.zeros(n, np.float32)
    e1, e2 = e0.copy(), e0.copy()
    for t in range(4):
        g = _rng_grad(rng, n)
        g[g == 0] = np.float32(1e-9)              # keep -0 out: fl(0*u) + (-0) = +0
        v1, i1 = orc.topk_ef_segment(g, e1, 50)
        v2, i2 = orc.topk_ef_segment(g, e2, 50, u=u, momentum=0.0)
        assert np.array_equal(i1, i2) and v1.tobytes() == v2.tobytes()
        assert e1.tobytes() == e2.tobytes()


def test_momentum_closed_form_and_conservation(orc):
    rng = np.random.default_rng(22)
    n, T, m, k = 3000, 6, 0.9, 30
    u = np.zeros(n, np.float32)
    e = np.zeros(n, np.float32)
    gs, sum_u, sum_sent = [], np.zeros(n), np.zeros(n)
    for t in range(T):
        g = _rng_grad(rng, n)
        gs.append(g.astype(np.float64))
        vals, idx = orc.topk_ef_segment(g, e, k, u=u, momentum=m)
        sum_u += u
        np.add.at(sum_sent, idx, vals.astype(np.float64))
        closed = sum(np.float64(np.float32(m)) ** (t - s) * gs[s] for s in range(t + 1))
        assert np.max(np.abs(u - closed)) <= 1e-5 * np.max(np.abs(closed))
    assert np.linalg.norm(sum_sent + e - sum_u) <= 1e-6 * np.linalg.norm(sum_u)


def test_momentum_mask_zeroes_sent_velocity(orc):
    rng = np.random.default_rng(23)
    n = 2000
    g = _rng_grad(rng, n)
    u0 = _rng_grad(rng, n)
    e = np.zeros(n, np.float32)
    u_a, u_b = u0.copy(), u0.copy()
    va, ia = orc.topk_ef_segment(g, e.copy(), 40, u=u_a, momentum=0.9, mask_u=False)
    vb, ib = orc.topk_ef_segment(g, e.copy(), 40, u=u_b, momentum=0.9, mask_u=True)
    assert np.array_equal(ia, ib)
    assert np.all(u_b[ib] == 0) and not np.any(np.signbit(u_b[ib]))
    keep = np.ones(n, bool)
    keep[ib] = False
    assert u_a[keep].tobytes() == u_b[keep].tobytes()
