"""GPU parity of the threshold and Random-k sparsifiers (C ABI) against the CPU oracle.

Ragged shapes (segment starts not on a multiple of 4, tails of every length), several EF
iterations, momentum with and without the mask, the exact fallback paths forced from the
host, and the full 7B shape in the bench's launch configuration: sampled segments bit for
bit against the oracle, every segment checked by properties that fix the result (threshold:
the kept set is every |acc| >= tau when at most k reach it, else the k largest; Random-k: k
ascending indices per segment, values and residual exact).
"""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from synth import gen, workload
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu


def _grads(n, iters, seed, scale=1.0, df=3.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_t(df, n) * scale).astype(np.float32) for _ in range(iters)]


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


# ------------------------------------------------------------------------- threshold
def run_threshold(sizes, k, grads, taus, momentum=None, mask=False, flags=0, label=""):
    off = _offsets(sizes)
    n = int(off[-1])
    ks = np.broadcast_to(np.asarray(k, np.int64), (len(sizes),)).copy()
    plan = gca.Plan(off, k=ks, flags=flags | (gca.GC_MOMENTUM_MASK if mask else 0))
    dev = torch.device("cuda")
    e_d = torch.zeros(n, device=dev)
    e_h = np.zeros(n, np.float32)
    u_d = torch.zeros(n, device=dev) if momentum is not None else None
    u_h = np.zeros(n, np.float32) if momentum is not None else None
    tk = max(plan.total_k, 1)
    vals = torch.empty(tk, device=dev)
    idx = torch.empty(tk, dtype=torch.int32, device=dev)
    cnt = torch.empty(len(sizes), dtype=torch.int32, device=dev)
    for t, g in enumerate(grads):
        tau = np.asarray(taus(t, g, e_h), np.float32)
        log(f"[threshold {label}] iteration {t}")
        vals.fill_(float("nan"))
        idx.fill_(-7)
        plan.threshold_compress(torch.from_numpy(g).to(dev), e_d, torch.from_numpy(tau).to(dev),
                                vals, idx, cnt, u=u_d, momentum=momentum or 0.0)
        torch.cuda.synchronize()
        v_d, i_d, c_d = vals.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
        for s in range(len(sizes)):
            a, b = int(off[s]), int(off[s + 1])
            ka, kb = int(plan.out_off[s]), int(plan.out_off[s + 1])
            hv, hi = oracle.threshold_ef_segment(
                g[a:b].copy(), e_h[a:b], int(ks[s]), float(tau[s]),
                u=None if u_h is None else u_h[a:b], momentum=momentum or 0.0, mask_u=mask)
            c = hi.size
            assert c_d[s] == c, f"{label} it{t} seg{s} count {c_d[s]} != {c}"
            assert_bitwise(i_d[ka:ka + c], hi, f"{label} it{t} seg{s} idx")
            assert_bitwise(v_d[ka:ka + c], hv, f"{label} it{t} seg{s} vals")
            assert np.all(i_d[ka + c:kb] == -1) and np.all(v_d[ka + c:kb] == 0), "padding"
        assert_bitwise(e_d, e_h, f"{label} it{t} residual")
        if u_h is not None:
            assert_bitwise(u_d, u_h, f"{label} it{t} velocity")
    return plan


def _taus_mixed(t, g, e):
    """Per-segment thresholds around the data: some segments keep fewer than k, some hit the
    cap, one keeps everything it can (tau 0), one nothing (tau above every value)."""
    return [0.5, 2.0 + t, 0.0, 1e30, 4.0, 1.5][:6]


SIZES = [1001, 70003, 8192 * 3 + 5, 300001, 4097, 129]


def test_threshold_ragged():
    run_threshold(SIZES, [50, 300, 40, 500, 4097, 3], _grads(sum(SIZES), 4, 1),
                  _taus_mixed, label="ragged")


def test_threshold_at_exact_value():
    """tau equal to an element's |acc|: that element reaches the threshold."""
    sizes = [5000, 9000]
    grads = _grads(sum(sizes), 2, 2)

    def taus(t, g, e):
        acc = np.add(e, g, dtype=np.float32)
        return [abs(acc[123]), -abs(acc[5000 + 77])]
    run_threshold(sizes, [5000, 9000], grads, taus, label="exact")


def test_threshold_momentum_mask():
    run_threshold(SIZES, [50, 300, 40, 500, 4097, 3], _grads(sum(SIZES), 3, 3),
                  _taus_mixed, momentum=0.9, mask=True, label="momentum-mask")


@pytest.mark.parametrize("flag", [gca.GC_DEBUG_FORCE_FALLBACK, gca.GC_DEBUG_NO_ESTIMATE],
                         ids=["forced-full", "no-estimate"])
def test_threshold_fallbacks(flag):
    plan = run_threshold(SIZES, [50, 300, 40, 500, 4097, 3], _grads(sum(SIZES), 2, 4),
                         _taus_mixed, flags=flag, label=f"flag{flag:#x}")
    st = plan.last_stats()
    if flag == gca.GC_DEBUG_FORCE_FALLBACK:
        assert all(m in (gca.MODE_SKIP, gca.MODE_FULL, gca.MODE_SMALL) for m in st["mode"]), \
            st["mode"]


def test_threshold_overflow_then_floor():
    """tau = 0 on a segment far larger than its candidate capacity: every element reaches
    the threshold, the first capture overflows and the k largest still come out exactly (the
    exact fallback); later calls capture above the floor estimated from the kept entries and
    stay on the candidate path."""
    sizes = [2_000_003, 300001]
    seen = []

    def taus(t, g, e):
        return [0.0, 3.0]
    plan = run_threshold(sizes, [1000, 300], _grads(sum(sizes), 1, 5), taus, label="overflow")
    seen.append(plan.last_stats()["mode"].tolist())
    assert seen[0][0] in (gca.MODE_FULL, gca.MODE_RECAPTURED)
    # continue on the same plan: the floor is per plan
    off = _offsets(sizes)
    n = int(off[-1])
    dev = torch.device("cuda")
    e_d = torch.zeros(n, device=dev)
    e_h = np.zeros(n, np.float32)
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    tau = torch.tensor([0.0, 3.0], device=dev)
    for t, g in enumerate(_grads(n, 6, 55)):
        plan.threshold_compress(torch.from_numpy(g).to(dev), e_d, tau, vals, idx)
        torch.cuda.synchronize()
        seen.append(plan.last_stats()["mode"].tolist())
        for s in range(2):
            a, b = int(off[s]), int(off[s + 1])
            ka = int(plan.out_off[s])
            hv, hi = oracle.threshold_ef_segment(g[a:b].copy(), e_h[a:b], int(plan.k[s]),
                                                 float(tau[s]))
            assert_bitwise(idx[ka:ka + hi.size], hi, f"floor it{t} seg{s} idx")
            assert_bitwise(vals[ka:ka + hi.size], hv, f"floor it{t} seg{s} vals")
        assert_bitwise(e_d, e_h, f"floor it{t} residual")
    log(f"[threshold floor] modes per call: {seen}")
    assert seen[-1] == [gca.MODE_CANDIDATES, gca.MODE_CANDIDATES], seen


def test_side_calls_keep_topk_estimate():
    """Threshold and Random-k calls leave the plan's Top-k threshold estimate alone: two plans
    with the same Top-k history, one of them also running both on side buffers, make the
    same next Top-k call (same path, same candidate count, same result)."""
    sizes = [300001, 70003]
    off = _offsets(sizes)
    n = int(off[-1])
    dev = torch.device("cuda")
    plans = [gca.Plan(off, ratio=0.001), gca.Plan(off, ratio=0.001)]
    g1, g2, g3 = (torch.from_numpy(x).to(dev) for x in _grads(n, 3, 6))
    es = [torch.zeros(n, device=dev), torch.zeros(n, device=dev)]
    tk = plans[0].total_k
    outs = [(torch.empty(tk, device=dev), torch.empty(tk, dtype=torch.int32, device=dev))
            for _ in plans]
    for p, e, (v, i) in zip(plans, es, outs):
        p.compress(g1, e, v, i)
    side_e = es[0].clone()
    v, i = outs[0]
    plans[0].threshold_compress(g2, side_e, torch.full((2,), 3.0, device=dev), v, i)
    plans[0].randk_compress(g2, v, i, e=side_e, seed=1, step=0)
    stats = []
    for p, e, (v, i) in zip(plans, es, outs):
        p.compress(g3, e, v, i)
        stats.append(p.last_stats())
    torch.cuda.synchronize()
    for key in ("mode", "candidates", "kth_key", "ties"):
        assert np.array_equal(stats[0][key], stats[1][key]), key
    assert_bitwise(outs[0][0], outs[1][0].cpu().numpy(), "vals")
    assert_bitwise(outs[0][1], outs[1][1].cpu().numpy(), "idx")
    assert_bitwise(es[0], es[1].cpu().numpy(), "residual")


def test_threshold_decompress_skips_padding():
    """P(|t_3| > 12) is about 0.12%: about 84 of 70003 reach tau = 12, below k = 200, so
    the segment's tail is padding, which decompression must skip."""
    sizes = [1001, 70003]
    ks = [100, 200]
    off = _offsets(sizes)
    plan = gca.Plan(off, k=ks)
    g = _grads(int(off[-1]), 1, 7)[0]
    e = torch.zeros(int(off[-1]), device="cuda")
    vals = torch.empty(300, device="cuda")
    idx = torch.empty(300, dtype=torch.int32, device="cuda")
    cnt = torch.empty(2, dtype=torch.int32, device="cuda")
    plan.threshold_compress(torch.from_numpy(g).cuda(), e, torch.tensor([2.5, 12.0]).cuda(),
                            vals, idx, cnt)
    dense = torch.full((int(off[-1]),), 7.0, device="cuda")
    plan.decompress(idx, dense, vals=vals)
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    assert 0 < c[1] < 200
    want = np.zeros(int(off[-1]), np.float32)
    v, i = vals.cpu().numpy(), idx.cpu().numpy()
    oo = plan.out_off
    for s in range(2):
        ka = int(oo[s])
        want[int(off[s]) + i[ka:ka + c[s]]] = v[ka:ka + c[s]]
    assert_bitwise(dense, want, "decompressed")


# -------------------------------------------------------------------------- Random-k
def run_randk(sizes, k, grads, ef=True, momentum=None, mask=False, flags=0, seed=5, label=""):
    off = _offsets(sizes)
    n = int(off[-1])
    ks = np.broadcast_to(np.asarray(k, np.int64), (len(sizes),)).copy()
    plan = gca.Plan(off, k=ks, flags=flags | (gca.GC_MOMENTUM_MASK if mask else 0))
    dev = torch.device("cuda")
    e_d = torch.zeros(n, device=dev) if ef else None
    e_h = np.zeros(n, np.float32) if ef else None
    u_d = torch.zeros(n, device=dev) if momentum is not None else None
    u_h = np.zeros(n, np.float32) if momentum is not None else None
    tk = max(plan.total_k, 1)
    vals = torch.empty(tk, device=dev)
    idx = torch.empty(tk, dtype=torch.int32, device=dev)
    for t, g in enumerate(grads):
        log(f"[randk {label}] iteration {t}")
        vals.fill_(float("nan"))
        idx.fill_(-7)
        plan.randk_compress(torch.from_numpy(g).to(dev), vals, idx, e=e_d, u=u_d,
                            momentum=momentum or 0.0, seed=seed, step=t)
        torch.cuda.synchronize()
        v_d, i_d = vals.cpu().numpy(), idx.cpu().numpy()
        for s in range(len(sizes)):
            a, b = int(off[s]), int(off[s + 1])
            ka, kb = int(plan.out_off[s]), int(plan.out_off[s + 1])
            hv, hi = oracle.randk_segment(
                g[a:b].copy(), int(ks[s]), e=None if e_h is None else e_h[a:b],
                u=None if u_h is None else u_h[a:b], momentum=momentum or 0.0, mask_u=mask,
                seed=seed, step=t, seg_base=a)
            assert_bitwise(i_d[ka:kb], hi, f"{label} it{t} seg{s} idx")
            assert_bitwise(v_d[ka:kb], hv, f"{label} it{t} seg{s} vals")
        if e_h is not None:
            assert_bitwise(e_d, e_h, f"{label} it{t} residual")
        if u_h is not None:
            assert_bitwise(u_d, u_h, f"{label} it{t} velocity")
    return plan


RK = [10, 100, 40, 300, 4097, 1]


def test_randk_ragged_ef():
    run_randk(SIZES, RK, _grads(sum(SIZES), 4, 11), label="ragged-ef")


def test_randk_unbiased_without_feedback():
    run_randk(SIZES, RK, _grads(sum(SIZES), 3, 12), ef=False, label="scaled")


@pytest.mark.parametrize("ef", [True, False], ids=["ef", "no-ef"])
def test_randk_momentum_mask(ef):
    run_randk(SIZES, RK, _grads(sum(SIZES), 3, 13), ef=ef, momentum=0.9, mask=True,
              label=f"momentum-{ef}")


def test_randk_k_edges():
    sizes = [1, 7, 8192, 8193, 100000]
    run_randk(sizes, [1, 0, 8192, 1, 100000], _grads(sum(sizes), 2, 14), label="edges")


@pytest.mark.parametrize("chain", [True, False], ids=["chain", "single"])
@pytest.mark.parametrize("flag", [gca.GC_DEBUG_FORCE_FALLBACK, gca.GC_DEBUG_NO_ESTIMATE],
                         ids=["forced-full", "recapture"])
def test_randk_fallbacks(flag, chain):
    """Both fallbacks, through the chain of kernels (re-capture or full path) and through the
    one-workgroup-per-segment select (always the whole segment)."""
    sizes = [300001, 70003, 1001]
    plan = run_randk(sizes, [300, 100, 10], _grads(sum(sizes), 2, 15),
                     flags=flag | (gca.GC_DEBUG_CHAIN if chain else 0),
                     label=f"flag{flag:#x} chain={chain}")
    st = plan.last_stats()
    recap = flag != gca.GC_DEBUG_FORCE_FALLBACK and chain
    want = gca.MODE_RECAPTURED if recap else gca.MODE_FULL
    assert st["mode"][0] == want, st["mode"]


def test_randk_mask_independent_of_values():
    """Same (seed, step) on different gradients: the same positions."""
    sizes = [300001, 4097]
    off = _offsets(sizes)
    plan = gca.Plan(off, ratio=0.01)
    out = []
    for seed in (21, 22):
        g = torch.from_numpy(_grads(int(off[-1]), 1, seed)[0]).cuda()
        vals = torch.empty(plan.total_k, device="cuda")
        idx = torch.empty(plan.total_k, dtype=torch.int32, device="cuda")
        plan.randk_compress(g, vals, idx, seed=99, step=3)
        out.append(idx.cpu().numpy())
    assert np.array_equal(out[0], out[1])


# ------------------------------------------------------------------------- full size
def _full_checks(plan, off, acc, e_new, vals, idx, scaled):
    oo = plan.out_off
    for s in range(len(off) - 1):
        a, b = int(off[s]), int(off[s + 1])
        ka, kb = int(oo[s]), int(oo[s + 1])
        ii = idx[ka:kb].long()
        resid = acc[a:b].clone()
        if kb > ka:
            assert int(ii.min()) >= 0 and int(ii.max()) < b - a, f"index range seg {s}"
            if kb - ka > 1:
                assert bool((ii[1:] > ii[:-1]).all()), f"ascending seg {s}"
            want = acc[a:b][ii]
            if scaled:
                want = torch.mul(want, float(np.float32((b - a) / (kb - ka))))
            assert torch.equal(vals[ka:kb].view(torch.int32), want.view(torch.int32)), f"vals {s}"
            resid[ii] = 0.0
        if e_new is not None:
            assert torch.equal(resid.view(torch.int32), e_new[a:b].view(torch.int32)), f"res {s}"


def test_randk_full_size_llama2_7b():
    wl = workload("c5p_llama2_7b_plain")
    off = wl.offsets()
    dev = torch.device("cuda")
    plan = gca.Plan(off, ratio=wl.ratio)
    g = torch.empty(wl.n, device=dev)
    e = torch.zeros(wl.n, device=dev)
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    sample = [2, 8, 150, 289]
    host = {s: np.zeros(int(off[s + 1] - off[s]), np.float32) for s in sample}
    for t in range(2):
        gen.fill_gradient(g, wl, t)
        acc = torch.add(e, g)
        plan.randk_compress(g, vals, idx, e=e, seed=17, step=t)
        torch.cuda.synchronize()
        st = plan.last_stats()
        log(f"[randk full] it{t}: modes={np.bincount(st['mode'], minlength=4).tolist()} "
            f"candidates/k={st['candidates'].sum() / plan.total_k:.3f}")
        _full_checks(plan, off, acc, e, vals, idx, scaled=False)
        del acc
        for s in sample:
            a, b = int(off[s]), int(off[s + 1])
            ka, kb = int(plan.out_off[s]), int(plan.out_off[s + 1])
            hv, hi = oracle.randk_segment(g[a:b].cpu().numpy(), int(plan.k[s]), e=host[s],
                                          seed=17, step=t, seg_base=a)
            assert_bitwise(idx[ka:kb], hi, f"randk full it{t} seg{s} idx")
            assert_bitwise(vals[ka:kb], hv, f"randk full it{t} seg{s} vals")
            assert_bitwise(e[a:b], host[s], f"randk full it{t} seg{s} residual")
    plan.close()


def test_threshold_full_size_llama2_7b():
    """tau_s = 1e-4 x (8 + s mod 10) on Student-t(3) x 1e-4 gradients: the 0.1% quantile
    of |t_3| is about 12.9, so segments below the cap and at it both occur."""
    wl = workload("c5p_llama2_7b_plain")
    off = wl.offsets()
    dev = torch.device("cuda")
    plan = gca.Plan(off, ratio=wl.ratio)
    g = torch.empty(wl.n, device=dev)
    e = torch.zeros(wl.n, device=dev)
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(wl.n_seg, dtype=torch.int32, device=dev)
    sample = [2, 8, 150, 289]
    host = {s: np.zeros(int(off[s + 1] - off[s]), np.float32) for s in sample}
    for t in range(2):
        gen.fill_gradient(g, wl, t)
        tau = torch.tensor([1e-4 * (8 + s % 10) for s in range(wl.n_seg)],
                           dtype=torch.float32, device=dev)
        acc = torch.add(e, g)
        plan.threshold_compress(g, e, tau, vals, idx, cnt)
        torch.cuda.synchronize()
        c = cnt.cpu().numpy()
        k = plan.k
        log(f"[threshold full] it{t}: at cap {int((c == k).sum())} of {wl.n_seg}, "
            f"kept {int(c.sum())} of {int(k.sum())}")
        oo = plan.out_off
        for s in range(wl.n_seg):
            a, b = int(off[s]), int(off[s + 1])
            ka = int(oo[s])
            ii = idx[ka:ka + int(c[s])].long()
            ge = acc[a:b].abs() >= tau[s]
            n_ge = int(ge.sum())
            assert c[s] == min(n_ge, int(k[s])), f"count seg {s}"
            assert bool((idx[ka + int(c[s]):int(oo[s + 1])] == -1).all()), f"padding seg {s}"
            resid = acc[a:b].clone()
            if c[s]:
                assert bool((ii[1:] > ii[:-1]).all()), f"ascending seg {s}"
                assert bool(ge[ii].all()), f"kept below tau seg {s}"
                assert torch.equal(vals[ka:ka + int(c[s])].view(torch.int32),
                                   acc[a:b][ii].view(torch.int32)), f"vals seg {s}"
                resid[ii] = 0.0
                if n_ge > int(k[s]):
                    dropped = torch.ones(b - a, dtype=torch.bool, device=dev)
                    dropped[ii] = False
                    lo = float(acc[a:b][ii].abs().min())
                    hi = float(acc[a:b][dropped].abs().max())
                    assert lo >= hi, f"top-k among those above tau seg {s}"
            assert torch.equal(resid.view(torch.int32), e[a:b].view(torch.int32)), f"res {s}"
        del acc
        for s in sample:
            a, b = int(off[s]), int(off[s + 1])
            ka = int(oo[s])
            hv, hi = oracle.threshold_ef_segment(g[a:b].cpu().numpy(), host[s], int(k[s]),
                                                 float(tau[s]))
            assert_bitwise(idx[ka:ka + hi.size], hi, f"threshold full it{t} seg{s} idx")
            assert_bitwise(vals[ka:ka + hi.size], hv, f"threshold full it{t} seg{s} vals")
            assert_bitwise(e[a:b], host[s], f"threshold full it{t} seg{s} residual")
    plan.close()


def test_int8_stage_on_threshold_payloads():
    """gc_quant_int8 on a threshold payload: the (+0, -1) padding neither moves the scale nor
    touches the residual; the kept entries' codes and the fed-back error match the oracle's
    int8 stage on the kept entries alone."""
    off = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int64)
    n = int(off[-1])
    ks = np.array([50, 300, 40, 500, 4097, 3], np.int64)
    plan = gca.Plan(off, k=ks)
    g = _grads(n, 1, 71)[0]
    tau = np.array(_taus_mixed(0, g, None), np.float32)
    dev = torch.device("cuda")
    e_d = torch.zeros(n, device=dev)
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(len(SIZES), dtype=torch.int32, device=dev)
    codes = torch.empty(plan.total_k, dtype=torch.int8, device=dev)
    scales = torch.empty(len(SIZES), device=dev)
    plan.threshold_compress(torch.from_numpy(g).to(dev), e_d, torch.from_numpy(tau).to(dev),
                            vals, idx, cnt)
    plan.quant_int8(vals, idx, codes, scales, e=e_d, seed=5, step=1)
    torch.cuda.synchronize()
    e_h = np.zeros(n, np.float32)
    c = cnt.cpu().numpy()
    for s in range(len(SIZES)):
        a, b = int(off[s]), int(off[s + 1])
        ka = int(plan.out_off[s])
        hv, hi = oracle.threshold_ef_segment(g[a:b].copy(), e_h[a:b], int(ks[s]), float(tau[s]))
        assert hi.size == c[s]
        hc, hs = oracle.quant_int8_segment(hv, hi, a, e_h[a:b], seed=5, step=1)
        assert_bitwise(codes[ka:ka + hi.size], hc, f"seg {s} codes")
        assert_bitwise(scales[s:s + 1], np.array([hs], np.float32), f"seg {s} scale")
        assert bool((codes[ka + hi.size:int(plan.out_off[s + 1])] == 0).all())
    assert_bitwise(e_d, e_h, "residual with the quantisation error fed back")
