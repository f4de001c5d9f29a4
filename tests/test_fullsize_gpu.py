"""GPU parity at the workloads' full sizes, in the launch configuration the bench times.

Every iteration checks
  * sampled segments bit for bit against the CPU oracle (the oracle runs on the segment's
    own copy of g, e and u taken before the call; segments are independent);
  * over EVERY segment, with plain torch ops on the GPU (independent of the HIP path),
    the properties that fix the result uniquely:
      - k entries per segment, indices strictly ascending and inside the segment;
      - vals == acc at the kept indices, bit for bit (acc = e_prev + x, x = g or
        u = fl(fl(0.9 u_prev) + g));
      - the new residual equals acc everywhere except the kept indices, where it is +0;
      - min |kept| >= max |dropped| (Top-k), and among equal magnitudes at the threshold
        every kept index is below every dropped one (the tie rule);
  * for the int8 workload: scales = fl(absmax / 127), codes in {floor(a), ceil(a)},
    the quantisation error fed back exactly, and the sampled codes bit for bit.
"""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from synth import gen, workload
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu

CASES = [
    # (workload, iterations, sampled segments for the oracle)
    ("c3_bert_large", 5, [0, 4, 100, 390]),
    ("c4_hybrid_int8", 4, [0, 37]),
    ("c5p_llama2_7b_plain", 3, [2, 8, 150, 289]),
    ("c5_llama2_7b", 3, [2, 8, 150, 289]),
]


def check_compress(plan, wl, off, g, e_prev, e_new, u_prev, u_new, vals, idx):
    """Full-size properties of one compress call over every segment (torch on the GPU)."""
    oo = plan.out_off
    m = np.float32(wl.momentum) if wl.momentum is not None else None
    assert not torch.isnan(vals).any().item()
    for s in range(wl.n_seg):
        a, b = int(off[s]), int(off[s + 1])
        ka, kb = int(oo[s]), int(oo[s + 1])
        ii = idx[ka:kb].long()
        vv = vals[ka:kb]
        if u_prev is not None:
            x = torch.add(torch.mul(u_prev[a:b], float(m)), g[a:b])
            assert torch.equal(x.view(torch.int32), u_new[a:b].view(torch.int32)), f"u seg {s}"
            x = u_new[a:b]
        else:
            x = g[a:b]
        acc = torch.add(e_prev[a:b], x)
        resid = acc.clone()
        if kb > ka:
            assert int(ii.min()) >= 0 and int(ii.max()) < b - a, f"index range seg {s}"
            if kb - ka > 1:
                assert bool((ii[1:] > ii[:-1]).all()), f"ascending seg {s}"
            assert torch.equal(vv.view(torch.int32), acc[ii].view(torch.int32)), f"vals seg {s}"
            resid[ii] = 0.0
        assert torch.equal(resid.view(torch.int32), e_new[a:b].view(torch.int32)), f"resid {s}"
        if 0 < kb - ka < b - a:
            kept_mag = acc[ii].abs()
            dropped = torch.ones(b - a, dtype=torch.bool, device=acc.device)
            dropped[ii] = False
            lo, hi = float(kept_mag.min()), float(acc[dropped].abs().max())
            assert lo >= hi, f"top-k property seg {s}: kept {lo} < dropped {hi}"
            if lo == hi:        # ties straddle the threshold: lower indices kept
                kept_t = ii[kept_mag == lo]
                drop_t = torch.nonzero(dropped & (acc.abs() == lo)).flatten()
                assert int(kept_t.max()) < int(drop_t.min()), f"tie rule seg {s}"


def check_int8(plan, wl, off, vals, idx, codes, scales, e_before, e_after):
    """Full-size properties of the int8 stage (numpy on the host, torch for the rest)."""
    oo = plan.out_off
    v = vals.cpu().numpy()
    c = codes.cpu().numpy().astype(np.int32)
    sc = scales.cpu().numpy()
    for s in range(wl.n_seg):
        a = int(off[s])
        ka, kb = int(oo[s]), int(oo[s + 1])
        vs = v[ka:kb]
        absmax = np.abs(vs).max()
        assert sc[s] == np.float32(np.float64(absmax) / 127.0), f"scale seg {s}"
        aa = np.minimum(np.divide(np.abs(vs), sc[s], dtype=np.float32), np.float32(127))
        q = np.abs(c[ka:kb])
        assert np.all((q == np.floor(aa)) | (q == np.ceil(aa))), f"code bracket seg {s}"
        gi = torch.from_numpy(a + idx[ka:kb].cpu().numpy().astype(np.int64)).to(e_after.device)
        deq = np.multiply(c[ka:kb].astype(np.float32), sc[s], dtype=np.float32)
        want = np.subtract(vs, deq, dtype=np.float32)
        assert e_after[gi].cpu().numpy().tobytes() == want.tobytes(), f"quant feedback seg {s}"
    kept = torch.zeros(e_after.numel(), dtype=torch.bool, device=e_after.device)
    for s in range(wl.n_seg):
        kept[int(off[s]) + idx[int(oo[s]):int(oo[s + 1])].long()] = True
    assert torch.equal(e_after[~kept].view(torch.int32), e_before[~kept].view(torch.int32))
    scale_per = np.repeat(sc, np.diff(oo)).astype(np.float64)
    err = (c.astype(np.float64) * scale_per - v.astype(np.float64)) / scale_per
    assert abs(err.mean()) < 3 * err.std() / np.sqrt(err.size) + 1e-12   # unbiased rounding


@pytest.mark.parametrize("name,iters,sample", CASES, ids=[c[0] for c in CASES])
def test_full_size(name, iters, sample):
    wl = workload(name)
    off = wl.offsets()
    dev = torch.device("cuda")
    log(f"[full {name}] n={wl.n} segs={wl.n_seg} iters={iters}")
    plan = gca.Plan(off, ratio=wl.ratio)
    k_or = np.array([oracle.k_from_ratio(int(off[s + 1] - off[s]), wl.ratio)
                     for s in range(wl.n_seg)], np.int64)
    assert np.array_equal(plan.k, k_or)
    g = torch.empty(wl.n, dtype=torch.float32, device=dev)
    e = torch.zeros(wl.n, dtype=torch.float32, device=dev)
    u = torch.zeros(wl.n, dtype=torch.float32, device=dev) if wl.momentum is not None else None
    vals = torch.empty(plan.total_k, dtype=torch.float32, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    codes = torch.empty(plan.total_k, dtype=torch.int8, device=dev) if wl.int8 else None
    scales = torch.empty(wl.n_seg, dtype=torch.float32, device=dev) if wl.int8 else None
    host = {s: {"e": np.zeros(int(off[s + 1] - off[s]), np.float32),
                "u": np.zeros(int(off[s + 1] - off[s]), np.float32) if u is not None else None}
            for s in sample}
    for t in range(iters):
        gen.fill_gradient(g, wl, t)
        e_prev = e.clone()
        u_prev = u.clone() if u is not None else None
        vals.fill_(float("nan"))
        idx.fill_(-1)
        plan.compress(g, e, vals, idx, u=u, momentum=wl.momentum or 0.0)
        e_cmp = e.clone() if wl.int8 else e
        if wl.int8:
            plan.quant_int8(vals, idx, codes, scales, e=e, seed=0, step=t)
        torch.cuda.synchronize()
        st = plan.last_stats()
        log(f"[full {name}] it{t}: modes={np.bincount(st['mode'], minlength=3).tolist()} "
            f"candidates/k={st['candidates'].sum() / max(plan.total_k, 1):.2f}")
        assert not (idx == -1).any().item()
        check_compress(plan, wl, off, g, e_prev, e_cmp, u_prev, u, vals, idx)
        if wl.int8:
            check_int8(plan, wl, off, vals, idx, codes, scales, e_cmp, e)
        log(f"[full {name}] it{t}: full-size properties hold")
        for s in sample:
            a, b = int(off[s]), int(off[s + 1])
            ka, kb = int(plan.out_off[s]), int(plan.out_off[s + 1])
            gs = g[a:b].cpu().numpy()
            hv, hi = oracle.topk_ef_segment(gs, host[s]["e"], int(plan.k[s]), u=host[s]["u"],
                                            momentum=wl.momentum or 0.0)
            assert_bitwise(idx[ka:kb], hi, f"{name} it{t} seg{s} idx")
            assert_bitwise(vals[ka:kb], hv, f"{name} it{t} seg{s} vals")
            if wl.int8:
                hc, hs = oracle.quant_int8_segment(hv, hi, a, host[s]["e"], seed=0, step=t)
                assert_bitwise(codes[ka:kb], hc, f"{name} it{t} seg{s} codes")
                assert_bitwise(scales[s:s + 1], np.array([hs], np.float32), f"seg{s} scale")
            assert_bitwise(e[a:b], host[s]["e"], f"{name} it{t} seg{s} residual")
            if u is not None:
                assert_bitwise(u[a:b], host[s]["u"], f"{name} it{t} seg{s} velocity")
        del e_prev, u_prev, e_cmp
    plan.close()


def test_fused_int8_full_size_matches_two_calls():
    """The hybrid workload at full size: the fused compress+int8 call and the two separate
    calls give bit-identical values, indices, codes, scales and residuals."""
    wl = workload("c4_hybrid_int8")
    off = wl.offsets()
    dev = torch.device("cuda")
    p1, p2 = gca.Plan(off, ratio=wl.ratio), gca.Plan(off, ratio=wl.ratio)
    g = torch.empty(wl.n, dtype=torch.float32, device=dev)
    e1 = torch.zeros(wl.n, dtype=torch.float32, device=dev)
    e2 = torch.zeros(wl.n, dtype=torch.float32, device=dev)
    mk = lambda dt: torch.empty(p1.total_k, dtype=dt, device=dev)   # noqa: E731
    v1, i1, c1 = mk(torch.float32), mk(torch.int32), mk(torch.int8)
    v2, i2, c2 = mk(torch.float32), mk(torch.int32), mk(torch.int8)
    s1 = torch.empty(wl.n_seg, dtype=torch.float32, device=dev)
    s2 = torch.empty(wl.n_seg, dtype=torch.float32, device=dev)
    for t in range(3):
        gen.fill_gradient(g, wl, t)
        p1.compress(g, e1, v1, i1)
        p1.quant_int8(v1, i1, c1, s1, e=e1, seed=0, step=t)
        p2.compress_int8(g, e2, i2, c2, s2, out_vals=v2, seed=0, step=t)
        torch.cuda.synchronize()
        log(f"[fused full] it{t}")
        for a, b, what in ((v1, v2, "vals"), (i1, i2, "idx"), (c1, c2, "codes"), (s1, s2, "scales")):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.int8 else a.view(torch.int32),
                               b.view(torch.uint8) if b.dtype == torch.int8 else b.view(torch.int32)), what
        assert torch.equal(e1.view(torch.int32), e2.view(torch.int32)), "residual"
    p1.close()
    p2.close()
