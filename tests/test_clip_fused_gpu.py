"""Clipping folded into the compress calls: with a per-segment gradient scale set on the
plan, every codec must give what clipping g first (the oracle's clip) and then running the
oracle's codec gives, bit for bit.  The factors are the oracle's fl32(c / norm)."""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu

SIZES = [1001, 70003, 8192 * 3 + 5, 300001, 4097]
KS = [10, 100, 40, 300, 41]


def _setup(seed):
    off = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int64)
    n = int(off[-1])
    rng = np.random.default_rng(seed)
    grads = [(rng.standard_t(3, n) * 1e-2).astype(np.float32) for _ in range(2)]
    return off, n, grads


def _clip_host(g, off, frac):
    """The oracle's clip of every segment to frac x its norm (segment 2 left alone);
    returns the clipped copy and the factors fl32(c / norm) (1 where not clipped)."""
    h = g.copy()
    f = np.ones(len(SIZES), np.float32)
    for s in range(len(SIZES)):
        a, b = int(off[s]), int(off[s + 1])
        true = np.linalg.norm(g[a:b].astype(np.float64))
        c = np.float32(true * (2.0 if s == 2 else frac))
        norm = oracle.clip_by_norm_segment(h[a:b], float(c))
        if norm > c:
            f[s] = np.float32(c) / np.float32(norm)
    return h, f


@pytest.mark.parametrize("codec", ["topk", "topk_momentum", "int8", "threshold", "randk_ef",
                                   "randk_plain", "sign", "sign_momentum", "qsgd_ef",
                                   "qsgd_plain", "qsgd_momentum"])
def test_fused_scale_matches_clip_then_codec(codec):
    off, n, grads = _setup(61)
    plan = gca.Plan(off, k=np.array(KS, np.int64))
    dev = torch.device("cuda")
    mom = codec.endswith("momentum")
    ef = codec not in ("randk_plain", "qsgd_plain", "qsgd_momentum")
    e_d = torch.zeros(n, device=dev) if ef else None
    e_h = np.zeros(n, np.float32) if ef else None
    u_d = torch.zeros(n, device=dev) if mom else None
    u_h = np.zeros(n, np.float32) if mom else None
    tk = plan.total_k
    vals = torch.empty(tk, device=dev)
    idx = torch.empty(tk, dtype=torch.int32, device=dev)
    codes = torch.empty(max(n, tk), dtype=torch.int8, device=dev)
    scales = torch.empty(len(SIZES), device=dev)
    bits = torch.empty(plan.total_words, dtype=torch.int32, device=dev)
    tau = torch.tensor([1e-2, 3e-2, 0.0, 5e-2, 1e-3], device=dev)
    for t, g in enumerate(grads):
        h, f = _clip_host(g, off, 0.5 if t == 0 else 0.3)
        fd = torch.from_numpy(f).to(dev)
        plan.set_gradient_scale(fd)
        gd = torch.from_numpy(g).to(dev)
        m = 0.9 if mom else 0.0
        if codec in ("topk", "topk_momentum"):
            plan.compress(gd, e_d, vals, idx, u=u_d, momentum=m)
        elif codec == "int8":
            plan.compress_int8(gd, e_d, idx, codes, scales, out_vals=vals, seed=4, step=t)
        elif codec == "threshold":
            plan.threshold_compress(gd, e_d, tau, vals, idx)
        elif codec.startswith("randk"):
            plan.randk_compress(gd, vals, idx, e=e_d, seed=4, step=t)
        elif codec.startswith("sign"):
            plan.sign_compress(gd, e_d, bits, scales, u=u_d, momentum=m)
        else:
            plan.qsgd_compress(gd, codes, scales, levels=31, e=e_d, u=u_d, momentum=m, seed=4,
                               step=t)
        torch.cuda.synchronize()
        log(f"[fused clip {codec}] iteration {t}")
        v_d, i_d = vals.cpu().numpy(), idx.cpu().numpy()
        for s in range(len(SIZES)):
            a, b = int(off[s]), int(off[s + 1])
            ka = int(plan.out_off[s])
            hs = h[a:b].copy()
            es = None if e_h is None else e_h[a:b]
            us = None if u_h is None else u_h[a:b]
            what = f"{codec} it{t} seg{s}"
            if codec in ("topk", "topk_momentum"):
                hv, hi = oracle.topk_ef_segment(hs, es, KS[s], u=us, momentum=m)
            elif codec == "int8":
                hv, hi = oracle.topk_ef_segment(hs, es, KS[s])
                hc, hsc = oracle.quant_int8_segment(hv, hi, a, es, seed=4, step=t)
                assert_bitwise(codes[ka:ka + KS[s]], hc, what + " codes")
                assert_bitwise(scales[s:s + 1], np.array([hsc], np.float32), what + " scale")
            elif codec == "threshold":
                hv, hi = oracle.threshold_ef_segment(hs, es, KS[s], float(tau[s]))
            elif codec.startswith("randk"):
                hv, hi = oracle.randk_segment(hs, KS[s], e=es, seed=4, step=t, seg_base=a)
            elif codec.startswith("sign"):
                hb, hsc = oracle.sign_ef_segment(hs, es, u=us, momentum=m)
                wa, wb = int(plan.word_off[s]), int(plan.word_off[s + 1])
                assert_bitwise(bits[wa:wb].cpu().numpy().view(np.uint32), hb, what + " bits")
                sd = float(scales[s])
                assert abs(sd - float(hsc)) <= float(np.spacing(np.float32(abs(hsc))))
                if sd != hsc:     # the scale's double sum order: continue from the GPU's
                    e_h[a:b] = e_d[a:b].cpu().numpy()
                continue
            else:
                hc, hn = oracle.qsgd_segment(hs, es, u=us, momentum=m, levels=31, seed=4,
                                             step=t, seg_base=a)
                nd = float(scales[s])
                assert abs(nd - float(hn)) <= float(np.spacing(np.float32(abs(hn))))
                if nd == hn:
                    assert_bitwise(codes[a:b], hc, what + " codes")
                elif e_h is not None:
                    e_h[a:b] = e_d[a:b].cpu().numpy()
                continue
            assert_bitwise(i_d[ka:ka + hi.size], hi, what + " idx")
            assert_bitwise(v_d[ka:ka + hv.size], hv, what + " vals")
        if e_h is not None:
            assert_bitwise(e_d, e_h, f"{codec} it{t} residual")
        if u_h is not None:
            assert_bitwise(u_d, u_h, f"{codec} it{t} velocity")
        assert_bitwise(gd, g, f"{codec} it{t} g untouched")
    plan.set_gradient_scale(None)
    plan.close()


def test_clip_factors_match_the_oracle():
    off, n, grads = _setup(62)
    plan = gca.Plan(off, k=0)
    g = grads[0]
    true = [np.linalg.norm(g[int(off[s]):int(off[s + 1])].astype(np.float64))
            for s in range(len(SIZES))]
    c = np.array([t * (2.0 if s == 2 else 0.5) for s, t in enumerate(true)], np.float32)
    fd = torch.empty(len(SIZES), device="cuda")
    nd = torch.empty(len(SIZES), device="cuda")
    gd = torch.from_numpy(g).cuda()
    plan.clip_factors(gd, torch.from_numpy(c).cuda(), fd, norms_out=nd)
    torch.cuda.synchronize()
    for s in range(len(SIZES)):
        a, b = int(off[s]), int(off[s + 1])
        hn = oracle.clip_by_norm_segment(g[a:b].copy(), float(c[s]))
        assert abs(float(nd[s]) - float(hn)) <= float(np.spacing(np.float32(hn)))
        if float(nd[s]) == hn:
            want = np.float32(c[s]) / np.float32(hn) if hn > c[s] else np.float32(1.0)
            assert float(fd[s]) == float(want), s
    assert_bitwise(gd, g, "g untouched")
    plan.close()
