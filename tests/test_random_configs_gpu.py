"""Seeded random configurations through every sparsifier, against the oracle bit for bit:
random segment tables (empty, tiny, ragged, misaligned, several tiles), random k (0..n),
random flags (momentum with or without the mask, forced fallback, no estimate) and random
value scales, two error-feedback steps each."""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu

CODECS = ("topk", "int8", "threshold", "randk", "randk_plain")


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    n_seg = int(rng.integers(1, 7))
    kinds = rng.integers(0, 4, n_seg)
    sizes = [int(x) for x in np.where(kinds == 0, rng.integers(0, 40, n_seg),
                                      np.where(kinds == 1, rng.integers(40, 9000, n_seg),
                                               np.where(kinds == 2, rng.integers(9000, 70000, n_seg),
                                                        rng.integers(70000, 300000, n_seg))))]
    ks = [int(rng.integers(0, n + 1)) if rng.random() < 0.3 else min(n, int(rng.integers(0, 60)))
          for n in sizes]
    flags = int(rng.choice([0, gca.GC_DEBUG_FORCE_FALLBACK, gca.GC_DEBUG_NO_ESTIMATE]))
    momentum = 0.9 if rng.random() < 0.4 else None
    mask = bool(momentum is not None and rng.random() < 0.5)
    codec = CODECS[seed % len(CODECS)]
    scale = float(10.0 ** rng.uniform(-5, 2))
    return sizes, ks, flags, momentum, mask, codec, scale, rng


@pytest.mark.parametrize("chain", [False, True], ids=["single", "chain"])
@pytest.mark.parametrize("seed", range(100))
def test_random_configuration(seed, chain):
    """chain: the chain of kernels over candidate chunks even where one workgroup per segment
    would select (most of these plans are small enough for that)."""
    sizes, ks, flags, momentum, mask, codec, scale, rng = _config(seed)
    if chain:
        flags |= gca.GC_DEBUG_CHAIN
    if codec == "int8":
        momentum, mask = None, False
    log(f"[random {seed}] {codec} sizes={sizes} k={ks} flags={flags:#x} momentum={momentum} "
        f"mask={mask}")
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, k=np.array(ks, np.int64), flags=flags | (gca.GC_MOMENTUM_MASK if mask else 0))
    dev = torch.device("cuda")
    ef = codec != "randk_plain"
    e_d = torch.zeros(max(n, 4), device=dev) if ef else None
    e_h = np.zeros(max(n, 4), np.float32)
    u_d = torch.zeros(max(n, 4), device=dev) if momentum else None
    u_h = np.zeros(max(n, 4), np.float32) if momentum else None
    tk = max(plan.total_k, 1)
    vals = torch.empty(tk, device=dev)
    idx = torch.empty(tk, dtype=torch.int32, device=dev)
    codes = torch.empty(tk, dtype=torch.int8, device=dev)
    scales = torch.empty(max(len(sizes), 1), device=dev)
    cnt = torch.empty(max(len(sizes), 1), dtype=torch.int32, device=dev)
    m = momentum or 0.0
    for t in range(2):
        g = np.zeros(max(n, 4), np.float32)
        g[:n] = (rng.standard_t(3, n) * scale).astype(np.float32)
        tau = (np.abs(rng.standard_t(3, len(sizes))) * scale * 2).astype(np.float32)
        gd = torch.from_numpy(g).to(dev)
        if codec == "topk":
            plan.compress(gd, e_d, vals, idx, u=u_d, momentum=m)
        elif codec == "int8":
            plan.compress_int8(gd, e_d, idx, codes, scales, out_vals=vals, seed=seed, step=t)
        elif codec == "threshold":
            plan.threshold_compress(gd, e_d, torch.from_numpy(tau).to(dev), vals, idx, cnt,
                                    u=u_d, momentum=m)
        else:
            plan.randk_compress(gd, vals, idx, e=e_d, u=u_d, momentum=m, seed=seed, step=t)
        torch.cuda.synchronize()
        v_d, i_d = vals.cpu().numpy(), idx.cpu().numpy()
        for s in range(len(sizes)):
            a, b = int(off[s]), int(off[s + 1])
            ka = int(plan.out_off[s])
            es = e_h[a:b] if ef else None
            us = u_h[a:b] if momentum else None
            what = f"seed {seed} it{t} seg{s}"
            if codec in ("topk", "int8"):
                hv, hi = oracle.topk_ef_segment(g[a:b].copy(), es, ks[s], u=us, momentum=m,
                                                mask_u=mask)
                if codec == "int8":
                    hc, hs = oracle.quant_int8_segment(hv, hi, a, es, seed=seed, step=t)
                    assert_bitwise(codes[ka:ka + ks[s]], hc, what + " codes")
                    assert_bitwise(scales[s:s + 1], np.array([hs], np.float32), what + " scale")
            elif codec == "threshold":
                hv, hi = oracle.threshold_ef_segment(g[a:b].copy(), es, ks[s], float(tau[s]),
                                                     u=us, momentum=m, mask_u=mask)
                assert int(cnt[s]) == hi.size, what + " count"
            else:
                hv, hi = oracle.randk_segment(g[a:b].copy(), ks[s], e=es, u=us, momentum=m,
                                              mask_u=mask, seed=seed, step=t, seg_base=a)
            assert_bitwise(i_d[ka:ka + hi.size], hi, what + " idx")
            assert_bitwise(v_d[ka:ka + hv.size], hv, what + " vals")
        if ef:
            assert_bitwise(e_d[:n], e_h[:n], f"seed {seed} it{t} residual")
        if momentum:
            assert_bitwise(u_d[:n], u_h[:n], f"seed {seed} it{t} velocity")
    plan.close()
