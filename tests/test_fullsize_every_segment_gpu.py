"""GPU parity at full size with the CPU oracle on EVERY segment, bit for bit, for every EF
step the workload states.

The ResNet-50-shaped workload (161 tensors, 25.6M elements, k = 1%, 10 EF steps), the
BERT-large-shaped one (391 tensors, 335M elements, k = 0.1%, 5 steps) and the hybrid int8
workload (64 segments of 2^24, k = 1%, fused int8 with the quantisation error fed back, 5
steps) run on one plan each, in the launch configuration the bench times.  After every call
the oracle recomputes each segment from its own state (carried from zero; a thread pool over
segments, since segments are independent), and values, indices, residual, codes and scales
must equal the GPU's bit for bit over the whole buffer.  The 7B shapes are compared over
every segment on one call and on sampled segments for the others (test_fullsize_gpu.py).
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from synth import gen, workload
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu


def _threads():
    return max(1, min(len(os.sched_getaffinity(0)), 16))


@pytest.mark.parametrize("name", ["c2_resnet50", "c3_bert_large", "c4_hybrid_int8"])
def test_every_segment_against_oracle(name):
    wl = workload(name)
    iters = wl.iters
    off = np.asarray(wl.offsets(), np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, ratio=wl.ratio)
    ks = np.array([oracle.k_from_ratio(int(off[s + 1] - off[s]), wl.ratio)
                   for s in range(wl.n_seg)], np.int64)
    assert np.array_equal(plan.k, ks)
    dev = torch.device("cuda")
    g = torch.empty(n, dtype=torch.float32, device=dev)
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    vals = torch.empty(plan.total_k, dtype=torch.float32, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    codes = torch.empty(plan.total_k, dtype=torch.int8, device=dev)
    scales = torch.empty(wl.n_seg, dtype=torch.float32, device=dev)
    e_h = np.zeros(n, np.float32)
    oracle.lib()
    order = sorted(range(wl.n_seg), key=lambda s: -(int(off[s + 1]) - int(off[s])))
    with cf.ThreadPoolExecutor(max_workers=_threads()) as ex:
        for t in range(iters):
            gen.fill_gradient(g, wl, t)
            g_h = g.cpu().numpy()
            log(f"[every segment {name}] iteration {t}: n={n} segs={wl.n_seg} "
                f"total_k={plan.total_k}")
            vals.fill_(float("nan"))
            idx.fill_(-1)
            if wl.int8:
                plan.compress_int8(g, e, idx, codes, scales, out_vals=vals, seed=0, step=t)
            else:
                plan.compress(g, e, vals, idx)

            def run(s):
                a, b = int(off[s]), int(off[s + 1])
                es = e_h[a:b]   # a view: the oracle updates the host residual in place
                v, i = oracle.topk_ef_segment(g_h[a:b], es, int(ks[s]))
                if not wl.int8:
                    return s, v, i, None, None
                c, sc = oracle.quant_int8_segment(v, i, a, e_seg=es, seed=0, step=t)
                return s, v, i, c, sc

            res = dict((r[0], r) for r in ex.map(run, order))
            res = [res[s] for s in range(wl.n_seg)]
            torch.cuda.synchronize()
            vals_o = np.concatenate([r[1] for r in res])
            idx_o = np.concatenate([r[2] for r in res])
            assert_bitwise(idx[:plan.total_k], idx_o, f"{name} it{t} idx")
            assert_bitwise(vals[:plan.total_k], vals_o, f"{name} it{t} vals")
            if wl.int8:
                assert_bitwise(codes, np.concatenate([r[3] for r in res]), f"{name} it{t} codes")
                assert_bitwise(scales, np.array([r[4] for r in res], np.float32),
                               f"{name} it{t} scales")
            assert_bitwise(e, e_h, f"{name} it{t} residual")
            st = plan.last_stats()
            log(f"[every segment {name}] iteration {t}: all {wl.n_seg} segments bit-exact "
                f"(modes {np.bincount(st['mode'], minlength=4).tolist()})")
    plan.close()
