"""GPU parity of the receiver-side sum of several workers' payloads (C ABI) against the CPU
oracle: payloads made by the oracle (or drawn by the seeded generator at full size), added
on the GPU in worker order, compared bit for bit."""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
import synth
from synth import workload
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu

SIZES = [1001, 70003, 8192 * 3 + 5, 300001, 4097]


def _oracle_payloads(seg_off, k, P, seed):
    n = int(seg_off[-1])
    rng = np.random.default_rng(seed)
    vals, idx = [], []
    for _ in range(P):
        g = rng.standard_t(3, n).astype(np.float32)
        v, i = oracle.topk_ef(g, np.zeros(n, np.float32), seg_off, k)
        vals.append(v)
        idx.append(i)
    return np.concatenate(vals), np.concatenate(idx)


@pytest.mark.parametrize("accumulate", [False, True], ids=["fresh", "accumulate"])
def test_gathered_topk_payloads(accumulate):
    seg_off = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int64)
    n = int(seg_off[-1])
    plan = gca.Plan(seg_off, ratio=0.01)
    P = 4
    vals, idx = _oracle_payloads(seg_off, plan.k, P, 41)
    base = np.random.default_rng(42).standard_normal(n).astype(np.float32)
    want = oracle.decompress_gathered(seg_off, plan.k, P, idx, vals=vals, dense=base.copy(),
                                      accumulate=accumulate)
    dense = torch.from_numpy(base).cuda()
    plan.decompress_gathered(P, torch.from_numpy(idx).cuda(), dense,
                             vals=torch.from_numpy(vals).cuda(), accumulate=accumulate)
    torch.cuda.synchronize()
    assert_bitwise(dense, want, "gathered sum")
    plan.close()


def test_gathered_int8_and_threshold_padding():
    seg_off = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int64)
    n = int(seg_off[-1])
    ks = np.array([50, 300, 40, 500, 4097], np.int64)
    plan = gca.Plan(seg_off, k=ks)
    P = 3
    rng = np.random.default_rng(43)
    # threshold payloads: kept entries then (+0, -1) padding
    vals, idx = [], []
    for w in range(P):
        g = rng.standard_t(3, n).astype(np.float32)
        e = np.zeros(n, np.float32)
        for s in range(len(SIZES)):
            a, b = int(seg_off[s]), int(seg_off[s + 1])
            v, i = oracle.threshold_ef_segment(g[a:b].copy(), e[a:b], int(ks[s]), 2.0 + w)
            pad = int(ks[s]) - i.size
            vals.append(np.concatenate([v, np.zeros(pad, np.float32)]))
            idx.append(np.concatenate([i, np.full(pad, -1, np.int32)]))
    vals, idx = np.concatenate(vals), np.concatenate(idx)
    assert (idx == -1).any()
    want = oracle.decompress_gathered(seg_off, ks, P, idx, vals=vals)
    dense = torch.empty(n, device="cuda")
    plan.decompress_gathered(P, torch.from_numpy(idx).cuda(), dense,
                             vals=torch.from_numpy(vals).cuda())
    torch.cuda.synchronize()
    assert_bitwise(dense, want, "threshold payloads")
    # int8 payloads: the same indices with drawn codes and per-worker scales
    codes = rng.integers(-127, 128, idx.size).astype(np.int8)
    scales = (rng.random(P * len(SIZES)) + 0.5).astype(np.float32)
    want = oracle.decompress_gathered(seg_off, ks, P, idx, codes=codes, scales=scales)
    plan.decompress_gathered(P, torch.from_numpy(idx).cuda(), dense,
                             codes=torch.from_numpy(codes).cuda(),
                             scales=torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    assert_bitwise(dense, want, "int8 payloads")
    plan.close()


def test_gathered_full_size_llama2_7b_eight_workers():
    """Eight workers' payloads of the 7B shape at k = 0.1% (synth.fill_payloads: sorted
    distinct indices per segment, Student-t values): every position against torch's
    index_add_ worker by worker (unique indices within a payload, so one fp32 add per worker
    and position, in worker order), sampled segments against the oracle."""
    wl = workload("c5p_llama2_7b_plain")
    off = wl.offsets()
    plan = gca.Plan(off, ratio=wl.ratio)
    P, K = 8, plan.total_k
    dev = torch.device("cuda")
    vals = torch.empty(P * K, device=dev)
    idx = torch.empty(P * K, dtype=torch.int32, device=dev)
    oo = plan.out_off
    synth.fill_payloads(vals, idx, off, plan.k, P, seed=5)
    log("[gathered full] payloads drawn")
    dense = torch.empty(wl.n, device=dev)
    plan.decompress_gathered(P, idx, dense, vals=vals)
    ref = torch.zeros(wl.n, device=dev)
    seg_of_entry = torch.from_numpy(np.repeat(np.arange(wl.n_seg), plan.k)).to(dev)
    base = torch.from_numpy(off[:-1]).to(dev)[seg_of_entry]
    for w in range(P):
        pos = base + idx[w * K:(w + 1) * K].long()
        ref.index_add_(0, pos, vals[w * K:(w + 1) * K])
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int32), ref.view(torch.int32))
    log(f"[gathered full] union density {(dense != 0).sum().item() / wl.n:.5f}")
    for s in (2, 8, 150, 289):
        a, b = int(off[s]), int(off[s + 1])
        ks = np.array([plan.k[s]], np.int64)
        sub_idx = np.concatenate([idx[w * K + int(oo[s]):w * K + int(oo[s + 1])].cpu().numpy()
                                  for w in range(P)])
        sub_val = np.concatenate([vals[w * K + int(oo[s]):w * K + int(oo[s + 1])].cpu().numpy()
                                  for w in range(P)])
        want = oracle.decompress_gathered(np.array([0, b - a], np.int64), ks, P, sub_idx,
                                          vals=sub_val)
        assert_bitwise(dense[a:b], want, f"segment {s}")
    plan.close()
