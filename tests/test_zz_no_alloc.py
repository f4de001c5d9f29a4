"""The entry point that allocates nothing (gc_topk_ef_compress_noalloc), through the C ABI:
two calls in a row, the second on a smaller input, each bit-identical to gc_topk_ef_compress
on a plan made from the same arguments (and to the CPU oracle); sizes past the static limits
are refused before anything is launched."""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu


def _one_call(sizes, ratio, momentum, flags, seed, base=0):
    off = (base + np.concatenate([[0], np.cumsum(sizes)])).astype(np.int64)
    n = int(off[-1])
    ks, out_off = gca.layout(off, ratio=ratio)
    tk = int(out_off[-1])
    rng = np.random.default_rng(seed)
    g_h = np.zeros(n, np.float32)
    g_h[base:] = (rng.standard_t(3, n - base) * 1e-3).astype(np.float32)
    e0 = np.zeros(n, np.float32)
    e0[base:] = (rng.standard_t(3, n - base) * 1e-3).astype(np.float32)
    u0 = np.zeros(n, np.float32)
    u0[base:] = (rng.standard_t(3, n - base) * 1e-3).astype(np.float32)
    dev = torch.device("cuda")
    g = torch.from_numpy(g_h).to(dev)
    outs = []
    for path in ("plan", "noalloc"):
        e = torch.from_numpy(e0).to(dev)
        u = torch.from_numpy(u0).to(dev) if momentum is not None else None
        vals = torch.full((max(tk, 1),), float("nan"), device=dev)
        idx = torch.full((max(tk, 1),), -1, dtype=torch.int32, device=dev)
        if path == "plan":
            plan = gca.Plan(off, ratio=ratio, flags=flags)
            plan.compress(g, e, vals, idx, u=u, momentum=momentum or 0.0)
            torch.cuda.synchronize()
            plan.close()
        else:
            gca.topk_ef_compress_noalloc(off, g, e, vals, idx, ratio=ratio, flags=flags, u=u,
                                         momentum=momentum or 0.0)
        torch.cuda.synchronize()
        outs.append((vals[:tk].cpu().numpy(), idx[:tk].cpu().numpy(), e.cpu().numpy(),
                     None if u is None else u.cpu().numpy()))
    (v1, i1, e1, u1), (v2, i2, e2, u2) = outs
    label = f"noalloc n={n} segs={len(sizes)}"
    assert_bitwise(i2, i1, f"{label} idx")
    assert_bitwise(v2, v1, f"{label} vals")
    assert_bitwise(e2, e1, f"{label} residual")
    if u1 is not None:
        assert_bitwise(u2, u1, f"{label} velocity")
    # and the oracle on the same inputs
    e_h, u_h = e0.copy(), (u0.copy() if momentum is not None else None)
    vo, io = oracle.topk_ef(g_h, e_h, off, ks, u=u_h, momentum=momentum or 0.0,
                            mask_u=bool(flags & gca.GC_MOMENTUM_MASK))
    assert_bitwise(i2, io, f"{label} idx vs oracle")
    assert_bitwise(v2, vo, f"{label} vals vs oracle")
    assert_bitwise(e2, e_h, f"{label} residual vs oracle")
    if u_h is not None:
        assert_bitwise(u2, u_h, f"{label} velocity vs oracle")
    log(f"[{label}] bit-identical to the plan entry point and the oracle")


def test_noalloc_matches_plan_two_calls():
    # a larger call (ragged, an empty segment, segments past the small size, momentum with
    # masking), then a smaller one on other segments, ratio and no momentum: the static array
    # keeps the first call's contents, which the second call must not see
    _one_call([5, 8192, 20001, 1 << 17, 300001, 65537, 0, 1_000_003, 77], 0.01, 0.9,
              gca.GC_MOMENTUM_MASK, seed=1)
    _one_call([100, 70000, 12345], 0.05, None, 0, seed=2, base=40)


def test_noalloc_tie_heavy_and_edges():
    # integer-valued data (ties straddle the k-th key), k = 0 and k = n segments
    sizes = [200003, 5000, 70001]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    rng = np.random.default_rng(5)
    g_h = rng.integers(-3, 4, n).astype(np.float32)
    dev = torch.device("cuda")
    for k in ([997, 0, 70001], [1, 5000, 0]):
        ks = np.asarray(k, np.int64)
        tk = int(ks.sum())
        e_ref = torch.zeros(n, device=dev)
        e_na = torch.zeros(n, device=dev)
        v_ref = torch.empty(max(tk, 1), device=dev)
        i_ref = torch.empty(max(tk, 1), dtype=torch.int32, device=dev)
        v_na = torch.empty(max(tk, 1), device=dev)
        i_na = torch.empty(max(tk, 1), dtype=torch.int32, device=dev)
        g = torch.from_numpy(g_h).to(dev)
        plan = gca.Plan(off, k=ks)
        plan.compress(g, e_ref, v_ref, i_ref)
        gca.topk_ef_compress_noalloc(off, g, e_na, v_na, i_na, k=ks)
        torch.cuda.synchronize()
        plan.close()
        assert_bitwise(i_na[:tk], i_ref[:tk].cpu().numpy(), "ties idx")
        assert_bitwise(v_na[:tk], v_ref[:tk].cpu().numpy(), "ties vals")
        assert_bitwise(e_na, e_ref.cpu().numpy(), "ties residual")


def test_noalloc_refuses_sizes_past_its_limits():
    dev = torch.device("cuda")
    g = torch.zeros(16, device=dev)
    e = torch.zeros(16, device=dev)
    v = torch.zeros(16, device=dev)
    i = torch.zeros(16, dtype=torch.int32, device=dev)
    too_many = np.arange(66, dtype=np.int64) * 0     # 65 empty segments
    with pytest.raises(gca.GCError) as ex:
        gca.topk_ef_compress_noalloc(too_many, g, e, v, i, k=0)
    assert ex.value.status == gca.GC_ERR_UNSUPPORTED
    big = np.array([0, (1 << 22) + 4], np.int64)   # one element past the largest buffer
    L = gca.lib()
    kk = np.zeros(1, np.int64)
    rc = L.gc_topk_ef_compress_noalloc(big.ctypes.data, 1, kk.ctypes.data, None, 0, None, None,
                                       None, 0.0, None, None, None)
    assert rc == gca.GC_ERR_UNSUPPORTED
