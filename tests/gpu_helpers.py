"""Shared driver of the GPU parity tests: run the HIP path (through the C ABI) and the CPU
oracle on the same seeded inputs and compare bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gradient_compression_amd as gca
import oracle


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype.itemsize == 4 else np.uint8)


def assert_bitwise(got, want, what: str):
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    bad = np.flatnonzero(g != w)
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i}: "
                             f"got {np.asarray(got.cpu() if isinstance(got, torch.Tensor) else got).ravel()[i]!r} "
                             f"want {np.asarray(want).ravel()[i]!r}")


def oracle_k(sizes, k=None, ratio=None):
    if k is not None:
        return np.broadcast_to(np.asarray(k, np.int64), (len(sizes),)).copy()
    r = np.broadcast_to(np.asarray(ratio, np.float64), (len(sizes),))
    return np.array([oracle.k_from_ratio(int(n), float(x)) for n, x in zip(sizes, r)], np.int64)


def run_parity(sizes, grads, *, k=None, ratio=None, momentum=None, mask=False, flags=0,
               int8=False, fused=False, with_vals=True, seed=0, plan=None, check_stats=None,
               label=""):
    """grads: iterable of float32 numpy gradients (one per EF iteration), or a pair
    (iters, f) with f(t, residual) -> gradient, the residual being the oracle's current one.

    Compares vals, idx, e (and u, codes, scales) after every iteration.  Returns the plan."""
    sizes = [int(n) for n in sizes]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    ks = oracle_k(sizes, k, ratio)
    own = plan is None
    if own:
        fl = flags | (gca.GC_MOMENTUM_MASK if mask else 0)
        plan = gca.Plan(off, k=ks if k is not None else None,
                        ratio=None if k is not None else ratio, flags=fl)
    assert np.array_equal(plan.k, ks), "k per segment differs from the oracle's"
    dev = torch.device("cuda")
    e_h = np.zeros(n, np.float32)
    e_d = torch.zeros(n, dtype=torch.float32, device=dev)
    u_h = u_d = None
    if momentum is not None:
        u_h = np.zeros(n, np.float32)
        u_d = torch.zeros(n, dtype=torch.float32, device=dev)
    tk = int(ks.sum())
    vals_d = torch.full((max(tk, 1),), float("nan"), dtype=torch.float32, device=dev)
    idx_d = torch.full((max(tk, 1),), -1, dtype=torch.int32, device=dev)
    codes_d = torch.zeros(max(tk, 1), dtype=torch.int8, device=dev)
    scales_d = torch.zeros(max(len(sizes), 1), dtype=torch.float32, device=dev)
    if isinstance(grads, tuple):
        iters, fn = grads
        grads = (fn(t, e_h.copy()) for t in range(iters))
    for t, g in enumerate(grads):
        g = np.ascontiguousarray(g, np.float32)
        assert g.size == n
        log(f"[parity {label}] iteration {t}: n={n} segs={len(sizes)} total_k={tk}")
        g_d = torch.from_numpy(g).to(dev)
        if fused:   # compress and int8 in one call
            plan.compress_int8(g_d, e_d, idx_d, codes_d, scales_d,
                               out_vals=vals_d if with_vals else None, u=u_d,
                               momentum=momentum or 0.0, seed=seed, step=t)
        else:
            plan.compress(g_d, e_d, vals_d, idx_d, u=u_d, momentum=momentum or 0.0)
        vals_o, idx_o = oracle.topk_ef(g, e_h, off, ks, u=u_h,
                                       momentum=momentum if momentum is not None else 0.0,
                                       mask_u=mask)
        torch.cuda.synchronize()
        stats = plan.last_stats()
        if check_stats:
            check_stats(t, stats)
        assert_bitwise(idx_d[:tk], idx_o, f"{label} it{t} idx")
        if with_vals:
            assert_bitwise(vals_d[:tk], vals_o, f"{label} it{t} vals")
        if u_d is not None:
            assert_bitwise(u_d, u_h, f"{label} it{t} velocity")
        if fused:
            codes_o, scales_o = oracle.quant_int8(vals_o, idx_o, off, ks, e=e_h, seed=seed,
                                                  step=t)
            assert_bitwise(scales_d[:len(sizes)], scales_o, f"{label} it{t} scales")
            assert_bitwise(codes_d[:tk], codes_o, f"{label} it{t} codes")
            assert_bitwise(e_d, e_h, f"{label} it{t} residual after fused int8")
            continue
        assert_bitwise(e_d, e_h, f"{label} it{t} residual")
        if int8:
            plan.quant_int8(vals_d, idx_d, codes_d, scales_d, e=e_d, seed=seed, step=t)
            codes_o, scales_o = oracle.quant_int8(vals_o, idx_o, off, ks, e=e_h, seed=seed,
                                                  step=t)
            torch.cuda.synchronize()
            assert_bitwise(scales_d[:len(sizes)], scales_o, f"{label} it{t} scales")
            assert_bitwise(codes_d[:tk], codes_o, f"{label} it{t} codes")
            assert_bitwise(e_d, e_h, f"{label} it{t} residual after int8")
    if own:
        plan.close()
    return plan
