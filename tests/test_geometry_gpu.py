"""GPU: no result depends on the tile geometry.

The library is also built at three other geometries (threads x slots 512 x 4, 1024 x 1 and
256 x 2: tiles of 8192, 4096 and 2048 elements).  Each moves every tile, candidate-chunk and
run boundary, the cold-start sample of tiles, the path a segment takes (candidates, re-capture
or the full radix select) and the grouping of the per-tile partial sums.  The tie rule and the
ordered emission are defined on indices, not on tiles, so:
  * Top-k (plain, momentum with the mask, fused int8, forced full path, ties, special values)
    is checked bit for bit against the CPU oracle on each geometry;
  * threshold, Random-k, sign and QSGD run on each geometry and on the default one from the
    same inputs and must agree bit for bit.  The one allowance: the per-segment sums of sign
    and QSGD are added tile by tile in double, in a grouping that follows the tiles, so their
    fp32 scale may differ by one ulp; where it does not, every output must be identical.
"""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
from gradient_compression_amd import build as gc_build
from tests.gpu_helpers import assert_bitwise, bits, log, oracle_k, run_parity

pytestmark = pytest.mark.gpu

VARIANTS = sorted(gc_build.VARIANTS)
# segment starts off a multiple of 4, tails of every length, segments under one tile of each
# geometry and over several
RAGGED = [1, 3, 64, 2047, 2049, 4095, 8192, 8193, 70001, 123457, 2, 65537]


def _off(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def _t_grads(n, iters, seed, scale=1e-3, df=3.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_t(df, n) * scale).astype(np.float32) for _ in range(iters)]


def _plan(sizes, variant, k=None, ratio=None, flags=0):
    off = _off(sizes)
    ks = oracle_k(sizes, k, ratio)
    return gca.Plan(off, k=ks if k is not None else None, ratio=None if k is not None else ratio,
                    flags=flags, variant=variant)


# ------------------------------------------------------------------ Top-k against the oracle
@pytest.mark.parametrize("variant", VARIANTS)
def test_topk_ragged_against_oracle(variant):
    plan = _plan(RAGGED, variant, ratio=0.01)
    run_parity(RAGGED, _t_grads(sum(RAGGED), 4, seed=21), ratio=0.01, plan=plan,
               label=f"{variant} ragged")
    plan.close()


@pytest.mark.parametrize("variant", VARIANTS)
def test_topk_momentum_mask_fused_int8_against_oracle(variant):
    plan = _plan(RAGGED, variant, ratio=0.005, flags=gca.GC_MOMENTUM_MASK)
    run_parity(RAGGED, _t_grads(sum(RAGGED), 3, seed=22, scale=1e-4), ratio=0.005,
               momentum=0.9, mask=True, fused=True, seed=5, plan=plan,
               label=f"{variant} momentum+mask+int8")
    plan.close()


@pytest.mark.parametrize("variant", VARIANTS)
def test_topk_ties_special_values_and_full_path_against_oracle(variant):
    sizes = [100000, 20003, 5000]
    n = sum(sizes)
    rng = np.random.default_rng(23)
    ties = [rng.integers(-3, 4, n).astype(np.float32) for _ in range(2)]
    special = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    special[::97] = np.float32(1e-41)
    special[::101] = -0.0
    special[7] = np.inf
    plan = _plan(sizes, variant, ratio=0.01)
    run_parity(sizes, ties + [special], ratio=0.01, plan=plan, label=f"{variant} ties+special")
    plan.close()
    plan = _plan(sizes, variant, ratio=0.01, flags=gca.GC_DEBUG_FORCE_FALLBACK)
    run_parity(sizes, _t_grads(n, 2, seed=24), ratio=0.01, plan=plan,
               flags=gca.GC_DEBUG_FORCE_FALLBACK, label=f"{variant} forced full path",
               check_stats=lambda t, st: np.all((st["mode"] == gca.MODE_FULL) |
                                                (st["mode"] == gca.MODE_SMALL)) or
               pytest.fail("forced full path not taken"))
    plan.close()


# ------------------------------------------------- other codecs against the default geometry
def _run_codec(variant, sizes, k, steps, call, state_names):
    """Run outs = call(plan, g, state, t) for every step on the default geometry
    and on `variant`, each from zero state; return the per-step outputs of both."""
    dev = torch.device("cuda")
    n = sum(sizes)
    results = []
    for v in (None, variant):
        plan = _plan(sizes, v, k=k) if k is not None else _plan(sizes, v, ratio=0.01)
        state = {name: torch.zeros(n, dtype=torch.float32, device=dev) for name in state_names}
        per_step = []
        for t, g in enumerate(steps):
            outs = call(plan, torch.from_numpy(g).to(dev), state, t)
            torch.cuda.synchronize()
            per_step.append({**{k_: bits(x) for k_, x in outs.items()},
                             **{f"state.{k_}": bits(x) for k_, x in state.items()}})
        plan.close()
        results.append(per_step)
    return results


def _compare_exact(ref, got, label):
    for t, (a, b) in enumerate(zip(ref, got)):
        for name in a:
            assert_bitwise(b[name], a[name], f"{label} step {t} {name}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_threshold_and_randk_match_default_geometry(variant):
    sizes = RAGGED
    k = [max(1, s // 200) for s in sizes]
    steps = _t_grads(sum(sizes), 3, seed=25)
    dev = torch.device("cuda")
    tk = int(sum(k))
    taus = torch.tensor([0.5, 2.0, 0.0, 1e30, 4.0, 1.5, 3.0, 0.2, 2.5, 5.0, 0.0, 6.0],
                        dtype=torch.float32, device=dev)

    def thr(plan, g, st, t):
        vals = torch.zeros(tk, device=dev)
        idx = torch.zeros(tk, dtype=torch.int32, device=dev)
        cnt = torch.zeros(len(sizes), dtype=torch.int32, device=dev)
        plan.threshold_compress(g, st["e"], taus, vals, idx, cnt, u=st["u"], momentum=0.9)
        return {"vals": vals, "idx": idx, "count": cnt}

    def rk(plan, g, st, t):
        vals = torch.zeros(tk, device=dev)
        idx = torch.zeros(tk, dtype=torch.int32, device=dev)
        plan.randk_compress(g, vals, idx, e=st["e"], seed=77, step=t)
        return {"vals": vals, "idx": idx}

    def rk_unbiased(plan, g, st, t):   # no feedback: values scaled by n / k
        vals = torch.zeros(tk, device=dev)
        idx = torch.zeros(tk, dtype=torch.int32, device=dev)
        plan.randk_compress(g, vals, idx, seed=78, step=t)
        return {"vals": vals, "idx": idx}

    for name, fn, st in (("threshold", thr, ("e", "u")), ("randk", rk, ("e",)),
                         ("randk without feedback", rk_unbiased, ())):
        log(f"[geometry {variant}] {name}")
        ref, got = _run_codec(variant, sizes, k, steps, fn, st)
        _compare_exact(ref, got, f"{variant} {name}")


def _one_ulp_apart(a, b):
    a = a.view(np.int32).astype(np.int64)
    b = b.view(np.int32).astype(np.int64)
    return np.abs(a - b) <= 1


@pytest.mark.parametrize("variant", VARIANTS)
def test_sign_and_qsgd_match_default_geometry(variant):
    sizes = RAGGED
    n = sum(sizes)
    steps = _t_grads(n, 3, seed=26)
    dev = torch.device("cuda")

    def sign(plan, g, st, t):
        words = torch.zeros(max(plan.total_words, 1), dtype=torch.int32, device=dev)
        scales = torch.zeros(len(sizes), device=dev)
        plan.sign_compress(g, st["e"], words, scales)
        return {"scale": scales, "bits": words}

    def qsgd(plan, g, st, t):
        codes = torch.zeros(n, dtype=torch.int8, device=dev)
        norms = torch.zeros(len(sizes), device=dev)
        plan.qsgd_compress(g, codes, norms, levels=127, e=st["e"], u=st["u"], momentum=0.9,
                           seed=3, step=t)
        return {"scale": norms, "codes": codes}

    for name, fn, st in (("sign", sign, ("e",)), ("qsgd", qsgd, ("e", "u"))):
        log(f"[geometry {variant}] {name}")
        ref, got = _run_codec(variant, sizes, None, steps, fn, st)
        for t, (a, b) in enumerate(zip(ref, got)):
            assert _one_ulp_apart(a["scale"], b["scale"]).all(), f"{variant} {name} step {t} scale"
            if not np.array_equal(a["scale"], b["scale"]):
                log(f"[geometry {variant}] {name} step {t}: a scale differs by one ulp; "
                    "later steps not compared")
                break
            for key in a:
                assert_bitwise(b[key], a[key], f"{variant} {name} step {t} {key}")
