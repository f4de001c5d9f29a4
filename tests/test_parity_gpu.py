"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for bit, on
seeded inputs at sizes the oracle finishes in seconds; every case spans several tiles of
8192 and ragged tails, and the edge cases of the method."""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from synth import gen, workload
from tests.gpu_helpers import assert_bitwise, log, run_parity

pytestmark = pytest.mark.gpu


def t_grads(n, iters, df=3.0, scale=1e-3, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(iters):
        yield (rng.standard_t(df, n) * scale).astype(np.float32)


def synth_grads(wl, iters, device="cpu"):
    buf = torch.empty(wl.n, dtype=torch.float32, device=device)
    for t in range(iters):
        gen.fill_gradient(buf, wl, t)
        yield buf.cpu().numpy().copy()


def test_single_segment_c1_full():
    """2^20 elements, k = 1049, 5 EF iterations of 1e-3 * t(3) (the first workload, full size)."""
    wl = workload("c1_single_1m")
    modes = []
    run_parity(wl.sizes, synth_grads(wl, wl.iters, "cuda"), ratio=wl.ratio, label="c1",
               check_stats=lambda t, st: modes.append(int(st["mode"][0])))
    log(f"c1 modes per iteration: {modes}")
    # a fresh plan starts from the threshold its tile sample suggests
    assert all(m == gca.MODE_CANDIDATES for m in modes), modes


RAGGED = [1, 3, 64, 4095, 8192, 8193, 70001, 123457, 300001, 2, 65536, 65537]


@pytest.mark.parametrize("ratio", [0.001, 0.01, 0.1])
def test_ragged_misaligned_segments(ratio):
    n = sum(RAGGED)
    run_parity(RAGGED, t_grads(n, 4, seed=int(ratio * 1000)), ratio=ratio,
               label=f"ragged r={ratio}")


def test_explicit_k_zero_one_and_all():
    sizes = [100000, 100000, 100000, 9000, 77777]
    k = [0, 1, 100000, 9000, 0]
    run_parity(sizes, t_grads(sum(sizes), 3, seed=5), k=k, label="k edge")


def test_tie_heavy_integer_gradients():
    sizes = [100000, 200003, 5000]
    rng = np.random.default_rng(11)
    grads = [rng.integers(-3, 4, sum(sizes)).astype(np.float32) for _ in range(4)]
    run_parity(sizes, grads, ratio=0.01, label="ties")


def test_all_zero_and_constant_segments():
    sizes = [150000, 150000, 70000]
    n = sum(sizes)
    g0 = np.zeros(n, np.float32)
    g1 = np.zeros(n, np.float32)
    g1[150000:300000] = -0.0
    g1[300000:] = 2.5
    seen = []
    run_parity(sizes, [g0, g1, g0], ratio=0.01, label="zeros",
               check_stats=lambda t, st: seen.append(st["mode"].tolist()))
    # every key ties at 0 (or 2.5): the tied bucket exceeds the candidate capacity, so the
    # radix select runs over the whole segment
    assert seen[0] == [gca.MODE_FULL] * 3


def test_special_values():
    sizes = [90000, 17, 40000]
    n = sum(sizes)
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[::97] = np.float32(1e-41)                 # denormals
    g[::101] = -0.0
    g[5] = np.inf
    g[90003] = -np.inf
    g2 = (rng.standard_normal(n) * 1e-38).astype(np.float32)   # denormal sums
    run_parity(sizes, [g, g2, g2], ratio=0.01, label="special")


@pytest.mark.parametrize("mask", [False, True])
def test_momentum_correction(mask):
    sizes = [4096, 4096 * 40, 11008 * 20, 4096]
    run_parity(sizes, t_grads(sum(sizes), 4, scale=1e-4, seed=7), ratio=0.001, momentum=0.9,
               mask=mask, label=f"momentum mask={mask}")


def _forced_modes(sizes):
    """The modes a forced full path gives: the full path, except small segments, which are
    always selected whole by one workgroup."""
    return [gca.MODE_SMALL if n <= gca.SMALL_SEGMENT else gca.MODE_FULL for n in sizes]


def test_forced_fallback_matches():
    sizes = [300000, 8192 * 5 + 3, 999, 70001]
    run_parity(sizes, t_grads(sum(sizes), 3, seed=9), ratio=0.01,
               flags=gca.GC_DEBUG_FORCE_FALLBACK, label="forced full path",
               check_stats=lambda t, st: st["mode"].tolist() == _forced_modes(sizes) or
               pytest.fail(f"forced full path not taken: {st['mode']}"))


def _many_sizes(n_seg, seed):
    """Mostly tiny segments, some below and some above a tile, a few large ones."""
    rng = np.random.default_rng(seed)
    kind = rng.choice(4, n_seg, p=[0.6, 0.3, 0.09, 0.01])
    lo = np.array([0, 64, 9000, 70000])[kind]
    hi = np.array([64, 9000, 70000, 300000])[kind]
    return [int(x) for x in rng.integers(lo, hi)]


def test_thousands_of_segments():
    """3000 segments (including empty ones) in one plan, k = 1%, three EF steps."""
    sizes = _many_sizes(3000, 41)
    log(f"many segments: n_seg={len(sizes)} n={sum(sizes)} empty={sizes.count(0)}")
    run_parity(sizes, t_grads(sum(sizes), 3, seed=42), ratio=0.01, label="3000 segments")


def test_thousands_of_segments_full_path():
    """Every one of 800 segments on the exact full path at once (its workgroups walk the
    whole list of full-path segments)."""
    sizes = _many_sizes(800, 43)
    run_parity(sizes, t_grads(sum(sizes), 2, seed=44), ratio=0.01,
               flags=gca.GC_DEBUG_FORCE_FALLBACK, label="800 segments, full path")


# These plans are modest enough for the one-workgroup-per-segment select; GC_DEBUG_CHAIN runs
# the chain of kernels instead.  Both must give the oracle's results; their paths differ: an
# incomplete capture is re-captured by the chain's fallback kernels (MODE_RECAPTURED) and
# selected over the whole segment by the segment's workgroup (MODE_FULL).
PATHS = pytest.mark.parametrize("chain", [True, False], ids=["chain", "single"])


def _fallback_mode(chain):
    return gca.MODE_RECAPTURED if chain else gca.MODE_FULL


@PATHS
def test_no_estimate_recaptures_every_call(chain):
    sizes = [200000, 20000, 8192 * 9 + 5]   # every segment allows the one-workgroup select
    seen = []
    run_parity(sizes, t_grads(sum(sizes), 3, seed=19), ratio=0.01,
               flags=gca.GC_DEBUG_NO_ESTIMATE | (gca.GC_DEBUG_CHAIN if chain else 0),
               label=f"no estimate chain={chain}",
               check_stats=lambda t, st: seen.append(st["mode"].tolist()))
    # no threshold is kept: every large segment takes the fallback on every call (a small one
    # is selected whole, as always)
    want = [gca.MODE_SMALL if n <= gca.SMALL_SEGMENT else _fallback_mode(chain) for n in sizes]
    assert all(m == want for m in seen), seen


@PATHS
def test_estimate_miss_and_overflow_fall_back(chain):
    """acc far smaller than at the last call (the threshold is too high: fewer than k
    candidates) and then far larger (more candidates than the capacity) must still give
    exact results, through the full-segment path."""
    sizes = [400000, 300000]
    n = sum(sizes)
    rng = np.random.default_rng(13)

    def grad(t, resid):
        noise = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
        if t == 2:      # cancel the residual: acc ~ 1e-9 * t(3)
            return (-resid + noise * np.float32(1e-6)).astype(np.float32)
        if t == 4:      # acc ~ 1e3 * t(3): far more than 16 k candidates
            return noise * np.float32(1e6)
        return noise

    seen = []
    run_parity(sizes, (6, grad), ratio=0.001, flags=gca.GC_DEBUG_CHAIN if chain else 0,
               label=f"miss/overflow chain={chain}",
               check_stats=lambda t, st: seen.append(st["mode"].tolist()))
    log(f"modes: {seen}")
    assert seen[0] == [gca.MODE_CANDIDATES] * 2        # fresh plan: the sampled estimate
    assert seen[1] == [gca.MODE_CANDIDATES] * 2
    assert seen[2] == [_fallback_mode(chain)] * 2      # too few candidates
    assert seen[4] == [_fallback_mode(chain)] * 2      # too many candidates


# Segment sizes per ratio that every segment of the plan allows the one-workgroup select for
# (at most 2^22 elements, and 4 k <= 8192 or at most 65536 elements; small ones always).
SINGLE_SIZES = {0.001: [1 << 20, 300007, 16384, 65536 + 17, 9000],
                0.01: [200000, 50000, 16384, 65536 + 17, 9000],
                0.1: [65536, 20000, 16385, 60000, 9000]}


@pytest.mark.parametrize("ratio", sorted(SINGLE_SIZES))
def test_single_and_chain_agree(ratio):
    """The same plan selected by one workgroup per segment and by the chain of kernels:
    bit-identical outputs and state on every step (ties, ragged tiles, small segments, and at
    10% segments captured whole, more candidates than one chunk)."""
    sizes = SINGLE_SIZES[ratio]
    n = sum(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rng = np.random.default_rng(23)
    grads = [(np.round(rng.standard_t(3, n) * 8.0) / 8.0 * 1e-3).astype(np.float32)
             for _ in range(4)]
    plans = [gca.Plan(off, ratio=ratio), gca.Plan(off, ratio=ratio, flags=gca.GC_DEBUG_CHAIN)]
    es = [torch.zeros(n, device="cuda") for _ in plans]
    outs = [(torch.empty(plans[0].total_k, device="cuda"),
             torch.empty(plans[0].total_k, dtype=torch.int32, device="cuda")) for _ in plans]
    for t, g in enumerate(grads):
        gd = torch.from_numpy(g).cuda()
        for p, e, (v, i) in zip(plans, es, outs):
            p.compress(gd, e, v, i)
        torch.cuda.synchronize()
        modes = [p.last_stats()["mode"].tolist() for p in plans]
        log(f"[single/chain ratio={ratio}] step {t}: modes {modes}")
        assert_bitwise(outs[0][1], outs[1][1].cpu().numpy(), f"step {t} idx")
        assert_bitwise(outs[0][0], outs[1][0].cpu().numpy(), f"step {t} vals")
        assert_bitwise(es[0], es[1].cpu().numpy(), f"step {t} residual")
    for p in plans:
        p.close()


def test_warm_and_cold_plans_agree():
    sizes = [200000, 50000]
    n = sum(sizes)
    grads = list(t_grads(n, 4, seed=21))
    off = np.array([0, 200000, n], np.int64)
    cold = gca.Plan(off, ratio=0.01)
    outs = []
    for reset in (False, True):
        e = torch.zeros(n, device="cuda")
        v = torch.empty(cold.total_k, device="cuda")
        i = torch.empty(cold.total_k, dtype=torch.int32, device="cuda")
        res = []
        for g in grads:
            if reset:
                cold.reset_estimate()
            cold.compress(torch.from_numpy(g).cuda(), e, v, i)
            res.append((v.cpu().numpy().copy(), i.cpu().numpy().copy(), e.cpu().numpy().copy()))
        outs.append(res)
    for a, b in zip(*outs):
        for x, y in zip(a, b):
            assert x.tobytes() == y.tobytes()


def test_hybrid_int8():
    """Top-k then int8 with stochastic rounding and error feedback of the quantisation
    error: 4 segments of 2^20, t(2.5), k = 1%, seed 0 (the hybrid workload, scaled down)."""
    sizes = [1 << 20] * 4
    run_parity(sizes, t_grads(sum(sizes), 3, df=2.5, scale=1.0, seed=4), ratio=0.01, int8=True,
               seed=0, label="int8")
    run_parity([1 << 16, 3, 77], t_grads((1 << 16) + 80, 2, seed=6), ratio=0.05, int8=True,
               seed=12345678901, label="int8 seed")


@pytest.mark.parametrize("flags,momentum,mask,with_vals", [
    (0, None, False, True),
    (0, None, False, False),
    (0x100, None, False, True),          # full-segment path
    (0x200, None, False, True),          # re-capture path
    (0, 0.9, True, True),                # momentum with masking
])
def test_fused_compress_int8(flags, momentum, mask, with_vals):
    """The fused call equals compress then int8 with error feedback of the quantisation error
    (checked against the oracle's two steps); every selection path, with and without values."""
    sizes = [1 << 18, 70001, 3, 0, 9000]
    run_parity(sizes, t_grads(sum(sizes), 3, df=2.5, scale=1.0, seed=8), ratio=0.01, fused=True,
               with_vals=with_vals, flags=flags, momentum=momentum, mask=mask, seed=77,
               label=f"fused f={flags:#x} m={momentum} mask={mask} vals={with_vals}")


def test_decompress_matches_oracle():
    import oracle
    sizes = [100000, 3, 54321]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, ratio=0.01)
    g = next(t_grads(n, 1, seed=2))
    e_h = np.zeros(n, np.float32)
    vals_o, idx_o = oracle.topk_ef(g, e_h, off, plan.k)
    codes_o, scales_o = oracle.quant_int8(vals_o, idx_o, off, plan.k, seed=1, step=0)
    vals = torch.from_numpy(vals_o).cuda()
    idx = torch.from_numpy(idx_o).cuda()
    codes = torch.from_numpy(codes_o).cuda()
    scales = torch.from_numpy(scales_o).cuda()
    base = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    for accumulate in (False, True):
        dense = torch.from_numpy(base).cuda()
        plan.decompress(idx, dense, vals=vals, accumulate=accumulate)
        want = oracle.decompress(off, plan.k, idx_o, vals=vals_o, dense=base.copy(),
                                 accumulate=accumulate)
        assert dense.cpu().numpy().tobytes() == want.tobytes()
        dense = torch.from_numpy(base).cuda()
        plan.decompress(idx, dense, codes=codes, scales=scales, accumulate=accumulate)
        want = oracle.decompress(off, plan.k, idx_o, codes=codes_o, scales=scales_o,
                                 dense=base.copy(), accumulate=accumulate)
        assert dense.cpu().numpy().tobytes() == want.tobytes()
    plan.close()


def test_empty_plan_and_empty_segments():
    plan = gca.Plan(np.array([0], np.int64), k=[])
    assert plan.total_k == 0
    plan.compress(torch.zeros(4, device="cuda"), torch.zeros(4, device="cuda"), None, None)
    plan.close()
    run_parity([0, 10, 0, 20000, 0], t_grads(20010, 2, seed=3), ratio=0.01, label="empty segs")


def test_argument_errors_on_gpu():
    off = np.array([0, 1000], np.int64)
    plan = gca.Plan(off, ratio=0.01)
    g = torch.zeros(1000, device="cuda")
    e = torch.zeros(1000, device="cuda")
    v = torch.empty(10, device="cuda")
    i = torch.empty(10, dtype=torch.int32, device="cuda")
    with pytest.raises(gca.GCError):          # misaligned g
        plan.compress(torch.zeros(1001, device="cuda")[1:], e, v, i)
    with pytest.raises(gca.GCError):          # g aliases e
        plan.compress(e, e, v, i)
    buf = torch.zeros(2000, device="cuda")
    with pytest.raises(gca.GCError):          # g and e overlap in part
        plan.compress(buf[:1000], buf[4:1004], v, i)
    with pytest.raises(gca.GCError):          # the output values lie inside e
        plan.compress(g, buf[:1000], buf[500:510], i)
    with pytest.raises(gca.GCError):          # the output indices lie inside g
        plan.compress(buf[:1000], e, v, buf[100:110].view(torch.int32))
    dense = torch.zeros(1000, device="cuda")
    with pytest.raises(gca.GCError):          # decompression into its own input
        plan.decompress(i, dense, vals=dense[:10])
    plan.compress(buf[:1000], buf[1000:], v, i)   # disjoint views of one buffer are fine
    plan.compress(g, e, v, i)
    plan.decompress(i, dense, vals=v)
    torch.cuda.synchronize()
    plan.close()


def test_workspace_out_of_memory_and_unsupported_size_are_reported():
    """A plan whose workspace does not fit in what the device has left fails with
    GC_ERR_OOM; one whose candidate buffers would pass the library's 32-bit chunk addressing
    (64 segments of 2^31 - 1 elements with k = n) fails with GC_ERR_UNSUPPORTED before any
    allocation.  The library and the device stay usable afterwards."""
    n_s = 2 ** 31 - 1
    with pytest.raises(gca.GCError) as err:
        gca.Plan(np.arange(65, dtype=np.int64) * n_s, ratio=1.0)
    assert err.value.status == gca.GC_ERR_UNSUPPORTED, err.value
    free, _ = torch.cuda.mem_get_info()
    hold = torch.empty(max(free - (8 << 30), 0), dtype=torch.uint8, device="cuda")
    try:
        # one segment with k = n: candidate buffers of 16 B per element, about 34 GB
        with pytest.raises(gca.GCError) as err:
            gca.Plan(np.array([0, n_s], np.int64), ratio=1.0)
        assert err.value.status == gca.GC_ERR_OOM, err.value
    finally:
        del hold
        torch.cuda.empty_cache()
    sizes = [30000, 4097]
    run_parity(sizes, t_grads(sum(sizes), 2, seed=13), ratio=0.01, label="after OOM")


def test_checkpoint_resume_matches_straight_run():
    """The error-feedback state is e (and u): five steps straight equal three steps, a
    save and restore of e and u into fresh buffers (and a fresh plan), then two steps."""
    sizes = [120000, 4096, 77777]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    grads = [torch.from_numpy(g).cuda() for g in t_grads(n, 5, scale=1e-4, seed=31)]

    def run(plan, e, u, gs):
        outs = []
        for g in gs:
            v = torch.empty(plan.total_k, device="cuda")
            i = torch.empty(plan.total_k, dtype=torch.int32, device="cuda")
            plan.compress(g, e, v, i, u=u, momentum=0.9)
            outs.append((v.cpu().numpy(), i.cpu().numpy()))
        return outs

    p1 = gca.Plan(off, ratio=0.01)
    e1, u1 = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    straight = run(p1, e1, u1, grads)
    p2 = gca.Plan(off, ratio=0.01)
    e2, u2 = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    first = run(p2, e2, u2, grads[:3])
    saved = (e2.cpu().numpy().copy(), u2.cpu().numpy().copy())
    p2.close()
    p3 = gca.Plan(off, ratio=0.01)
    e3, u3 = torch.from_numpy(saved[0]).cuda(), torch.from_numpy(saved[1]).cuda()
    rest = run(p3, e3, u3, grads[3:])
    for (a, b), (c, d) in zip(straight, first + rest):
        assert a.tobytes() == c.tobytes() and b.tobytes() == d.tobytes()
    assert e1.cpu().numpy().tobytes() == e3.cpu().numpy().tobytes()
    assert u1.cpu().numpy().tobytes() == u3.cpu().numpy().tobytes()


def test_side_stream_and_interleaved_plans():
    """Calls run in order on the stream they are given; two plans over different segment
    tables interleave without sharing state."""
    import oracle
    sizes_a, sizes_b = [100000, 3000], [50000, 50000, 7]
    off_a = np.concatenate([[0], np.cumsum(sizes_a)]).astype(np.int64)
    off_b = np.concatenate([[0], np.cumsum(sizes_b)]).astype(np.int64)
    pa, pb = gca.Plan(off_a, ratio=0.01), gca.Plan(off_b, ratio=0.002)
    ka = np.array([oracle.k_from_ratio(s, 0.01) for s in sizes_a], np.int64)
    kb = np.array([oracle.k_from_ratio(s, 0.002) for s in sizes_b], np.int64)
    ga = list(t_grads(int(off_a[-1]), 3, seed=41))
    gb = list(t_grads(int(off_b[-1]), 3, seed=42))
    side = torch.cuda.Stream()
    ea, eb = torch.zeros(int(off_a[-1]), device="cuda"), torch.zeros(int(off_b[-1]), device="cuda")
    ea_h, eb_h = np.zeros(int(off_a[-1]), np.float32), np.zeros(int(off_b[-1]), np.float32)
    va, ia = torch.empty(pa.total_k, device="cuda"), torch.empty(pa.total_k, dtype=torch.int32, device="cuda")
    vb, ib = torch.empty(pb.total_k, device="cuda"), torch.empty(pb.total_k, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for t in range(3):
        with torch.cuda.stream(side):
            gda = torch.from_numpy(ga[t]).to("cuda", non_blocking=False)
            gdb = torch.from_numpy(gb[t]).to("cuda", non_blocking=False)
            pa.compress(gda, ea, va, ia, stream=side)
            pb.compress(gdb, eb, vb, ib, stream=side)
        side.synchronize()
        vo, io = oracle.topk_ef(ga[t], ea_h, off_a, ka)
        assert va.cpu().numpy().tobytes() == vo.tobytes() and np.array_equal(ia.cpu().numpy(), io)
        vo, io = oracle.topk_ef(gb[t], eb_h, off_b, kb)
        assert vb.cpu().numpy().tobytes() == vo.tobytes() and np.array_equal(ib.cpu().numpy(), io)
    assert ea.cpu().numpy().tobytes() == ea_h.tobytes()
    assert eb.cpu().numpy().tobytes() == eb_h.tobytes()


def test_cold_plan_starts_from_a_sampled_threshold():
    """A fresh plan (and one after reset_estimate) samples tiles of each large segment for its
    first threshold: on the BERT-large shape (without the sample 147 of 391 segments had to
    re-capture on a cold call) at least 90% of the segments stay on the candidate path from
    the first call, and the result is exact either way (the oracle, sampled segments)."""
    wl = workload("c3_bert_large")
    off = wl.offsets()
    plan = gca.Plan(off, ratio=wl.ratio)
    g = torch.empty(wl.n, device="cuda")
    e = torch.zeros(wl.n, device="cuda")
    vals = torch.empty(plan.total_k, device="cuda")
    idx = torch.empty(plan.total_k, dtype=torch.int32, device="cuda")
    sample = [0, 4, 100, 390]
    host = {s: np.zeros(int(off[s + 1] - off[s]), np.float32) for s in sample}
    for t in range(2):
        if t == 1:
            plan.reset_estimate()
        gen.fill_gradient(g, wl, t)
        plan.compress(g, e, vals, idx)
        torch.cuda.synchronize()
        st = plan.last_stats()
        modes = st["mode"]
        on_path = (modes == gca.MODE_CANDIDATES) | (modes == gca.MODE_SMALL)
        off_path = int((~on_path).sum())
        bad = np.flatnonzero(~on_path)
        log(f"[cold] call {t}: {off_path} of {wl.n_seg} segments off the candidate path: "
            f"{[(int(s), int(off[s + 1] - off[s]), int(plan.k[s])) for s in bad[:8]]}")
        assert off_path <= wl.n_seg // 10
        for s in sample:
            a, b = int(off[s]), int(off[s + 1])
            ka, kb = int(plan.out_off[s]), int(plan.out_off[s + 1])
            hv, hi = oracle.topk_ef_segment(g[a:b].cpu().numpy(), host[s], int(plan.k[s]))
            assert_bitwise(idx[ka:kb], hi, f"cold call {t} seg {s} idx")
            assert_bitwise(vals[ka:kb], hv, f"cold call {t} seg {s} vals")
            assert_bitwise(e[a:b], host[s], f"cold call {t} seg {s} residual")
    plan.close()


def test_calibration_kernels_match_torch():
    """The bandwidth references the bench reports: the copy and the y += x stream give the
    bytes torch's own copy and fp32 add give (whole tiles and a ragged tail)."""
    n = 8192 * 37 + 12
    rng = np.random.default_rng(31)
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    y0 = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    y = y0.clone()
    gca.add_f32(x, y)
    dst = torch.empty_like(x)
    gca.copy_f32(x, dst)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), torch.add(y0, x).view(torch.int32))
    assert torch.equal(dst.view(torch.int32), x.view(torch.int32))
    with pytest.raises(gca.GCError):          # x and y overlap
        gca.add_f32(y[:100], y[52:152])


def test_two_plans_on_two_streams_concurrently():
    """Two plans (one that selects with one workgroup per segment, one on the chain) called
    alternately on two streams with no synchronisation between their calls: each keeps its own
    state, and every call is bit-exact against the oracle."""
    rng = np.random.default_rng(1212)
    cases = [([300007, 20000, 9000], 0.001), ([400003, 70001, 5000], 0.01)]
    dev = torch.device("cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for sizes, ratio in cases:
        off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        n = int(off[-1])
        plan = gca.Plan(off, ratio=ratio)
        grads = [(rng.standard_t(3, n) * 1e-3).astype(np.float32) for _ in range(4)]
        runs.append(dict(off=off, plan=plan, grads=grads,
                         g=[torch.from_numpy(x).to(dev) for x in grads],
                         e=torch.zeros(n, device=dev), e_h=np.zeros(n, np.float32),
                         vals=[torch.empty(plan.total_k, device=dev) for _ in grads],
                         idx=[torch.empty(plan.total_k, dtype=torch.int32, device=dev)
                              for _ in grads]))
    torch.cuda.synchronize()
    for t in range(4):
        for r, st in zip(runs, streams):
            with torch.cuda.stream(st):
                r["plan"].compress(r["g"][t], r["e"], r["vals"][t], r["idx"][t])
    torch.cuda.synchronize()
    for j, r in enumerate(runs):
        for t in range(4):
            hv, hi = oracle.topk_ef(r["grads"][t], r["e_h"], r["off"], r["plan"].k)
            assert_bitwise(r["idx"][t], hi, f"plan {j} call {t} idx")
            assert_bitwise(r["vals"][t], hv, f"plan {j} call {t} vals")
        assert_bitwise(r["e"], r["e_h"], f"plan {j} residual")
        r["plan"].close()
