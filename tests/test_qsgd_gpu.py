"""GPU parity of the QSGD codec (C ABI) against the CPU oracle.

Codes are compared bit for bit whenever the segment's norm matches the oracle's; the norm
(a double sum of squares in an unspecified order, rounded once) must be within one ulp by definition,
and the tests require it to be equal (a one-ulp difference would be a one-in-a-million event).
"""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from synth import gen, workload
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu


def ulp(x):
    return float(np.spacing(np.float32(abs(x))))


def run_qsgd(sizes, grads, levels, ef=True, momentum=None, seed=3, label=""):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, k=0)
    dev = torch.device("cuda")
    e_d = torch.zeros(n, device=dev) if ef else None
    e_h = np.zeros(n, np.float32) if ef else None
    u_d = torch.zeros(n, device=dev) if momentum is not None else None
    u_h = np.zeros(n, np.float32) if momentum is not None else None
    codes = torch.empty(max(n, 4), dtype=torch.int8, device=dev)
    norms = torch.empty(max(len(sizes), 1), device=dev)
    mism = 0
    for t, g in enumerate(grads):
        log(f"[qsgd {label}] iteration {t}")
        plan.qsgd_compress(torch.from_numpy(g).to(dev), codes, norms, levels=levels, e=e_d,
                           u=u_d, momentum=momentum or 0.0, seed=seed, step=t)
        torch.cuda.synchronize()
        c_d, n_d = codes.cpu().numpy(), norms.cpu().numpy()
        for s in range(len(sizes)):
            a, b = int(off[s]), int(off[s + 1])
            hc, hn = oracle.qsgd_segment(g[a:b].copy(), None if e_h is None else e_h[a:b],
                                         None if u_h is None else u_h[a:b], momentum or 0.0,
                                         levels, seed, t, a)
            assert abs(float(n_d[s]) - float(hn)) <= ulp(hn), f"{label} it{t} seg{s} norm"
            if n_d[s] == hn:
                assert_bitwise(c_d[a:b], hc, f"{label} it{t} seg{s} codes")
                if e_h is not None:
                    assert_bitwise(e_d[a:b], e_h[a:b], f"{label} it{t} seg{s} residual")
            else:
                mism += 1
                if e_h is not None:
                    e_h[a:b] = e_d[a:b].cpu().numpy()
        if u_h is not None:
            assert_bitwise(u_d, u_h, f"{label} it{t} velocity")
    plan.close()
    # One ulp is allowed by the definition, but the two double sums differ by about 1e-13
    # relative, so a norm on the other side of an fp32 rounding boundary has odds near 1e-6
    # per segment: any difference is treated as a failure, so that a drift cannot hide.
    assert mism == 0, f"{label}: {mism} norms differed from the oracle's by one ulp"
    return mism


def grads(n, T, seed, scale=1e-3):
    rng = np.random.default_rng(seed)
    return [(rng.standard_t(3, n) * scale).astype(np.float32) for _ in range(T)]


SIZES = [1, 33, 4095, 8192, 8193, 100003, 262144, 0, 7]


@pytest.mark.parametrize("levels", [1, 7, 127])
def test_qsgd_error_feedback(levels):
    log(f"norm mismatches: {run_qsgd(SIZES, grads(sum(SIZES), 3, levels), levels, label=f's={levels}')}")


@pytest.mark.parametrize("momentum", [None, 0.9])
def test_qsgd_without_feedback(momentum):
    run_qsgd(SIZES, grads(sum(SIZES), 3, 11), 15, ef=False, momentum=momentum,
             label=f"noef m={momentum}")


def test_qsgd_feedback_with_momentum():
    run_qsgd([4096, 40000, 11008 * 3], grads(4096 + 40000 + 33024, 3, 12, 1e-4), 127,
             momentum=0.9, label="ef+momentum")


def test_qsgd_decompress():
    sizes = [1000, 37, 8192 * 3 + 1]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, k=0)
    g = grads(n, 1, 5)[0]
    codes = torch.empty(n, dtype=torch.int8, device="cuda")
    norms = torch.empty(len(sizes), device="cuda")
    plan.qsgd_compress(torch.from_numpy(g).cuda(), codes, norms, levels=31, seed=1)
    c_h, n_h = codes.cpu().numpy(), norms.cpu().numpy()
    base = np.random.default_rng(6).standard_normal(n).astype(np.float32)
    for acc in (False, True):
        dense = torch.from_numpy(base).cuda()
        plan.qsgd_decompress(codes, norms, dense, levels=31, accumulate=acc)
        want = base.copy()
        for s in range(len(sizes)):
            a, b = int(off[s]), int(off[s + 1])
            want[a:b] = oracle.qsgd_decompress_segment(c_h[a:b], n_h[s], 31,
                                                       dense=want[a:b].copy(), accumulate=acc)
        assert dense.cpu().numpy().tobytes() == want.tobytes()
    plan.close()


def test_qsgd_full_size_bert_large():
    """BERT-large shape at full size with error feedback, s = 127: sampled segments against
    the oracle; every segment's norm against a torch fp64 norm (one ulp) and its codes within
    {floor(a), ceil(a)} with the residual exact."""
    wl = workload("c3_bert_large")
    off = wl.offsets()
    dev = torch.device("cuda")
    plan = gca.Plan(off, k=0)
    g = torch.empty(wl.n, device=dev)
    e = torch.zeros(wl.n, device=dev)
    codes = torch.empty(wl.n, dtype=torch.int8, device=dev)
    norms = torch.empty(wl.n_seg, device=dev)
    sample = [0, 4, 100, 390]
    host = {s: np.zeros(int(off[s + 1] - off[s]), np.float32) for s in sample}
    for t in range(2):
        gen.fill_gradient(g, wl, t)
        e_prev = e.clone()
        plan.qsgd_compress(g, codes, norms, levels=127, e=e, seed=9, step=t)
        torch.cuda.synchronize()
        log(f"[qsgd full] it{t}")
        nn = norms.cpu().numpy()
        for s in range(wl.n_seg):
            a, b = int(off[s]), int(off[s + 1])
            acc = torch.add(e_prev[a:b], g[a:b])
            want = float(torch.sqrt(acc.double().pow(2).sum()).item())
            assert abs(float(nn[s]) - want) <= ulp(want) * 1.01, f"norm seg {s}"
            # IEEE division on the host: torch divides by a scalar through its reciprocal
            step = float(np.float32(nn[s]) / np.float32(127.0))
            aa = torch.clamp(acc.abs().double() / step, max=127.0)
            q = codes[a:b].to(torch.float64).abs()
            assert bool(((q >= torch.floor(aa) - 1e-9) & (q <= torch.ceil(aa) + 1e-9)).all()), \
                f"codes seg {s}"
            deq = torch.mul(codes[a:b].to(torch.float32), step)
            assert torch.equal(torch.sub(acc, deq).view(torch.int32), e[a:b].view(torch.int32))
        for s in sample:
            a, b = int(off[s]), int(off[s + 1])
            hc, hn = oracle.qsgd_segment(g[a:b].cpu().numpy(), host[s], levels=127, seed=9, step=t,
                                         seg_base=a)
            assert nn[s] == hn, f"seg{s} norm differs from the oracle's by one ulp"
            assert_bitwise(codes[a:b], hc, f"seg{s} codes")
            assert_bitwise(e[a:b], host[s], f"seg{s} residual")
        del e_prev
    plan.close()
