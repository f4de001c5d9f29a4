"""The compress calls under HIP graph capture.

A call launches only kernels on the caller's stream (no host round trip, no memset, no
allocation), so it can be recorded once and replayed.  Each replay runs on the graph's fixed
buffers: the test writes a new gradient into the captured input between replays, runs eager
work and synchronisations in between, and checks every replay bit for bit against the CPU
oracle stepping the same residual.
"""
import numpy as np
import pytest
import torch

import gradient_compression_amd as gca
import oracle
from tests.gpu_helpers import assert_bitwise, log

pytestmark = pytest.mark.gpu

SIZES = [1001, 70003, 8192 * 3 + 5, 300001, 4097]
# at k = 1% this plan selects with the chain (its 300001-element segment is past the
# one-workgroup rule); this one with one workgroup per segment
SINGLE_SIZES = [1001, 70003, 8192 * 3 + 5, 200000, 4097]


def _grads(n, iters, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_t(3.0, n)).astype(np.float32) for _ in range(iters)]


@pytest.mark.parametrize("sizes", [SIZES, SINGLE_SIZES], ids=["chain", "single"])
@pytest.mark.parametrize("momentum", [None, 0.9], ids=["plain", "momentum"])
def test_topk_compress_graph_replays(momentum, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, ratio=0.01, flags=gca.GC_MOMENTUM_MASK if momentum else 0)
    dev = torch.device("cuda")
    grads = _grads(n, 6, 31)
    g = torch.from_numpy(grads[0]).to(dev)
    e = torch.zeros(n, device=dev)
    u = torch.zeros(n, device=dev) if momentum else None
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    e_h = np.zeros(n, np.float32)
    u_h = np.zeros(n, np.float32) if momentum else None

    def oracle_step(gh):
        return oracle.topk_ef(gh, e_h, off, plan.k, u=u_h, momentum=momentum or 0.0,
                              mask_u=bool(momentum))

    # eager first call (also the warm-up torch asks for before a capture), on a side stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.compress(g, e, vals, idx, u=u, momentum=momentum or 0.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    hv, hi = oracle_step(grads[0])
    assert_bitwise(idx, hi, "eager idx")
    assert_bitwise(vals, hv, "eager vals")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.compress(g, e, vals, idx, u=u, momentum=momentum or 0.0)
    scratch = torch.zeros(1 << 20, device=dev)
    for t in range(1, 6):
        g.copy_(torch.from_numpy(grads[t]).to(dev))
        scratch.add_(1.0)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[graph] replay {t}")
        hv, hi = oracle_step(grads[t])
        assert_bitwise(idx, hi, f"replay {t} idx")
        assert_bitwise(vals, hv, f"replay {t} vals")
        assert_bitwise(e, e_h, f"replay {t} residual")
        if momentum:
            assert_bitwise(u, u_h, f"replay {t} velocity")
    del graph
    plan.close()


def test_threshold_and_sign_graph_replays():
    off = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int64)
    n = int(off[-1])
    plan = gca.Plan(off, k=[50, 300, 40, 500, 4097])
    dev = torch.device("cuda")
    grads = _grads(n, 4, 32)
    g = torch.from_numpy(grads[0]).to(dev)
    e1 = torch.zeros(n, device=dev)
    e2 = torch.zeros(n, device=dev)
    tau = torch.tensor([0.5, 2.0, 0.0, 4.0, 1.5], device=dev)
    vals = torch.empty(plan.total_k, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(len(SIZES), dtype=torch.int32, device=dev)
    bits = torch.empty(plan.total_words, dtype=torch.int32, device=dev)
    scales = torch.empty(len(SIZES), device=dev)
    h1 = np.zeros(n, np.float32)
    h2 = np.zeros(n, np.float32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up before the capture, outputs not checked
        plan.threshold_compress(g, torch.zeros(n, device=dev), tau, vals, idx, cnt)
        plan.sign_compress(g, torch.zeros(n, device=dev), bits, scales)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.threshold_compress(g, e1, tau, vals, idx, cnt)
        plan.sign_compress(g, e2, bits, scales)
    tau_h = tau.cpu().numpy()
    for t in range(4):
        g.copy_(torch.from_numpy(grads[t]).to(dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[graph] threshold+sign replay {t}")
        c = cnt.cpu().numpy()
        b = bits.cpu().numpy().view(np.uint32)
        for s in range(len(SIZES)):
            a, z = int(off[s]), int(off[s + 1])
            ka = int(plan.out_off[s])
            hv, hi = oracle.threshold_ef_segment(grads[t][a:z].copy(), h1[a:z], int(plan.k[s]),
                                                 float(tau_h[s]))
            assert c[s] == hi.size
            assert_bitwise(idx[ka:ka + hi.size], hi, f"replay {t} seg {s} threshold idx")
            assert_bitwise(vals[ka:ka + hi.size], hv, f"replay {t} seg {s} threshold vals")
            hb, hs = oracle.sign_ef_segment(grads[t][a:z].copy(), h2[a:z])
            wa, wb = int(plan.word_off[s]), int(plan.word_off[s + 1])
            assert_bitwise(b[wa:wb], hb, f"replay {t} seg {s} sign bits")
            # the scale is a double sum in an unspecified order: one ulp, and the residual is
            # exact whenever the scales agree (else the oracle continues from the GPU's)
            sd = float(scales[s])
            assert abs(sd - float(hs)) <= float(np.spacing(np.float32(abs(hs))))
            if sd == hs:
                assert_bitwise(e2[a:z], h2[a:z], f"replay {t} seg {s} sign residual")
            else:
                h2[a:z] = e2[a:z].cpu().numpy()
        assert_bitwise(e1, h1, f"replay {t} threshold residual")
    del graph
    plan.close()
