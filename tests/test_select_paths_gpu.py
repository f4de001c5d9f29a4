"""GPU parity of the select's sub-paths, each forced by the shape of the data, bit for bit
against the CPU oracle over several EF steps (and every segment's path checked where the
plan's statistics show it).

After the streaming pass a candidate segment's k-th key is found in the *near list*: the
candidates whose keys fall in the bin of 2^13 keys (of a 2048-bin histogram that starts at
the capture floor and spans two binades, the top bin open upwards) that holds the k-th key.
The finish kernel then ranks the near list by counting when it has at most 256 keys, runs
LDS histogram passes over it when it has at most 4096, and otherwise narrows it with
histogram passes over global memory first.  Segments of at most 16384 elements skip all of
this: they are selected whole from the residual in the emission launch.

The data here set those sizes on purpose: a cluster of m magnitudes within 2e-4 of 1.0 (a
span of about 1700 keys, inside one or two bins), on a ~1e-3 background, with k inside the
cluster.  Each step's gradient is drawn so that acc = e + g is the designed vector whatever
the residual (g = target - e), the oracle then defines the exact result.
"""
import numpy as np
import pytest

import gradient_compression_amd as gca
from tests.gpu_helpers import log, run_parity

pytestmark = pytest.mark.gpu

N = 1 << 20


def _cluster(rng, n, m, grid=False):
    """Background N(0, 1e-3^2), plus m positions at magnitude 1 + U(0, 2e-4) with random
    signs (grid: on a 256-value grid 2^-22 apart, so that many of them tie)."""
    a = rng.normal(0.0, 1e-3, n)
    pos = rng.choice(n, m, replace=False)
    if grid:
        mag = 1.0 + rng.integers(0, 256, m) * 2.0 ** -22
    else:
        mag = 1.0 + rng.uniform(0.0, 2e-4, m)
    a[pos] = mag * rng.choice([-1.0, 1.0], m)
    return a


def _target_grads(targets):
    """(iters, f) for run_parity: step t's gradient makes acc equal targets[t] (to within the
    rounding of g = target - e)."""
    def f(t, resid):
        return (targets[t].astype(np.float64) - resid.astype(np.float64)).astype(np.float32)
    return len(targets), f


def test_near_list_size_classes():
    """Three segments whose near lists are about 200 keys (counting ranks), about 3000 (LDS
    histogram passes) and about 40000 (narrowed over global memory first), the k-th key in
    the middle of each cluster so that either side of a bin boundary keeps the class."""
    rng = np.random.default_rng(101)
    ms, ks = [200, 3000, 40000], [100, 1500, 20000]
    iters = 4
    targets = [np.concatenate([_cluster(rng, N, m) for m in ms]) for _ in range(iters)]
    seen = []
    run_parity([N] * 3, _target_grads(targets), k=ks, label="near-classes",
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist())))
    log(f"modes/candidates: {seen}")
    for modes, cands in seen[1:]:   # warm calls: every segment on the candidate path
        assert modes == [gca.MODE_CANDIDATES] * 3
        assert all(c >= k for c, k in zip(cands, ks))


def test_near_list_ties():
    """The same three classes with the cluster on a grid of 256 magnitudes: hundreds of
    entries tie at the k-th key, in a ranked list, in an LDS list and in a narrowed one (which
    may narrow down to the single tied value)."""
    rng = np.random.default_rng(202)
    ms, ks = [230, 3500, 50000], [117, 1711, 24999]
    iters = 3
    targets = [np.concatenate([_cluster(rng, N, m, grid=True) for m in ms])
               for _ in range(iters)]
    seen = []
    run_parity([N] * 3, _target_grads(targets), k=ks, label="near-ties",
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["ties"].tolist())))
    log(f"modes/ties: {seen}")
    for modes, ties in seen[1:]:
        assert modes == [gca.MODE_CANDIDATES] * 3
    assert any(t > 1 for _, ties in seen for t in ties), "the grid gave no ties at the k-th key"


@pytest.mark.parametrize("grid", [False, True], ids=["distinct", "ties"])
@pytest.mark.parametrize("chain", [False, True], ids=["single", "chain"])
def test_near_list_classes_both_paths(chain, grid):
    """Segments of 2^20 with k = 100, 1500 and 2000 (a plan the single-workgroup select
    takes, or with GC_DEBUG_CHAIN the chain): near lists of about 200 keys (ranked), 3000
    (LDS passes) and 40000 (narrowed first; on the single path the candidates span five
    chunks and are read from the candidate buffer), optionally with the cluster on a grid of
    256 magnitudes so that hundreds of entries tie at the k-th key."""
    rng = np.random.default_rng(707)
    ms, ks = [200, 3000, 40000], [100, 1500, 2000]
    targets = [np.concatenate([_cluster(rng, N, m, grid=grid) for m in ms]) for _ in range(3)]
    seen = []
    run_parity([N] * 3, _target_grads(targets), k=ks,
               label=f"near-classes chain={chain} grid={grid}",
               flags=gca.GC_DEBUG_CHAIN if chain else 0,
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist(),
                                                      st["ties"].tolist())))
    log(f"modes/candidates/ties: {seen}")
    for modes, cands, _ in seen[1:]:
        assert modes == [gca.MODE_CANDIDATES] * 3
        assert all(c >= m for c, m in zip(cands, ms))
    if grid:
        assert any(t > 1 for _, _, ties in seen for t in ties), "no ties at the k-th key"


@pytest.mark.parametrize("chain", [False, True], ids=["single", "chain"])
@pytest.mark.parametrize("m,k", [(200, 120), (600, 300)], ids=["ranked", "lds-passes"])
def test_kth_key_in_the_open_top_bin(m, k, chain):
    """The k-th key far above the capture floor: a call with m magnitudes near 1 sets the
    next floor near 1, then the same positions jump to 4..4000 (log-uniform, distinct), all of
    them in the histogram's top bin, which is open upwards.  The near list is then every
    candidate of that bin, over a key range of many binades."""
    rng = np.random.default_rng(303)
    pos = rng.choice(N, m, replace=False)
    targets = []
    for t in range(4):
        a = rng.normal(0.0, 1e-3, N)
        if t % 2 == 0:
            a[pos] = (1.0 + rng.uniform(0.0, 1e-3, m)) * rng.choice([-1.0, 1.0], m)
        else:
            a[pos] = np.exp(rng.uniform(np.log(4.0), np.log(4000.0), m)) * rng.choice(
                [-1.0, 1.0], m)
        targets.append(a)
    seen = []
    run_parity([N], _target_grads(targets), k=[k], label=f"top-bin m={m} chain={chain}",
               flags=gca.GC_DEBUG_CHAIN if chain else 0,
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist())))
    log(f"modes/candidates: {seen}")
    assert seen[1][0] == [gca.MODE_CANDIDATES]   # the jump is still captured in one pass


def test_small_segment_boundary():
    """Segments of 16383 and 16384 elements are selected whole (small); 16385 and larger take
    the candidate path, with the same results as the oracle's on every step."""
    sizes = [16383, 16384, 16385, 16386, 40000]
    rng = np.random.default_rng(404)
    n = sum(sizes)
    grads = [(rng.standard_t(3, n) * 1e-3).astype(np.float32) for _ in range(4)]
    seen = []
    run_parity(sizes, grads, ratio=0.01, label="small-boundary",
               check_stats=lambda t, st: seen.append(st["mode"].tolist()))
    log(f"modes: {seen}")
    for modes in seen:
        assert modes[:2] == [gca.MODE_SMALL] * 2
        assert all(m != gca.MODE_SMALL for m in modes[2:])
    for modes in seen[1:]:
        assert modes[2:] == [gca.MODE_CANDIDATES] * 3


def test_capture_all_segments_with_ties():
    """Segments where 16 k >= n capture every element (no threshold): k = 10% of 20000 and
    of 100003 elements, integer-valued gradients so that the k-th key is tied many times."""
    sizes = [20000, 100003]
    rng = np.random.default_rng(505)
    n = sum(sizes)
    grads = [rng.integers(-8, 9, n).astype(np.float32) for _ in range(3)]
    seen = []
    run_parity(sizes, grads, ratio=0.1, label="capture-all ties",
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist())))
    log(f"modes/candidates: {seen}")
    for modes, cands in seen:
        assert modes == [gca.MODE_CANDIDATES] * 2
        assert cands == sizes


@pytest.mark.parametrize("grid", [False, True], ids=["distinct", "ties"])
@pytest.mark.parametrize("chain", [False, True], ids=["single", "chain"])
def test_many_complete_candidates(chain, grid):
    """One 2^20-element segment with k = 1000 (a plan the single-workgroup select takes): a
    first call with 3000 magnitudes near 1 sets the threshold just below 1, then 30000
    magnitudes in [0.996, 0.9999] (on a grid of 64 values with ties) are all captured, so
    the complete candidates span four chunks of 8192, gathered and emitted a chunk at a
    time in index order."""
    rng = np.random.default_rng(606)
    k = 1000
    targets = [_cluster(rng, N, 3000)]
    for _ in range(3):
        a = rng.normal(0.0, 1e-3, N)
        pos = rng.choice(N, 30000, replace=False)
        if grid:
            mag = 0.996 + rng.integers(0, 64, pos.size) * (0.0039 / 64)
        else:
            mag = rng.uniform(0.996, 0.9999, pos.size)
        a[pos] = mag * rng.choice([-1.0, 1.0], pos.size)
        targets.append(a)
    seen = []
    run_parity([N], _target_grads(targets), k=[k], label=f"many-cands chain={chain}",
               flags=gca.GC_DEBUG_CHAIN if chain else 0,
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist(),
                                                      st["ties"].tolist())))
    log(f"modes/candidates/ties: {seen}")
    for modes, cands, _ in seen[1:]:
        assert modes == [gca.MODE_CANDIDATES]
        assert cands[0] > 3 * 8192
    if grid:
        assert any(t[0] > 1 for _, _, t in seen[1:]), "the grid gave no ties at the k-th key"


@pytest.mark.parametrize("k", [2048, 2049], ids=["single-4k-8192", "chain-4k-8196"])
def test_single_rule_limit_at_4m_elements(k):
    """A segment of 2^22 elements (the largest one workgroup selects: 512 tiles, its LDS run
    tables full) with k at the rule's limit (4k = 8192, one chunk) and one past it (the chain):
    a first call with 3k magnitudes near 1 sets the threshold just below 1, then 12k magnitudes
    in [0.996, 0.9999] are all captured (candidates over several chunks, gathered across all
    512 tiles on the single path), against the oracle on every call."""
    n = 1 << 22
    rng = np.random.default_rng(808)
    targets = [_cluster(rng, n, 3 * k)]
    for _ in range(2):
        a = rng.normal(0.0, 1e-3, n)
        pos = rng.choice(n, 12 * k, replace=False)
        a[pos] = rng.uniform(0.996, 0.9999, pos.size) * rng.choice([-1.0, 1.0], pos.size)
        targets.append(a)
    seen = []
    run_parity([n], _target_grads(targets), k=[k], label=f"4M k={k}",
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist())))
    log(f"modes/candidates: {seen}")
    for modes, cands in seen[1:]:
        assert modes == [gca.MODE_CANDIDATES]
        assert cands[0] > 8192


@pytest.mark.parametrize("n", [65536, 65537], ids=["single-whole", "chain"])
def test_single_rule_limit_at_65536_elements(n):
    """k = 10% of a 65536-element segment (the largest a workgroup selects whatever its k; every
    element captured, eight chunks of candidates) and of 65537 (the chain), with ties from
    integer-valued gradients."""
    rng = np.random.default_rng(909)
    grads = [rng.integers(-8, 9, n).astype(np.float32) for _ in range(3)]
    seen = []
    run_parity([n], grads, ratio=0.1, label=f"whole n={n}",
               check_stats=lambda t, st: seen.append((st["mode"].tolist(),
                                                      st["candidates"].tolist())))
    log(f"modes/candidates: {seen}")
    for modes, cands in seen:
        assert modes == [gca.MODE_CANDIDATES]
        assert cands == [n]
