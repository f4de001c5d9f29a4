"""The plan's host logic on the CPU (no GPU): k per segment from a ratio and the output
layout, through the library's host-only gc_layout, against the oracle's k rule; and the
argument checks gc_plan_create shares with it."""
import numpy as np
import pytest

import gradient_compression_amd as gca
import oracle


@pytest.mark.parametrize("seed", range(4))
def test_ratio_rule_and_offsets_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    n_seg = int(rng.integers(1, 400))
    sizes = rng.integers(0, 1 << 31, n_seg) if seed == 0 else rng.integers(0, 10 ** 6, n_seg)
    ratios = rng.choice([0.0, 1.0, 0.001, 0.01, 1e-9, 0.5, 0.3333333], n_seg)
    ratios = np.where(rng.random(n_seg) < 0.5, rng.random(n_seg), ratios)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    k, out_off = gca.layout(off, ratio=ratios)
    want = np.array([oracle.k_from_ratio(int(n), float(r)) for n, r in zip(sizes, ratios)])
    assert np.array_equal(k, want)
    assert np.array_equal(out_off, np.concatenate([[0], np.cumsum(want)]))


def test_given_k_and_the_pages_figures():
    k, off = gca.layout([0, 1 << 20], ratio=0.001)
    assert k.tolist() == [1049] and off.tolist() == [0, 1049]      # the single-segment workload
    k, off = gca.layout([0, 6400, 6400, 6410], k=[64, 0, 10])
    assert k.tolist() == [64, 0, 10] and off.tolist() == [0, 64, 64, 74]
    k, off = gca.layout([5], k=[])                                  # no segments
    assert k.size == 0 and off.tolist() == [0]


@pytest.mark.parametrize("args", [
    dict(seg_off=[0, 10], k=[11]),                  # k above the segment size
    dict(seg_off=[0, 10], k=[-1]),
    dict(seg_off=[0, 10, 5], k=[1, 1]),             # decreasing offsets
    dict(seg_off=[-1, 10], k=[1]),
    dict(seg_off=[0, 1 << 31], k=[1]),              # segment of 2^31 elements
    dict(seg_off=[0, 10], ratio=[1.5]),
    dict(seg_off=[0, 10], ratio=[-0.1]),
    dict(seg_off=[0, 10], ratio=[float("nan")]),
    dict(seg_off=[0, 10], k=[1], ratio=[0.1]),      # both given
    dict(seg_off=[0, 10]),                          # neither given
])
def test_invalid_arguments(args):
    with pytest.raises(gca.GCError) as ex:
        gca.layout(**args)
    assert ex.value.status == -1
