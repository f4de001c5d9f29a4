"""The synthetic workloads: shapes, and the distributions the pages describe.

* segment counts and totals of the three model shapes;
* the mixture workload reproduces the heavy-tail figure of "Communication Optimization >
  Gradient Compression" (motivation section): about 0.1% of components carry over 90% of
  the norm (expected share 0.001 / (0.001 + 0.999e-4) = 0.909);
* Bailey's polar Student-t draws against scipy's t quantiles (Kolmogorov-Smirnov);
* a segment regenerates identically on its own.
"""
import json
import os

import numpy as np
import torch
from scipy import stats

from synth import gen, shapes, workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_shapes():
    for f, cnt, tot, lo, hi in [(shapes.resnet50_segments, 161, 25_557_032, 64, 2_359_296),
                                (shapes.bert_large_segments, 391, 335_141_888, 1024, 31_254_528),
                                (shapes.llama2_7b_segments, 291, 6_738_415_616, 4096, 131_072_000)]:
        sz = [n for _, n in f()]
        assert (len(sz), sum(sz), min(sz), max(sz)) == (cnt, tot, lo, hi)
    assert workload("c4_hybrid_int8").n == 1 << 30
    off = shapes.seg_offsets([3, 0, 5])
    assert off.tolist() == [0, 3, 3, 8]


def test_mixture_heavy_tail():
    with open(os.path.join(GOLD, "pages_figures.json")) as f:
        ht = json.load(f)["heavy_tail"]
    wl = workload("c3_bert_large")
    b = torch.zeros(wl.n, dtype=torch.float32)
    gen.fill_gradient(b, wl, 0, segments=[3, 9, 100])
    off = wl.offsets()
    x = torch.cat([b[off[s]:off[s + 1]] for s in (3, 9, 100)]).double()
    # the largest 0.1% of components by magnitude carry more than 90% of the squared norm
    k = int(np.ceil(ht["max_component_fraction"] * x.numel()))
    top = torch.topk(x.abs(), k).values
    share = float((top ** 2).sum() / (x ** 2).sum())
    assert share > ht["min_norm_share"]


def test_student_t_matches_scipy():
    g = torch.Generator().manual_seed(3)
    for df in (2.5, 3.0):
        x = gen.student_t(200_000, df, g, "cpu").numpy()
        ks = stats.kstest(x, stats.t(df).cdf)
        assert ks.pvalue > 1e-3, (df, ks)


def test_segment_regenerates_alone():
    wl = workload("c2_resnet50")
    a = torch.zeros(wl.n)
    b = torch.zeros(wl.n)
    gen.fill_gradient(a, wl, 2, segments=range(0, 20))
    gen.fill_gradient(b, wl, 2, segments=[7])
    off = wl.offsets()
    assert torch.equal(a[off[7]:off[8]], b[off[7]:off[8]])
    assert not torch.equal(a[off[7]:off[8]], torch.zeros(int(off[8] - off[7])))
    c = torch.zeros(wl.n)
    gen.fill_gradient(c, wl, 3, segments=[7])
    assert not torch.equal(a[off[7]:off[8]], c[off[7]:off[8]])
