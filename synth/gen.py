"""Workload definitions and seeded gradient generators.

Every gradient value is drawn in float64 and rounded once to fp32.  The random stream is
torch's generator on the device the buffer lives on, re-seeded for every chunk of at most
2**24 elements from a 63-bit hash of (seed, workload, iteration, segment, chunk); so any
single segment can be regenerated on its own, and a run is reproducible for a given torch
build and device type (CPU and GPU generators give different, equally valid, draws).

Distributions (the heavy-tailed shape follows the motivation section of "Communication
Optimization > Gradient Compression": a small fraction of components carries most of the
gradient norm):
  * Student-t with real degrees of freedom by Bailey's polar method (Math. Comp. 1994):
    U, V ~ U(-1, 1) until W = U^2 + V^2 lies in (0, 1]; T = U * sqrt(df (W^(-2/df) - 1) / W).
  * Normal: torch's normal draw in float64.
  * Mixture: Bernoulli(p_out) chooses N(0, 1) over N(0, sigma_in^2), positions uniform.
"""
from __future__ import annotations

import dataclasses

import torch

from .shapes import (bert_large_segments, llama2_7b_segments, resnet50_segments,
                     seg_offsets)

CHUNK = 1 << 24
_MASK64 = (1 << 64) - 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    sizes: tuple            # elements per segment
    ratio: float            # k_s = ceil(n_s * ratio)
    iters: int              # EF iterations, each with a fresh gradient
    dist: str               # "t" | "normal_layer_scale" | "mixture"
    df: float = 0.0         # Student-t degrees of freedom
    scale: float = 1.0      # global multiplier of the draw
    momentum: float | None = None
    int8: bool = False

    @property
    def n(self) -> int:
        return int(sum(self.sizes))

    @property
    def n_seg(self) -> int:
        return len(self.sizes)

    def offsets(self):
        return seg_offsets(self.sizes)


def _sizes(segs):
    return tuple(n for _, n in segs)


WORKLOADS = {
    # single fp32 segment of 2^20, g ~ 1e-3 * t(3), k = 0.1% (1049), 5 EF iterations
    "c1_single_1m": Workload("c1_single_1m", 1, (1 << 20,), 0.001, 5, "t", df=3.0, scale=1e-3),
    # ResNet-50's 161 tensors, g ~ N(0, (1e-3)^2) * per-layer U(0.1, 10), k = 1%, 10 iterations
    "c2_resnet50": Workload("c2_resnet50", 2, _sizes(resnet50_segments()), 0.01, 10,
                            "normal_layer_scale", scale=1e-3),
    # BERT-large's 391 tensors, 0.1% outliers ~ N(0,1) in N(0, 0.01^2), k = 0.1%
    "c3_bert_large": Workload("c3_bert_large", 3, _sizes(bert_large_segments()), 0.001, 5,
                              "mixture"),
    # 64 segments of 2^24, g ~ t(2.5), k = 1%, then int8 with stochastic rounding
    "c4_hybrid_int8": Workload("c4_hybrid_int8", 4, (1 << 24,) * 64, 0.01, 5, "t", df=2.5,
                               int8=True),
    # Llama-2-7B's 291 tensors, g ~ 1e-4 * t(3), momentum correction u = 0.9 u + g, k = 0.1%
    "c5_llama2_7b": Workload("c5_llama2_7b", 5, _sizes(llama2_7b_segments()), 0.001, 5, "t",
                             df=3.0, scale=1e-4, momentum=0.9),
    # the same 7B shape without momentum: the plain EF-Top-k compress step
    "c5p_llama2_7b_plain": Workload("c5p_llama2_7b_plain", 6, _sizes(llama2_7b_segments()),
                                    0.001, 5, "t", df=3.0, scale=1e-4),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def _seed(*parts: int) -> int:
    h = 0x243F6A8885A308D3
    for p in parts:
        h = _splitmix64(h ^ (int(p) & _MASK64))
    return h & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def student_t(n: int, df: float, gen: torch.Generator, device) -> torch.Tensor:
    """n draws of Student-t(df) in float64 by Bailey's polar method."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    todo = torch.arange(n, device=device)
    while todo.numel():
        m = todo.numel()
        uv = torch.rand((2, m), dtype=torch.float64, generator=gen, device=device) * 2.0 - 1.0
        u, v = uv[0], uv[1]
        w = u * u + v * v
        ok = (w <= 1.0) & (w > 0.0)
        wk = w[ok]
        out[todo[ok]] = u[ok] * torch.sqrt(df * (wk.pow(-2.0 / df) - 1.0) / wk)
        todo = todo[~ok]
    return out


def layer_scale(wl: Workload, seg: int, seed: int = 0) -> float:
    """Per-segment multiplier ~ U(0.1, 10), drawn once (fixed across iterations)."""
    g = _gen("cpu", seed, wl.cfg_id, 0x5CA1E, seg)
    return float(0.1 + 9.9 * torch.rand(1, dtype=torch.float64, generator=g).item())


def _draw(wl: Workload, n: int, seg: int, gen, device) -> torch.Tensor:
    if wl.dist == "t":
        x = student_t(n, wl.df, gen, device)
        return x * wl.scale if wl.scale != 1.0 else x
    if wl.dist == "normal_layer_scale":
        return torch.randn(n, dtype=torch.float64, generator=gen, device=device) * (
            wl.scale * layer_scale(wl, seg))
    if wl.dist == "mixture":
        u = torch.rand(n, dtype=torch.float64, generator=gen, device=device)
        z = torch.randn(n, dtype=torch.float64, generator=gen, device=device)
        return torch.where(u < 0.001, z, z * 0.01)
    raise ValueError(wl.dist)


def fill_gradient(buf: torch.Tensor, wl: Workload, it: int, seed: int = 0, segments=None):
    """Write iteration ``it``'s gradient of workload ``wl`` into the flat fp32 ``buf``.

    ``segments``: optional iterable of segment ids to fill (the others are left as is).
    """
    assert buf.dtype == torch.float32 and buf.dim() == 1 and buf.numel() == wl.n
    off = wl.offsets()
    segs = range(wl.n_seg) if segments is None else segments
    dev = buf.device
    for s in segs:
        o, n = int(off[s]), int(off[s + 1] - off[s])
        for c0 in range(0, n, CHUNK):
            m = min(CHUNK, n - c0)
            gen = _gen(dev, seed, wl.cfg_id, it, s, c0 // CHUNK)
            buf[o + c0:o + c0 + m].copy_(_draw(wl, m, s, gen, dev).to(torch.float32))
    return buf


def fill_payloads(vals: torch.Tensor, idx: torch.Tensor, seg_off, ks, n_workers: int,
                  seed: int = 0):
    """Write n_workers synthetic payloads of the plan layout (per segment s, k_s distinct
    segment-local indices in ascending order and Student-t(3) x 1e-3 values), back to back in
    worker order, into vals / idx (device tensors of n_workers * sum(k) entries).  They stand
    in for what the other workers of a data-parallel group would send."""
    ks = [int(k) for k in ks]
    kk = sum(ks)
    assert vals.numel() >= n_workers * kk and idx.numel() >= n_workers * kk
    dev = vals.device
    for w in range(n_workers):
        base = w * kk
        for s, k_s in enumerate(ks):
            n_s = int(seg_off[s + 1] - seg_off[s])
            if k_s:
                gen = _gen(dev, seed, 0x9A7, w, s)
                r = torch.rand(n_s, generator=gen, device=dev)
                sel = torch.topk(r, k_s).indices.sort().values   # k distinct, ascending
                idx[base:base + k_s] = sel.to(torch.int32)
                vals[base:base + k_s] = (student_t(k_s, 3.0, gen, dev) * 1e-3).to(torch.float32)
            base += k_s
    return vals, idx
