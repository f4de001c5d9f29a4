"""Segment tables (one segment per parameter tensor) of the five synthetic workloads.

A worker's gradient is one flat fp32 buffer cut into per-tensor segments; selection
happens per layer tensor ("Gradient Compression" glossary, sparsification section:
top-k is taken per layer; "Gradient Sparsification" glossary, mechanism section).
The model shapes below are the standard published architectures, listed in the
framework's usual parameter order; only their sizes matter here.
"""
from __future__ import annotations

import numpy as np


def resnet50_segments() -> list[tuple[str, int]]:
    """ResNet-50 (ImageNet, 1000 classes): 161 tensors, 25,557,032 parameters."""
    segs: list[tuple[str, int]] = [("conv1.weight", 64 * 3 * 7 * 7),
                                   ("bn1.weight", 64), ("bn1.bias", 64)]
    inplanes = 64
    for li, (planes, blocks) in enumerate([(64, 3), (128, 4), (256, 6), (512, 3)], start=1):
        for b in range(blocks):
            p = f"layer{li}.{b}"
            segs += [(f"{p}.conv1.weight", planes * inplanes),
                     (f"{p}.bn1.weight", planes), (f"{p}.bn1.bias", planes),
                     (f"{p}.conv2.weight", planes * planes * 9),
                     (f"{p}.bn2.weight", planes), (f"{p}.bn2.bias", planes),
                     (f"{p}.conv3.weight", planes * 4 * planes),
                     (f"{p}.bn3.weight", planes * 4), (f"{p}.bn3.bias", planes * 4)]
            if b == 0:
                segs += [(f"{p}.downsample.0.weight", planes * 4 * inplanes),
                         (f"{p}.downsample.1.weight", planes * 4),
                         (f"{p}.downsample.1.bias", planes * 4)]
            inplanes = planes * 4
    segs += [("fc.weight", 1000 * 2048), ("fc.bias", 1000)]
    return segs


def bert_large_segments() -> list[tuple[str, int]]:
    """BERT-large encoder with pooler: 391 tensors, 335,141,888 parameters."""
    h, ffn, vocab, layers = 1024, 4096, 30522, 24
    segs = [("embeddings.word", vocab * h), ("embeddings.position", 512 * h),
            ("embeddings.token_type", 2 * h), ("embeddings.ln.weight", h),
            ("embeddings.ln.bias", h)]
    for i in range(layers):
        p = f"layer{i}"
        for m in ("query", "key", "value"):
            segs += [(f"{p}.attn.{m}.weight", h * h), (f"{p}.attn.{m}.bias", h)]
        segs += [(f"{p}.attn.out.weight", h * h), (f"{p}.attn.out.bias", h),
                 (f"{p}.attn.ln.weight", h), (f"{p}.attn.ln.bias", h),
                 (f"{p}.ffn.in.weight", ffn * h), (f"{p}.ffn.in.bias", ffn),
                 (f"{p}.ffn.out.weight", h * ffn), (f"{p}.ffn.out.bias", h),
                 (f"{p}.ffn.ln.weight", h), (f"{p}.ffn.ln.bias", h)]
    segs += [("pooler.weight", h * h), ("pooler.bias", h)]
    return segs


def llama2_7b_segments() -> list[tuple[str, int]]:
    """Llama-2-7B with untied output head: 291 tensors, 6,738,415,616 parameters."""
    h, ffn, vocab, layers = 4096, 11008, 32000, 32
    segs = [("embed_tokens", vocab * h)]
    for i in range(layers):
        p = f"layer{i}"
        segs += [(f"{p}.q_proj", h * h), (f"{p}.k_proj", h * h), (f"{p}.v_proj", h * h),
                 (f"{p}.o_proj", h * h), (f"{p}.gate_proj", ffn * h),
                 (f"{p}.up_proj", ffn * h), (f"{p}.down_proj", h * ffn),
                 (f"{p}.input_norm", h), (f"{p}.post_attn_norm", h)]
    segs += [("norm", h), ("lm_head", vocab * h)]
    return segs


def seg_offsets(sizes) -> np.ndarray:
    """Exclusive prefix sum of segment sizes: int64[n_seg + 1]."""
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(np.asarray(sizes, dtype=np.int64), out=off[1:])
    return off
