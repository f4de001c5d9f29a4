"""Seeded synthetic inputs for the compression path: workload shapes and gradient draws.

This module is shared by the tests, the bench and the CPU baseline.  It holds none of
the compression method's arithmetic: it only decides which gradients are fed in.
"""
from .shapes import (bert_large_segments, llama2_7b_segments, resnet50_segments,
                     seg_offsets)
from .gen import WORKLOADS, Workload, fill_gradient, fill_payloads, workload

__all__ = ["WORKLOADS", "Workload", "workload", "fill_gradient", "fill_payloads", "seg_offsets",
           "resnet50_segments", "bert_large_segments", "llama2_7b_segments"]
