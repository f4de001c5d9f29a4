"""The C-ABI library loads, exports every entry point gc.h declares, and rejects bad
arguments on the host before touching a GPU (no compute calls here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import gradient_compression_amd as gca
from gradient_compression_amd import build as gc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "gc.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gc_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = gca.lib()
    names = declared_functions()
    assert len(names) >= 13
    for name in names:
        assert hasattr(L, name), name
    assert sorted(gca.EXPORTS) == names


@pytest.mark.parametrize("variant", sorted(gc_build.VARIANTS))
def test_tile_geometry_variants_export_every_symbol(variant):
    """The same library at the other tile geometries (the GPU tests check that their results
    equal the default geometry's)."""
    L = gca.lib(variant)
    for name in declared_functions():
        assert hasattr(L, name), f"{variant}: {name}"


def test_status_strings():
    assert gca.status_string(0) == "success"
    assert gca.status_string(-1) == "invalid argument"
    assert gca.status_string(12345) == "unknown status"


def _create(seg_off, k=None, ratio=None, flags=0, n_seg=None):
    L = gca.lib()
    h = ctypes.c_void_p()
    off = np.ascontiguousarray(seg_off, np.int64)
    ns = len(off) - 1 if n_seg is None else n_seg
    kp = None if k is None else np.ascontiguousarray(k, np.int64).ctypes.data_as(ctypes.c_void_p)
    rp = None if ratio is None else np.ascontiguousarray(ratio, np.float64).ctypes.data_as(
        ctypes.c_void_p)
    return L.gc_plan_create(off.ctypes.data_as(ctypes.c_void_p), ns, kp, rp, flags,
                            ctypes.byref(h))


@pytest.mark.parametrize("case", [
    dict(seg_off=[0, 10, 5], k=[1, 1]),              # decreasing offsets
    dict(seg_off=[0, 10], k=[11]),                   # k > n
    dict(seg_off=[0, 10], k=[-1]),                   # negative k
    dict(seg_off=[0, 10], ratio=[1.5]),              # ratio > 1
    dict(seg_off=[0, 10], ratio=[float("nan")]),     # ratio NaN
    dict(seg_off=[0, 10]),                           # neither k nor ratio
    dict(seg_off=[0, 10], k=[1], ratio=[0.1]),       # both
    dict(seg_off=[-4, 10], k=[1]),                   # negative base
    dict(seg_off=[0, 1 << 31], k=[1]),               # segment >= 2^31
    dict(seg_off=[0, 10], k=[1], flags=0x8000),      # unknown flag
    dict(seg_off=[0, 10], k=[1], n_seg=-1),          # negative count
])
def test_plan_create_rejects(case):
    assert _create(**case) == gca.GC_ERR_INVALID_ARG


def test_null_handles_rejected():
    L = gca.lib()
    assert L.gc_plan_create(None, 0, None, None, 0, None) == gca.GC_ERR_INVALID_ARG
    assert L.gc_topk_ef_compress(None, None, None, None, 0.0, None, None, None) == -1
    assert L.gc_quant_int8(None, None, None, None, 0, 0, None, None, None) == -1
    assert L.gc_decompress(None, None, None, None, None, None, 0, None) == -1
    assert L.gc_plan_total_k(None, None) == -1
    assert L.gc_plan_layout(None, None, None) == -1
    assert L.gc_plan_reset_estimate(None, None) == -1
    assert L.gc_plan_last_stats(None, None, None, None, None, None) == -1
    assert L.gc_plan_set_timing(None, 1) == -1
    assert L.gc_plan_timing(None, None, None) == -1
    assert L.gc_plan_destroy(None) == 0
    # copy: n not a multiple of 4, or misaligned pointers
    assert L.gc_copy_f32(None, None, 3, None) == -1
    assert L.gc_copy_f32(ctypes.c_void_p(16), ctypes.c_void_p(20), 4, None) == -1
