"""CPU oracle of error-feedback Top-k compression (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may import
this package.  The arithmetic lives in ``oracle.c`` (plain C, full sort per segment, exact
fp32); this module only builds it with gcc and marshals numpy arrays into it.  It shares
no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load(path: str):
    """Open an oracle shared library and declare its C signatures."""
    L = ctypes.CDLL(path)
    i64, i32, u64, f32, vp = (ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float,
                              ctypes.c_void_p)
    L.orc_k_from_ratio.argtypes = [i64, ctypes.c_double]
    L.orc_k_from_ratio.restype = i64
    L.orc_topk_ef_segment.argtypes = [i64, i64, vp, vp, vp, f32, ctypes.c_int, vp, vp]
    L.orc_topk_ef_segment.restype = ctypes.c_int
    L.orc_topk_ef.argtypes = [i32, vp, vp, vp, vp, vp, f32, ctypes.c_int, vp, vp]
    L.orc_topk_ef.restype = ctypes.c_int
    L.orc_philox4x32_10.argtypes = [vp, vp, vp]
    L.orc_philox4x32_10.restype = None
    L.orc_quant_int8_segment.argtypes = [i64, vp, vp, i64, vp, u64, u64, vp, vp]
    L.orc_quant_int8_segment.restype = None
    L.orc_quant_int8.argtypes = [i32, vp, vp, vp, vp, vp, u64, u64, vp, vp]
    L.orc_quant_int8.restype = None
    L.orc_decompress.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    L.orc_decompress.restype = None
    L.orc_sign_ef_segment.argtypes = [i64, vp, vp, vp, f32, vp, vp]
    L.orc_sign_ef_segment.restype = None
    L.orc_sign_decompress_segment.argtypes = [i64, vp, f32, vp, ctypes.c_int]
    L.orc_sign_decompress_segment.restype = None
    L.orc_clip_by_norm_segment.argtypes = [i64, vp, f32, vp]
    L.orc_clip_by_norm_segment.restype = None
    L.orc_decompress_gathered.argtypes = [i32, vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_int]
    L.orc_decompress_gathered.restype = None
    L.orc_threshold_ef_segment.argtypes = [i64, i64, f32, vp, vp, vp, f32, ctypes.c_int, vp,
                                           vp, vp]
    L.orc_threshold_ef_segment.restype = ctypes.c_int
    L.orc_randk_segment.argtypes = [i64, i64, i64, vp, vp, vp, f32, ctypes.c_int, u64, u64,
                                    vp, vp]
    L.orc_randk_segment.restype = ctypes.c_int
    L.orc_qsgd_segment.argtypes = [i64, i64, vp, vp, vp, f32, i32, u64, u64, vp, vp]
    L.orc_qsgd_segment.restype = ctypes.c_int
    L.orc_qsgd_decompress_segment.argtypes = [i64, vp, f32, i32, vp, ctypes.c_int]
    L.orc_qsgd_decompress_segment.restype = None
    return L


def lib():
    """The oracle library: liboracle.so, or the build of oracle.c that GC_ORACLE_LIB names
    (the sanitizer test runs the oracle's tests against an ASan/UBSan build that way)."""
    global _lib
    if _lib is None:
        other = os.environ.get("GC_ORACLE_LIB")
        if other:
            _lib = load(other)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = load(_LIB)
    return _lib


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile a (test-planted) variant of oracle.c with the oracle's own flags."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *_CFLAGS, c_path, "-o", out_path, "-lm"], check=True)
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def _p(a):
    return None if a is None else a.ctypes.data


def _f32(a, name):
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a contiguous float32 array")
    return a


def k_from_ratio(n: int, ratio: float) -> int:
    """k = min(n, ceil(n * ratio)) in exact parts-per-billion arithmetic."""
    return int(lib().orc_k_from_ratio(int(n), float(ratio)))


def topk_ef_segment(g, e, k, u=None, momentum=0.9, mask_u=False):
    """One segment, in place on e (and u).  Returns (vals float32[k], idx int32[k])."""
    _f32(g, "g"), _f32(e, "e")
    if u is not None:
        _f32(u, "u")
    n = g.size
    assert e.size == n and (u is None or u.size == n)
    vals = np.empty(max(k, 0), np.float32)
    idx = np.empty(max(k, 0), np.int32)
    rc = lib().orc_topk_ef_segment(n, int(k), _p(g), _p(e), _p(u), float(momentum),
                                   int(bool(mask_u)), _p(vals), _p(idx))
    if rc:
        raise ValueError("oracle rejected the segment arguments")
    return vals, idx


def topk_ef(g, e, seg_off, k, u=None, momentum=0.9, mask_u=False):
    """Whole segmented buffer, in place on e (and u).  Returns (vals, idx) grouped by
    segment in segment order, ascending segment-local index inside each segment."""
    _f32(g, "g"), _f32(e, "e")
    seg_off = np.ascontiguousarray(seg_off, np.int64)
    k = np.ascontiguousarray(k, np.int64)
    tot = int(k.sum())
    vals = np.empty(tot, np.float32)
    idx = np.empty(tot, np.int32)
    rc = lib().orc_topk_ef(len(k), _p(seg_off), _p(k), _p(g), _p(e), _p(u), float(momentum),
                           int(bool(mask_u)), _p(vals), _p(idx))
    if rc:
        raise ValueError("oracle rejected the arguments")
    return vals, idx


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint32)
    kk = np.ascontiguousarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(kk), _p(out))
    return out


def quant_int8_segment(vals, idx, seg_base, e_seg=None, seed=0, step=0):
    """Returns (codes int8[k], scale float32); writes the quantisation error into e_seg."""
    _f32(vals, "vals")
    idx = np.ascontiguousarray(idx, np.int32)
    codes = np.empty(vals.size, np.int8)
    scale = np.empty(1, np.float32)
    lib().orc_quant_int8_segment(vals.size, _p(vals), _p(idx), int(seg_base), _p(e_seg),
                                 int(seed), int(step), _p(codes), _p(scale))
    return codes, scale[0]


def quant_int8(vals, idx, seg_off, k, e=None, seed=0, step=0):
    """Whole buffer.  Returns (codes int8[sum k], scales float32[n_seg])."""
    _f32(vals, "vals")
    idx = np.ascontiguousarray(idx, np.int32)
    seg_off = np.ascontiguousarray(seg_off, np.int64)
    k = np.ascontiguousarray(k, np.int64)
    codes = np.empty(vals.size, np.int8)
    scales = np.empty(len(k), np.float32)
    lib().orc_quant_int8(len(k), _p(seg_off), _p(k), _p(vals), _p(idx), _p(e), int(seed),
                         int(step), _p(codes), _p(scales))
    return codes, scales


def decompress(seg_off, k, idx, vals=None, codes=None, scales=None, dense=None,
               accumulate=False):
    seg_off = np.ascontiguousarray(seg_off, np.int64)
    k = np.ascontiguousarray(k, np.int64)
    idx = np.ascontiguousarray(idx, np.int32)
    if dense is None:
        dense = np.empty(int(seg_off[-1]), np.float32)
    if vals is None:
        codes = np.ascontiguousarray(codes, np.int8)
        scales = np.ascontiguousarray(scales, np.float32)
    lib().orc_decompress(len(k), _p(seg_off), _p(k), _p(vals), _p(codes), _p(scales), _p(idx),
                         _p(dense), int(bool(accumulate)))
    return dense


def decompress_gathered(seg_off, k, n_workers, idx, vals=None, codes=None, scales=None,
                        dense=None, accumulate=False):
    """Add n_workers payloads (back to back in worker order) into dense, worker by worker."""
    seg_off = np.ascontiguousarray(seg_off, np.int64)
    k = np.ascontiguousarray(k, np.int64)
    idx = np.ascontiguousarray(idx, np.int32)
    assert idx.size == n_workers * int(k.sum())
    if dense is None:
        dense = np.empty(int(seg_off[-1]), np.float32)
    if vals is None:
        codes = np.ascontiguousarray(codes, np.int8)
        scales = np.ascontiguousarray(scales, np.float32)
    lib().orc_decompress_gathered(len(k), _p(seg_off), _p(k), int(n_workers), _p(vals),
                                  _p(codes), _p(scales), _p(idx), _p(dense),
                                  int(bool(accumulate)))
    return dense


def sign_ef_segment(g, e, u=None, momentum=0.9):
    """1-bit sign compression of one segment with error feedback, in place on e (and u).
    Returns (bits uint32[ceil(n/32)], scale float32)."""
    _f32(g, "g"), _f32(e, "e")
    n = g.size
    bits = np.empty((n + 31) // 32, np.uint32)
    scale = np.empty(1, np.float32)
    lib().orc_sign_ef_segment(n, _p(g), _p(e), _p(u), float(momentum), _p(bits), _p(scale))
    return bits, scale[0]


def sign_decompress_segment(bits, scale, n, dense=None, accumulate=False):
    bits = np.ascontiguousarray(bits, np.uint32)
    if dense is None:
        dense = np.empty(n, np.float32)
    lib().orc_sign_decompress_segment(n, _p(bits), float(scale), _p(dense), int(bool(accumulate)))
    return dense


def qsgd_segment(g, e=None, u=None, momentum=0.9, levels=127, seed=0, step=0, seg_base=0):
    """QSGD with `levels` levels of one segment; with e, error feedback in place on e.
    Returns (codes int8[n], norm float32)."""
    _f32(g, "g")
    n = g.size
    codes = np.empty(n, np.int8)
    norm = np.empty(1, np.float32)
    rc = lib().orc_qsgd_segment(n, int(seg_base), _p(g), _p(e), _p(u), float(momentum),
                                int(levels), int(seed), int(step), _p(codes), _p(norm))
    if rc:
        raise ValueError("oracle rejected the QSGD arguments")
    return codes, norm[0]


def qsgd_decompress_segment(codes, norm, levels, dense=None, accumulate=False):
    codes = np.ascontiguousarray(codes, np.int8)
    if dense is None:
        dense = np.empty(codes.size, np.float32)
    lib().orc_qsgd_decompress_segment(codes.size, _p(codes), float(norm), int(levels), _p(dense),
                                      int(bool(accumulate)))
    return dense


def threshold_ef_segment(g, e, k_cap, tau, u=None, momentum=0.9, mask_u=False):
    """Threshold sparsification of one segment (at most k_cap entries with |acc| >= |tau|),
    in place on e (and u).  Returns (vals, idx) of the sent entries."""
    _f32(g, "g"), _f32(e, "e")
    n = g.size
    vals = np.empty(max(k_cap, 1), np.float32)
    idx = np.empty(max(k_cap, 1), np.int32)
    cnt = np.zeros(1, np.int64)
    rc = lib().orc_threshold_ef_segment(n, int(k_cap), float(tau), _p(g), _p(e), _p(u),
                                        float(momentum), int(bool(mask_u)), _p(vals), _p(idx),
                                        _p(cnt))
    if rc:
        raise ValueError("oracle rejected the segment arguments")
    return vals[:cnt[0]].copy(), idx[:cnt[0]].copy()


def randk_segment(g, k, e=None, u=None, momentum=0.9, mask_u=False, seed=0, step=0,
                  seg_base=0):
    """Random-k of one segment (global offset seg_base); with e, error feedback in place on
    e, else values scaled by n/k.  Returns (vals float32[k], idx int32[k])."""
    _f32(g, "g")
    n = g.size
    vals = np.empty(max(k, 1), np.float32)
    idx = np.empty(max(k, 1), np.int32)
    rc = lib().orc_randk_segment(n, int(k), int(seg_base), _p(g), _p(e), _p(u),
                                 float(momentum), int(bool(mask_u)), int(seed), int(step),
                                 _p(vals), _p(idx))
    if rc:
        raise ValueError("oracle rejected the Random-k arguments")
    return vals[:k].copy(), idx[:k].copy()


def clip_by_norm_segment(g, c):
    """l2-norm clipping of one segment in place on g; returns the norm before clipping."""
    _f32(g, "g")
    norm = np.empty(1, np.float32)
    lib().orc_clip_by_norm_segment(g.size, _p(g), float(c), _p(norm))
    return norm[0]
