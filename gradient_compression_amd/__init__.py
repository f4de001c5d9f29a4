"""MI355X-native error-feedback Top-k gradient compression.

A thin Python binding over the C ABI of ``libgc.so`` (``include/gc.h``): argument
marshalling only, every step of the path runs in the library's HIP kernels.  PyTorch is used
for device memory and streams.  The package fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GC_LIB_PATH: load another build of the same library (the host-sanitizer test uses it)
LIB_PATH = os.environ.get("GC_LIB_PATH") or os.path.join(_HERE, "libgc.so")

GC_OK = 0
GC_ERR_INVALID_ARG = -1
GC_ERR_OOM = -2
GC_ERR_HIP = -3
GC_ERR_UNSUPPORTED = -4
GC_MOMENTUM_MASK = 0x1
GC_DEBUG_FORCE_FALLBACK = 0x100
GC_DEBUG_NO_ESTIMATE = 0x200
# Select with the chain of kernels over candidate chunks even where one workgroup per segment
# would do (same results; tests).
GC_DEBUG_CHAIN = 0x400

MODE_SKIP, MODE_CANDIDATES, MODE_FULL, MODE_RECAPTURED, MODE_SMALL = 0, 1, 2, 3, 5
# Segments of at most this many elements are selected whole by one workgroup (MODE_SMALL).
SMALL_SEGMENT = 16384

EXPORTS = ("gc_plan_create", "gc_plan_destroy", "gc_plan_total_k", "gc_plan_layout",
           "gc_topk_ef_compress", "gc_topk_ef_compress_int8", "gc_quant_int8", "gc_decompress", "gc_plan_reset_estimate",
           "gc_plan_last_stats", "gc_plan_set_timing", "gc_plan_timing", "gc_copy_f32", "gc_add_f32",
           "gc_read_f32", "gc_topk_ef_compress_noalloc",
           "gc_status_string", "gc_sign_ef_compress", "gc_plan_sign_layout",
           "gc_sign_decompress", "gc_qsgd_compress", "gc_qsgd_decompress",
           "gc_threshold_ef_compress", "gc_randk_compress", "gc_decompress_gathered",
           "gc_clip_by_norm", "gc_clip_factors", "gc_plan_set_gradient_scale", "gc_layout")

_libs: dict = {}


class GCError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def lib(variant: str | None = None) -> ctypes.CDLL:
    """Load libgc.so (built by ``__graft_entry__.build()``); raise if it is not built.

    ``variant``: one of the other tile geometries that the build also compiles
    (``build.VARIANTS``, e.g. "t256s2"); the default geometry when None."""
    key = variant or ""
    if key in _libs:
        return _libs[key]
    if variant is None:
        path = LIB_PATH
    else:
        from . import build as _build
        path = _build.variant_path(variant)
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run __graft_entry__.build() "
                          "(there is no fallback implementation)")
    L = ctypes.CDLL(path)
    vp, i32, i64, u32, u64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float)
    sig = {
        "gc_plan_create": [vp, i32, vp, vp, u32, vp],
        "gc_plan_destroy": [vp],
        "gc_plan_total_k": [vp, vp],
        "gc_plan_layout": [vp, vp, vp],
        "gc_topk_ef_compress": [vp, vp, vp, vp, f32, vp, vp, vp],
        "gc_topk_ef_compress_int8": [vp, vp, vp, vp, f32, u64, u64, vp, vp, vp, vp, vp],
        "gc_quant_int8": [vp, vp, vp, vp, u64, u64, vp, vp, vp],
        "gc_decompress": [vp, vp, vp, vp, vp, vp, ctypes.c_int, vp],
        "gc_plan_reset_estimate": [vp, vp],
        "gc_plan_last_stats": [vp, vp, vp, vp, vp, vp],
        "gc_plan_set_timing": [vp, ctypes.c_int],
        "gc_plan_timing": [vp, vp, vp],
        "gc_copy_f32": [vp, vp, i64, vp],
        "gc_add_f32": [vp, vp, i64, vp],
        "gc_read_f32": [vp, i64, vp, vp],
        "gc_topk_ef_compress_noalloc": [vp, i32, vp, vp, u32, vp, vp, vp, f32, vp, vp, vp],
        "gc_status_string": [ctypes.c_int],
        "gc_sign_ef_compress": [vp, vp, vp, vp, f32, vp, vp, vp],
        "gc_plan_sign_layout": [vp, vp],
        "gc_sign_decompress": [vp, vp, vp, vp, ctypes.c_int, vp],
        "gc_qsgd_compress": [vp, vp, vp, vp, f32, i32, u64, u64, vp, vp, vp],
        "gc_qsgd_decompress": [vp, vp, vp, i32, vp, ctypes.c_int, vp],
        "gc_threshold_ef_compress": [vp, vp, vp, vp, f32, vp, vp, vp, vp, vp],
        "gc_randk_compress": [vp, vp, vp, vp, f32, u64, u64, vp, vp, vp],
        "gc_decompress_gathered": [vp, i32, vp, vp, vp, vp, vp, ctypes.c_int, vp],
        "gc_clip_by_norm": [vp, vp, vp, vp, vp],
        "gc_clip_factors": [vp, vp, vp, vp, vp, vp],
        "gc_plan_set_gradient_scale": [vp, vp],
        "gc_layout": [vp, i32, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "gc_status_string" else ctypes.c_int
    _libs[key] = L
    return L


def status_string(status: int) -> str:
    return lib().gc_status_string(int(status)).decode()


def _check(rc: int, what: str):
    if rc != GC_OK:
        raise GCError(rc, what)


def layout(seg_off, k=None, ratio=None):
    """Host-only: (k per segment, output offsets) of a plan with these arguments."""
    off = np.ascontiguousarray(seg_off, dtype=np.int64)
    n_seg = int(off.size - 1)
    kp = rp = None
    if k is not None:
        k_in = np.ascontiguousarray(np.broadcast_to(np.asarray(k, np.int64), (n_seg,)))
        kp = _np_ptr(k_in)
    if ratio is not None:
        r_in = np.ascontiguousarray(np.broadcast_to(np.asarray(ratio, np.float64), (n_seg,)))
        rp = _np_ptr(r_in)
    k_out = np.zeros(max(n_seg, 0), np.int64)
    out_off = np.zeros(max(n_seg, 0) + 1, np.int64)
    _check(lib().gc_layout(_np_ptr(off), n_seg, kp, rp, _np_ptr(k_out), _np_ptr(out_off)),
           "gc_layout")
    return k_out, out_off


def topk_ef_compress_noalloc(seg_off, g, e, out_vals, out_idx, k=None, ratio=None,
                             flags: int = 0, u=None, momentum: float = 0.0, stream=None,
                             variant: str | None = None):
    """The Top-k step without a plan, for callers that cannot allocate device memory: the
    library keeps the call's state in a static device array (limits: GC_NOALLOC_MAX_*).
    Results equal Plan(seg_off, k, ratio, flags).compress(...) bit for bit."""
    import torch
    off = np.ascontiguousarray(seg_off, dtype=np.int64)
    n_seg = int(off.size - 1)
    kp = rp = None
    if k is not None:
        k_in = np.ascontiguousarray(np.broadcast_to(np.asarray(k, np.int64), (n_seg,)))
        kp = _np_ptr(k_in)
    if ratio is not None:
        r_in = np.ascontiguousarray(np.broadcast_to(np.asarray(ratio, np.float64), (n_seg,)))
        rp = _np_ptr(r_in)
    k_out, out_off = layout(off, k=k, ratio=ratio)
    n = int(off[-1]) if n_seg >= 0 else 0
    tk = int(out_off[-1])
    rc = lib(variant).gc_topk_ef_compress_noalloc(
        _np_ptr(off), n_seg, kp, rp, int(flags), _dev_ptr(g, torch.float32, "g", n),
        _dev_ptr(e, torch.float32, "e", n), _dev_ptr(u, torch.float32, "u", n), float(momentum),
        _dev_ptr(out_vals, torch.float32, "out_vals", tk),
        _dev_ptr(out_idx, torch.int32, "out_idx", tk), _stream(stream))
    _check(rc, "gc_topk_ef_compress_noalloc")


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t, dtype, name, numel=None):
    """Device pointer of a contiguous CUDA/HIP tensor of the given dtype (None -> NULL)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    cur = torch.cuda.current_device()
    if t.device.index is not None and t.device.index != cur:
        # the library runs on the current device (which must be the plan's)
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{cur}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Plan:
    """A compression plan over a segmented buffer (one segment per parameter tensor).

    ``seg_off``: int64[n_seg + 1] segment offsets; give per-segment ``k`` or ``ratio``.
    ``variant``: run on a library built at another tile geometry (see ``lib``).
    """

    def __init__(self, seg_off, k=None, ratio=None, flags: int = 0, variant: str | None = None):
        self._L = L = lib(variant)
        self.variant = variant
        self._h = ctypes.c_void_p()
        off = np.ascontiguousarray(seg_off, dtype=np.int64)
        self.n_seg = int(off.size - 1)
        if self.n_seg < 0:
            raise ValueError("seg_off needs at least one entry")
        kp = rp = None
        if k is not None:
            self._k_in = np.ascontiguousarray(np.broadcast_to(np.asarray(k, np.int64), (self.n_seg,)))
            kp = _np_ptr(self._k_in)
        if ratio is not None:
            self._r_in = np.ascontiguousarray(np.broadcast_to(np.asarray(ratio, np.float64),
                                                              (self.n_seg,)))
            rp = _np_ptr(self._r_in)
        _check(L.gc_plan_create(_np_ptr(off), self.n_seg, kp, rp, int(flags),
                                ctypes.byref(self._h)), "gc_plan_create")
        self.seg_off = off.copy()
        self.n = int(off[-1])
        self.flags = int(flags)
        tk = ctypes.c_int64()
        _check(L.gc_plan_total_k(self._h, ctypes.byref(tk)), "gc_plan_total_k")
        self.total_k = tk.value
        self.k = np.zeros(self.n_seg, np.int64)
        self.out_off = np.zeros(self.n_seg + 1, np.int64)
        _check(L.gc_plan_layout(self._h, _np_ptr(self.k), _np_ptr(self.out_off)),
               "gc_plan_layout")
        self.word_off = np.zeros(self.n_seg + 1, np.int64)
        _check(L.gc_plan_sign_layout(self._h, _np_ptr(self.word_off)), "gc_plan_sign_layout")
        self.total_words = int(self.word_off[-1])

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._L.gc_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---------------------------------------------------------------- entry points
    def compress(self, g, e, out_vals, out_idx, u=None, momentum: float = 0.0, stream=None):
        """g^ = TopK(g + e) per segment into (out_vals, out_idx); e <- the residual.

        With ``u`` (velocity): u <- momentum*u + g first, and acc = e + u.
        """
        import torch
        n = self.n
        rc = self._L.gc_topk_ef_compress(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum),
            _dev_ptr(out_vals, torch.float32, "out_vals", self.total_k),
            _dev_ptr(out_idx, torch.int32, "out_idx", self.total_k), _stream(stream))
        _check(rc, "gc_topk_ef_compress")

    def compress_int8(self, g, e, out_idx, out_codes, out_scales, out_vals=None, u=None,
                      momentum: float = 0.0, seed: int = 0, step: int = 0, stream=None):
        """compress then int8 in one call (the quantisation error goes back into e)."""
        import torch
        n = self.n
        rc = self._L.gc_topk_ef_compress_int8(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum), int(seed) & (2 ** 64 - 1),
            int(step) & (2 ** 64 - 1),
            _dev_ptr(out_vals, torch.float32, "out_vals", self.total_k),
            _dev_ptr(out_idx, torch.int32, "out_idx", self.total_k),
            _dev_ptr(out_codes, torch.int8, "out_codes", self.total_k),
            _dev_ptr(out_scales, torch.float32, "out_scales", self.n_seg), _stream(stream))
        _check(rc, "gc_topk_ef_compress_int8")

    def quant_int8(self, vals, idx, out_codes, out_scales, e=None, seed: int = 0, step: int = 0,
                   stream=None):
        """int8 codes and per-segment scales of the kept values (stochastic rounding);
        with ``e`` the quantisation error is fed back into the residual."""
        import torch
        rc = self._L.gc_quant_int8(
            self._h, _dev_ptr(vals, torch.float32, "vals", self.total_k),
            _dev_ptr(idx, torch.int32, "idx", self.total_k), _dev_ptr(e, torch.float32, "e", self.n),
            int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1),
            _dev_ptr(out_codes, torch.int8, "out_codes", self.total_k),
            _dev_ptr(out_scales, torch.float32, "out_scales", self.n_seg), _stream(stream))
        _check(rc, "gc_quant_int8")

    def decompress(self, idx, dense, vals=None, codes=None, scales=None, accumulate=False,
                   stream=None):
        import torch
        rc = self._L.gc_decompress(
            self._h, _dev_ptr(vals, torch.float32, "vals", self.total_k),
            _dev_ptr(codes, torch.int8, "codes", self.total_k),
            _dev_ptr(scales, torch.float32, "scales", self.n_seg),
            _dev_ptr(idx, torch.int32, "idx", self.total_k),
            _dev_ptr(dense, torch.float32, "dense", self.n), int(bool(accumulate)),
            _stream(stream))
        _check(rc, "gc_decompress")

    def sign_compress(self, g, e, out_bits, out_scales, u=None, momentum: float = 0.0,
                      stream=None):
        """1-bit sign compression with error feedback: bits (uint32 words, torch.int32
        storage) and one L1 scale per segment; e <- acc - sign * scale."""
        import torch
        n = self.n
        rc = self._L.gc_sign_ef_compress(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum),
            _dev_ptr(out_bits, torch.int32, "out_bits", self.total_words),
            _dev_ptr(out_scales, torch.float32, "out_scales", self.n_seg), _stream(stream))
        _check(rc, "gc_sign_ef_compress")

    def sign_decompress(self, bits, scales, dense, accumulate=False, stream=None):
        import torch
        rc = self._L.gc_sign_decompress(
            self._h, _dev_ptr(bits, torch.int32, "bits", self.total_words),
            _dev_ptr(scales, torch.float32, "scales", self.n_seg),
            _dev_ptr(dense, torch.float32, "dense", self.n), int(bool(accumulate)),
            _stream(stream))
        _check(rc, "gc_sign_decompress")

    def qsgd_compress(self, g, out_codes, out_norms, levels: int = 127, e=None, u=None,
                      momentum: float = 0.0, seed: int = 0, step: int = 0, stream=None):
        """QSGD with `levels` levels, one l2 norm per segment; with e, error feedback."""
        import torch
        n = self.n
        rc = self._L.gc_qsgd_compress(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum), int(levels),
            int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1),
            _dev_ptr(out_codes, torch.int8, "out_codes", n),
            _dev_ptr(out_norms, torch.float32, "out_norms", self.n_seg), _stream(stream))
        _check(rc, "gc_qsgd_compress")

    def qsgd_decompress(self, codes, norms, dense, levels: int = 127, accumulate=False,
                        stream=None):
        import torch
        rc = self._L.gc_qsgd_decompress(
            self._h, _dev_ptr(codes, torch.int8, "codes", self.n),
            _dev_ptr(norms, torch.float32, "norms", self.n_seg), int(levels),
            _dev_ptr(dense, torch.float32, "dense", self.n), int(bool(accumulate)),
            _stream(stream))
        _check(rc, "gc_qsgd_decompress")

    def clip_by_norm(self, g, max_norm, norms_out=None, stream=None):
        """Per segment: when ||g_s||_2 > max_norm[s], g_s *= max_norm[s] / ||g_s||_2 (in place).
        ``max_norm``: device float32[n_seg]; ``norms_out`` receives the norms before."""
        import torch
        rc = self._L.gc_clip_by_norm(
            self._h, _dev_ptr(g, torch.float32, "g", self.n),
            _dev_ptr(max_norm, torch.float32, "max_norm", self.n_seg),
            _dev_ptr(norms_out, torch.float32, "norms_out", self.n_seg), _stream(stream))
        _check(rc, "gc_clip_by_norm")

    def clip_factors(self, g, max_norm, factors_out, norms_out=None, stream=None):
        """Per segment f_s = max_norm[s] / ||g_s||_2 where the norm exceeds it, else 1."""
        import torch
        rc = self._L.gc_clip_factors(
            self._h, _dev_ptr(g, torch.float32, "g", self.n),
            _dev_ptr(max_norm, torch.float32, "max_norm", self.n_seg),
            _dev_ptr(norms_out, torch.float32, "norms_out", self.n_seg),
            _dev_ptr(factors_out, torch.float32, "factors_out", self.n_seg), _stream(stream))
        _check(rc, "gc_clip_factors")

    def set_gradient_scale(self, factors):
        """Later compress calls read x = g * factors[s] (device float32[n_seg]); None: off.
        The tensor is kept referenced while it is set."""
        import torch
        self._gscale = factors
        _check(self._L.gc_plan_set_gradient_scale(
            self._h, _dev_ptr(factors, torch.float32, "factors", self.n_seg)),
            "gc_plan_set_gradient_scale")

    def decompress_gathered(self, n_workers: int, idx, dense, vals=None, codes=None,
                            scales=None, accumulate=False, stream=None):
        """Add n_workers payloads (back to back in worker order) into dense, worker by worker."""
        import torch
        tk = self.total_k * n_workers
        rc = self._L.gc_decompress_gathered(
            self._h, int(n_workers), _dev_ptr(vals, torch.float32, "vals", tk),
            _dev_ptr(codes, torch.int8, "codes", tk),
            _dev_ptr(scales, torch.float32, "scales", self.n_seg * n_workers),
            _dev_ptr(idx, torch.int32, "idx", tk), _dev_ptr(dense, torch.float32, "dense", self.n),
            int(bool(accumulate)), _stream(stream))
        _check(rc, "gc_decompress_gathered")

    def threshold_compress(self, g, e, tau, out_vals, out_idx, out_count=None, u=None,
                           momentum: float = 0.0, stream=None):
        """Keep |acc| >= |tau_s|, at most k_s per segment (the largest); e <- the residual.

        ``tau``: device float32 tensor of n_seg thresholds.  Unused output slots get value 0
        and index -1; ``out_count`` (device int32[n_seg]) receives the kept counts.
        """
        import torch
        n = self.n
        rc = self._L.gc_threshold_ef_compress(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum),
            _dev_ptr(tau, torch.float32, "tau", self.n_seg),
            _dev_ptr(out_vals, torch.float32, "out_vals", self.total_k),
            _dev_ptr(out_idx, torch.int32, "out_idx", self.total_k),
            _dev_ptr(out_count, torch.int32, "out_count", self.n_seg), _stream(stream))
        _check(rc, "gc_threshold_ef_compress")

    def randk_compress(self, g, out_vals, out_idx, e=None, u=None, momentum: float = 0.0,
                       seed: int = 0, step: int = 0, stream=None):
        """Random-k: k_s uniformly random positions per segment (Philox keys of (seed, step,
        index)); with e, error feedback, else values scaled by n_s / k_s."""
        import torch
        n = self.n
        rc = self._L.gc_randk_compress(
            self._h, _dev_ptr(g, torch.float32, "g", n), _dev_ptr(e, torch.float32, "e", n),
            _dev_ptr(u, torch.float32, "u", n), float(momentum), int(seed) & (2 ** 64 - 1),
            int(step) & (2 ** 64 - 1),
            _dev_ptr(out_vals, torch.float32, "out_vals", self.total_k),
            _dev_ptr(out_idx, torch.int32, "out_idx", self.total_k), _stream(stream))
        _check(rc, "gc_randk_compress")

    def reset_estimate(self, stream=None):
        _check(self._L.gc_plan_reset_estimate(self._h, _stream(stream)), "gc_plan_reset_estimate")

    def last_stats(self, stream=None) -> dict:
        """Per-segment mode, candidate count, k-th key and ties of the last call (syncs)."""
        out = {name: np.zeros(self.n_seg, np.uint32)
               for name in ("mode", "candidates", "kth_key", "ties")}
        rc = self._L.gc_plan_last_stats(self._h, _np_ptr(out["mode"]), _np_ptr(out["candidates"]),
                                      _np_ptr(out["kth_key"]), _np_ptr(out["ties"]),
                                      _stream(stream))
        _check(rc, "gc_plan_last_stats")
        return out

    def set_timing(self, enable: bool = True):
        _check(self._L.gc_plan_set_timing(self._h, int(bool(enable))), "gc_plan_set_timing")

    def timing(self):
        """(milliseconds, launches) of the streaming pass since the last query."""
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(self._L.gc_plan_timing(self._h, ctypes.byref(ms), ctypes.byref(n)), "gc_plan_timing")
        return ms.value, n.value


def copy_f32(src, dst, stream=None):
    """Reference streaming copy (16-byte loads and stores) for bandwidth calibration."""
    import torch
    n = src.numel()
    _check(lib().gc_copy_f32(_dev_ptr(src, torch.float32, "src"),
                             _dev_ptr(dst, torch.float32, "dst", n), n, _stream(stream)),
           "gc_copy_f32")


def add_f32(x, y, stream=None):
    """y += x (fp32, in place) with the error-feedback pass's memory pattern: a reference
    two-read/one-write stream (not a ceiling: the pass streams faster than it)."""
    import torch
    n = x.numel()
    _check(lib().gc_add_f32(_dev_ptr(x, torch.float32, "x"), _dev_ptr(y, torch.float32, "y", n),
                            n, _stream(stream)), "gc_add_f32")


def read_f32(x, sink, stream=None):
    """A pure read stream over x (the pass's tile layout and non-temporal loads); sink is a
    device int32[64] that nothing is written to for real data."""
    import torch
    _check(lib().gc_read_f32(_dev_ptr(x, torch.float32, "x"), x.numel(),
                             _dev_ptr(sink, torch.int32, "sink", 64), _stream(stream)),
           "gc_read_f32")


__all__ = ["Plan", "GCError", "lib", "status_string", "copy_f32", "add_f32", "read_f32", "layout",
           "topk_ef_compress_noalloc", "EXPORTS",
           "GC_MOMENTUM_MASK", "GC_DEBUG_FORCE_FALLBACK", "GC_DEBUG_NO_ESTIMATE", "GC_DEBUG_CHAIN", "MODE_SKIP",
           "MODE_CANDIDATES", "MODE_FULL", "MODE_RECAPTURED", "MODE_SMALL", "SMALL_SEGMENT"]
