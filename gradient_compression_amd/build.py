"""Build the HIP library libgc.so (gfx950 only) next to this file, and the same library at
other tile geometries (libgc_<name>.so, see VARIANTS) for the tests that check that no result
depends on the geometry.

Flags that the results depend on:
  -ffp-contract=off                  no fused multiply-add: u = fl(fl(m*u) + g)
  -fno-gpu-flush-denormals-to-zero   fp32 denormals are kept
  -fhip-fp32-correctly-rounded-divide-sqrt   |v| / scale is correctly rounded
  -target-feature -packed-fp32-ops   no packed fp32 instructions
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgc.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("gc_pass.hip", "gc_topk.hip", "gc_codecs.hip",
                                                       "gc_scatter.hip", "gc_api.hip")]
ARCH = "gfx950"

# Tile geometries besides the default (1024 threads x 2 slots, 8192-element tiles).  A tile is
# threads * 4 * slots elements; a different geometry moves every tile, chunk and run boundary,
# the cold-start sample and the order of the per-tile partial sums.
VARIANTS = {
    "t512s4": ("GC_TILE_THREADS=512", "GC_TILE_SLOTS=4"),    # 8192 elements, 8 waves
    "t1024s1": ("GC_TILE_THREADS=1024", "GC_TILE_SLOTS=1"),  # 4096 elements, 16 waves
    "t256s2": ("GC_TILE_THREADS=256", "GC_TILE_SLOTS=2"),    # 2048 elements, 4 waves
}


def variant_path(name: str) -> str:
    if name not in VARIANTS:
        raise KeyError(f"unknown tile geometry {name!r}; built ones: {sorted(VARIANTS)}")
    return os.path.join(HERE, f"libgc_{name}.so")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
            "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libgc.so; ``defines`` (e.g. "GC_TILE_SLOTS=4") override the compile-time
    configuration of the streaming pass."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(), *[f"-D{d}" for d in defines], *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    """libgc.so and every VARIANTS geometry (the hipcc runs in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(LIB, ())] + [(variant_path(n), d) for n, d in VARIANTS.items()]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        futs = [ex.submit(build, verbose, out, d) for out, d in jobs]
        return [f.result() for f in futs]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
