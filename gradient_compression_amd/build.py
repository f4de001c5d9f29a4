"""Build the HIP library libgc.so (gfx950 only) next to this file.

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
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("gc_topk.hip", "gc_codecs.hip", "gc_scatter.hip",
                                                       "gc_api.hip")]
ARCH = "gfx950"


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


if __name__ == "__main__":
    print(build(verbose=True))
