"""Build libslim.so (gfx950) in-tree with hipcc.

The translation units are compiled in parallel into _build/ and linked into
causal_linear_attention_amd/libslim.so.  All HIP code is built with packed
fp32 instructions disabled (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libslim.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["slim_bf16_favor.hip", "slim_f32_favor.hip", "slim_bf16_favor_dw.hip", "slim_f32_favor_dw.hip",
           "slim_f32_elu1.hip", "slim_bf16_elu1.hip", "slim_host.hip"]

# -amdgpu-use-amdgpu-trackers: the scheduler's AMDGPU register-pressure tracking; it
# spills less in the dQ kernel at 64 features (1.30 -> 1.17 ms on 1M tokens x 8 heads)
# and changes nothing measurable at the 16K-token, 64-head shape.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-use-amdgpu-trackers=1",
          "-I", os.path.join(ROOT, "include")]


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return out


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libslim.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    args = sys.argv[1:]
    build(verbose="-v" in args, extra=[a for a in args if a != "-v"])
    print(LIB)
