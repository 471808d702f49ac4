"""Build libvinf.so (HIP, gfx950) in-tree.

    python -m video_diffusion_temporal_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links them into
video_diffusion_temporal_amd/libvinf.so.  Packed fp32 VALU instructions are
disabled for all device code (the kernels use scalar fp32, bf16 dot2 and MFMA).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(PKG, "libvinf.so")
ARCH = "gfx950"
SOURCES = ["api.cpp", "groupnorm.hip", "temporal_conv3.hip", "dual_domain_attn.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libvinf)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, out_dir: str, extra: list[str]) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *common_flags(), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile and link libvinf.so; returns its path.  Always recompiles."""
    extra = list(extra or [])
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), SOURCES))
    tmp = SO + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libvinf.so failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SO)
    if verbose:
        print(f"built {SO}")
    return SO


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
