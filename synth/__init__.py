"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

The numbers come from ``gen.c`` (counter-based SplitMix64 + Box-Muller, see its
header); this module only builds that file, calls it and describes the
workloads.  It holds none of the temporal module's arithmetic, and imports
neither the oracle nor the HIP binding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16 = 0, 1


def build() -> str:
    """Compile gen.c into libsynth.so next to it (always recompiles)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", os.path.join(_HERE, "gen.c"),
         "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        L.synth_normal.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_double, ctypes.c_uint64, ctypes.c_double, ctypes.c_int]
        L.synth_normal.restype = ctypes.c_int
        L.synth_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.synth_splitmix64.restype = ctypes.c_uint64
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def normal(n: int, seed: int, dtype: int = BF16, scale: float = 1.0, frame_elems: int = 0,
           frame_slope: float = 0.0, nthreads: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """n values ``scale*z + frame_slope*(e // frame_elems)``, z ~ N(0,1).

    Returns float32, or uint16 bf16 bit patterns when ``dtype == BF16``.
    """
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(int(n), dtype=npdt)
    assert out.dtype == npdt and out.size == n and out.flags.c_contiguous
    rc = lib().synth_normal(out.ctypes.data, int(n), int(dtype), int(seed) & (2**64 - 1), float(scale),
                            int(frame_elems), float(frame_slope), int(nthreads))
    if rc != 0:
        raise RuntimeError("synth_normal failed")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def seed_for(config: int, tensor_id: int) -> int:
    """Seed of tensor ``tensor_id`` (Q=0, K=1, V=2, X_gn=3, X_conv=4, W=5, ctx_pre=6, ctx_post=7,
    W_qkv=8)."""
    return 0x5EED0000 + 16 * config + tensor_id


Q, K, V, X_GN, X_CONV, W, CTX_PRE, CTX_POST, W_QKV = range(9)

# Workloads.  Shapes are those of VideoCrafter2 latents at 512x320 (64x40 at
# the top level, 32x20x640 and 16x10x1280 further down), frame counts 16, 128,
# 1024 and 2300.  "m1024" is the throughput shape (F=1024 at 64x40x320).
CONFIGS = {
    1: dict(name="c1_tiny_f32", F=16, H=8, W=5, C=64, G=8, dtype=F32, slope=0.0, chain=False),
    2: dict(name="c2_f128_64x40x320", F=128, H=64, W=40, C=320, G=32, dtype=BF16, slope=0.0, chain=False),
    3: dict(name="c3_f1024_32x20x640", F=1024, H=32, W=20, C=640, G=32, dtype=BF16, slope=0.0, chain=False),
    4: dict(name="c4_f2300_16x10x1280", F=2300, H=16, W=10, C=1280, G=32, dtype=BF16, slope=0.3, chain=False),
    5: dict(name="c5_chain_f2300_64x40x320", F=2300, H=64, W=40, C=320, G=32, dtype=BF16, slope=0.0, chain=True),
    6: dict(name="m1024_f1024_64x40x320", F=1024, H=64, W=40, C=320, G=32, dtype=BF16, slope=0.0, chain=True),
}


def make_tensor(config: int, tensor_id: int, F: int, H: int, W: int, C: int, dtype: int,
                slope: float = 0.0, nthreads: int = 0) -> np.ndarray:
    """A [F,H,W,C] input: N(0,1), plus ``slope*t/F`` on frame t when slope != 0."""
    n = F * H * W * C
    fe = H * W * C if slope else 0
    return normal(n, seed_for(config, tensor_id), dtype, 1.0, fe, (slope / F) if slope else 0.0,
                  nthreads).reshape(F, H, W, C)


def make_conv_weight(config: int, C: int, dtype: int, nthreads: int = 0) -> np.ndarray:
    """[3][C_out][C_in] weights with variance 1/(3C)."""
    return normal(3 * C * C, seed_for(config, W), dtype, (1.0 / (3.0 * C)) ** 0.5, 0, 0.0,
                  nthreads).reshape(3, C, C)


def make_qkv_weight(config: int, C: int, dtype: int, nthreads: int = 0) -> np.ndarray:
    """[3][C_out][C_in] Q/K/V projection weights with variance 1/C (a token of
    unit variance maps to unit variance)."""
    return normal(3 * C * C, seed_for(config, W_QKV), dtype, (1.0 / C) ** 0.5, 0, 0.0,
                  nthreads).reshape(3, C, C)


def make_ctx(config: int, tensor_id: int, H: int, W: int, C: int, dtype: int) -> np.ndarray:
    """A [H,W,C] context frame (ctx_pre or ctx_post), N(0,1)."""
    return normal(H * W * C, seed_for(config, tensor_id), dtype).reshape(H, W, C)
