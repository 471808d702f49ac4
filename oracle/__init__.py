"""CPU oracle of the temporal module -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  It wraps ``oracle.c`` (plain fp64 C, see
``oracle.h`` for the passages each routine follows) with ctypes over numpy
arrays.  Inputs are float32 arrays (dt = F32), uint16 bf16 bit patterns
(dt = BF16) or float64 arrays (dt = F64, e.g. an unrounded intermediate)
shaped [F, H, W, C] (or [F, S, C]); outputs are float64 arrays
[F, n_locs, C] for the requested spatial locations (flattened h*W + w).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2
_i64p = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread",
                           os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, d, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        L.oracle_gn_stats.argtypes = [vp, i, i64, i64, i64, i64, d, vp, vp, vp, i]
        L.oracle_groupnorm.argtypes = [vp, i, i64, i64, i64, i64, d, vp, vp, vp, i64, vp, vp, vp, i]
        L.oracle_conv3.argtypes = [vp, vp, vp, vp, vp, i, i64, i64, i64, vp, i64, vp, i]
        L.oracle_dda_keys.argtypes = [i64, i64, i, i, vp]
        L.oracle_dda.argtypes = [vp, vp, vp, i, i64, i64, i64, i, i, i, d, vp, i64, vp, i]
        L.oracle_gn_clip_sums.argtypes = [vp, i, i64, i64, i64, i64, vp, vp, i]
        L.oracle_dda_clip.argtypes = [vp, vp, vp, vp, vp, i, i64, i64, i64, i64, i64, i64, i64, i, i, i, d, vp, i64,
                                      vp, i]
        L.oracle_chain.argtypes = [vp, vp, i, i64, i64, i64, i64, d, i, i, i, d, i, vp, i64, vp, vp, vp, vp, vp, vp,
                                   vp, i]
        L.oracle_qkv_project.argtypes = [vp, vp, vp, i, i64, i64, i64, vp, i64, vp, i]
        L.oracle_qkv_dda.argtypes = [vp, vp, vp, i, i64, i64, i64, i, i, i, d, vp, i64, vp, vp, i]
        L.oracle_broadcast_schedule.argtypes = [i, i, vp]
        L.oracle_broadcast_schedule.restype = ctypes.c_int
        L.oracle_round_to.argtypes = [d, i]
        L.oracle_round_to.restype = d
        for fn in ("oracle_gn_stats", "oracle_groupnorm", "oracle_conv3", "oracle_dda_keys", "oracle_dda",
                   "oracle_chain", "oracle_gn_clip_sums", "oracle_dda_clip", "oracle_qkv_project",
                   "oracle_qkv_dda"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, uint16 bf16 bits or float64, got {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _locs(locs, S):
    if locs is None:
        locs = np.arange(S, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(locs, dtype=np.int64))


def _fsc(x):
    if x.ndim == 4:
        F, H, W, C = x.shape
        return F, H * W, C
    F, S, C = x.shape
    return F, S, C


def gn_stats(x, G, eps=1e-5, nthreads=0):
    """(mean[G], var[G], rstd[G]) over the whole tensor, fp64."""
    x = _c(x)
    F, S, C = _fsc(x)
    mean, var, rstd = (np.empty(G) for _ in range(3))
    rc = lib().oracle_gn_stats(_ptr(x), _dt(x), F, S, C, G, eps, _ptr(mean), _ptr(var), _ptr(rstd), nthreads)
    if rc:
        raise ValueError(f"oracle_gn_stats rc={rc}")
    return mean, var, rstd


def gn_clip_sums(x, G, mean=None, nthreads=0):
    """sums[G] (fp64) of one clip: of x (mean None) or of (x - mean[g])^2."""
    x = _c(x)
    F, S, C = _fsc(x)
    m = None if mean is None else np.ascontiguousarray(mean, dtype=np.float64)
    assert m is None or m.size == G
    sums = np.empty(G)
    rc = lib().oracle_gn_clip_sums(_ptr(x), _dt(x), F, S, C, G, _ptr(m), _ptr(sums), nthreads)
    if rc:
        raise ValueError(f"oracle_gn_clip_sums rc={rc}")
    return sums


def groupnorm(x, G, eps=1e-5, gamma=None, beta=None, locs=None, nthreads=0):
    """(y[F, n_locs, C], mean[G], rstd[G])."""
    x = _c(x)
    F, S, C = _fsc(x)
    locs = _locs(locs, S)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float64)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float64)
    y = np.empty((F, locs.size, C))
    mean, rstd = np.empty(G), np.empty(G)
    rc = lib().oracle_groupnorm(_ptr(x), _dt(x), F, S, C, G, eps, _ptr(g), _ptr(b), _ptr(locs), locs.size,
                                _ptr(y), _ptr(mean), _ptr(rstd), nthreads)
    if rc:
        raise ValueError(f"oracle_groupnorm rc={rc}")
    return y, mean, rstd


def conv3(x, w, ctx_pre=None, ctx_post=None, bias=None, locs=None, nthreads=0):
    """y[F, n_locs, C] of the kernel-3 temporal conv; w is [3, C_out, C_in]."""
    x, w, ctx_pre, ctx_post = _c(x), _c(w), _c(ctx_pre), _c(ctx_post)
    F, S, C = _fsc(x)
    assert w.shape == (3, C, C) and w.dtype == x.dtype
    for c in (ctx_pre, ctx_post):
        assert c is None or (c.size == S * C and c.dtype == x.dtype)
    locs = _locs(locs, S)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    y = np.empty((F, locs.size, C))
    rc = lib().oracle_conv3(_ptr(x), _ptr(ctx_pre), _ptr(ctx_post), _ptr(w), _ptr(b), _dt(x), F, S, C,
                            _ptr(locs), locs.size, _ptr(y), nthreads)
    if rc:
        raise ValueError(f"oracle_conv3 rc={rc}")
    return y


def dda_keys(F, t, n_local=16, n_global=16):
    keys = np.empty(n_local + n_global, dtype=np.int64)
    n = lib().oracle_dda_keys(F, t, n_local, n_global, _ptr(keys))
    return keys[:n].copy()


def dda(q, k, v, head_dim=64, n_local=16, n_global=16, scale=0.0, locs=None, nthreads=0):
    """o[F, n_locs, C] of dual-domain attention (scale <= 0 means 1/sqrt(head_dim))."""
    q, k, v = _c(q), _c(k), _c(v)
    F, S, C = _fsc(q)
    assert k.shape == q.shape == v.shape and k.dtype == q.dtype == v.dtype
    locs = _locs(locs, S)
    o = np.empty((F, locs.size, C))
    rc = lib().oracle_dda(_ptr(q), _ptr(k), _ptr(v), _dt(q), F, S, C, head_dim, n_local, n_global, scale,
                          _ptr(locs), locs.size, _ptr(o), nthreads)
    if rc:
        raise ValueError(f"oracle_dda rc={rc}")
    return o


def dda_clip(q, k, v, F_total, f0, kf0, k_glob=None, v_glob=None, head_dim=64, n_local=16, n_global=16,
             scale=0.0, locs=None, nthreads=0):
    """o[Fc, n_locs, C] for query frames f0 .. f0+Fc-1 of an F_total-frame video.

    q is [Fc, ...]; k, v hold frames kf0 .. kf0+len(k)-1; k_glob, v_glob hold
    the global frames floor(i*F_total/n_global) (None: read from k, v)."""
    q, k, v, kg, vg = _c(q), _c(k), _c(v), _c(k_glob), _c(v_glob)
    Fc, S, C = _fsc(q)
    n_ext = _fsc(k)[0]
    assert k.shape == v.shape and k.dtype == v.dtype == q.dtype and _fsc(k)[1:] == (S, C)
    assert (kg is None) == (vg is None)
    if kg is not None:
        assert kg.shape == vg.shape and _fsc(kg) == (n_global, S, C) and kg.dtype == q.dtype == vg.dtype
    locs = _locs(locs, S)
    o = np.empty((Fc, locs.size, C))
    rc = lib().oracle_dda_clip(_ptr(q), _ptr(k), _ptr(v), _ptr(kg), _ptr(vg), _dt(q), F_total, f0, Fc, kf0, n_ext,
                               S, C, head_dim, n_local, n_global, scale, _ptr(locs), locs.size, _ptr(o), nthreads)
    if rc:
        raise ValueError(f"oracle_dda_clip rc={rc}")
    return o


def chain(x, w, G, eps=1e-5, head_dim=64, n_local=16, n_global=16, scale=0.0, locs=None, nthreads=0,
          intermediates=False, exact=False, round_gn=True):
    """GroupNorm -> conv3 -> dual-domain attention (Q = K = V), at sampled locations.

    Returns (out, mean, rstd); with intermediates=True (out, gn, conv, mean,
    rstd) where gn and conv are the rounded intermediates; with exact=True
    also (gn_exact, conv_exact), the intermediates before rounding.
    round_gn=False: GroupNorm folded into the conv, so the conv reads the
    exact GroupNorm output (gn is then that exact output).
    """
    x, w = _c(x), _c(w)
    F, S, C = _fsc(x)
    locs = _locs(locs, S)
    out = np.empty((F, locs.size, C))
    want = intermediates or exact
    gn = np.empty_like(out) if want else None
    cv = np.empty_like(out) if want else None
    gx = np.empty_like(out) if exact else None
    cx = np.empty_like(out) if exact else None
    mean, rstd = np.empty(G), np.empty(G)
    rc = lib().oracle_chain(_ptr(x), _ptr(w), _dt(x), F, S, C, G, eps, head_dim, n_local, n_global, scale,
                            1 if round_gn else 0, _ptr(locs), locs.size, _ptr(out), _ptr(gn), _ptr(cv), _ptr(gx), _ptr(cx), _ptr(mean),
                            _ptr(rstd), nthreads)
    if rc:
        raise ValueError(f"oracle_chain rc={rc}")
    if exact:
        return out, gn, cv, gx, cx, mean, rstd
    if intermediates:
        return out, gn, cv, mean, rstd
    return out, mean, rstd


def qkv_project(x, w, bias=None, locs=None, nthreads=0):
    """out[3, F, n_locs, C]: Q, K and V of every token; w is [3, C_out, C_in], bias [3, C] or None."""
    x, w = _c(x), _c(w)
    F, S, C = _fsc(x)
    assert w.shape == (3, C, C) and w.dtype == x.dtype
    locs = _locs(locs, S)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64).reshape(3 * C)
    out = np.empty((3, F, locs.size, C))
    rc = lib().oracle_qkv_project(_ptr(x), _ptr(w), _ptr(b), _dt(x), F, S, C, _ptr(locs), locs.size, _ptr(out),
                                  nthreads)
    if rc:
        raise ValueError(f"oracle_qkv_project rc={rc}")
    return out


def qkv_dda(x, w, bias=None, head_dim=64, n_local=16, n_global=16, scale=0.0, locs=None, nthreads=0,
            intermediates=False):
    """Projection -> Q, K, V rounded to the I/O type -> dual-domain attention.

    Returns o[F, n_locs, C]; with intermediates=True (o, qkv) where qkv
    [3, F, n_locs, C] holds the rounded Q, K and V the attention read."""
    x, w = _c(x), _c(w)
    F, S, C = _fsc(x)
    assert w.shape == (3, C, C) and w.dtype == x.dtype
    locs = _locs(locs, S)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64).reshape(3 * C)
    out = np.empty((F, locs.size, C))
    qkv = np.empty((3, F, locs.size, C)) if intermediates else None
    rc = lib().oracle_qkv_dda(_ptr(x), _ptr(w), _ptr(b), _dt(x), F, S, C, head_dim, n_local, n_global, scale,
                              _ptr(locs), locs.size, _ptr(out), _ptr(qkv), nthreads)
    if rc:
        raise ValueError(f"oracle_qkv_dda rc={rc}")
    return (out, qkv) if intermediates else out


def broadcast_schedule(n_steps, range_):
    """recompute[n_steps] (0/1 uint8): which diffusion steps compute their temporal attention."""
    out = np.empty(n_steps, dtype=np.uint8)
    rc = lib().oracle_broadcast_schedule(int(n_steps), int(range_), _ptr(out))
    if rc:
        raise ValueError(f"oracle_broadcast_schedule rc={rc}")
    return out


def round_to(v: float, dt: int) -> float:
    return lib().oracle_round_to(float(v), int(dt))
