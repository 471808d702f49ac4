"""Python binding of libvinf (the Video-Infinity temporal module on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libvinf.so.  PyTorch supplies device memory and the current stream.
Call names match the C ABI in include/vinf.h:

    groupnorm_global(x, groups, eps=1e-5, ...)      -> (y, mean, rstd)
    temporal_conv3(x, weight, ctx_pre=None, ...)     -> y
    dual_domain_attn(q, k, v, ...)                   -> o

GroupNorm applied inside the conv (the normalised tensor is never written):

    groupnorm_stats(x, groups, eps=1e-5)                      -> (mean, rstd)
    temporal_conv3_gn(x, weight, mean, rstd, ...)             -> y = conv3(GroupNorm(x))

and the clip-parallel forms (one clip of a longer video plus its context):

    groupnorm_clip_sums(x, groups, F_total, mean_sums=None)  -> sums (float64 [groups])
    groupnorm_clip_apply(x, groups, F_total, sums, sq_sums)  -> (y, mean, rstd)
    dda_clip_halo(F_total, f0, Fc, n_local=16)               -> (n_pre, n_post)
    dual_domain_attn_clip(q, k, v, F_total, f0, n_pre, n_post, k_global, v_global) -> o

and the reuse of attention outputs across diffusion steps:

    attn_broadcast_schedule(n_steps, range)          -> list of 0/1 (1: the step computes)
    dual_domain_attn_broadcast(q, k, v, out, step, schedule)  -> out (recomputed or kept)

Tensors are CUDA (HIP) tensors, contiguous, channels-last [F, H, W, C],
float32 or bfloat16.  There is no CPU fallback: without the built library
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["groupnorm_global", "groupnorm_global_noalloc", "groupnorm_workspace_bytes", "temporal_conv3", "dual_domain_attn",
           "groupnorm_clip_sums", "groupnorm_clip_apply", "dda_clip_halo", "dual_domain_attn_clip", "groupnorm_stats",
           "temporal_conv3_gn", "temporal_conv3_gn_workspace_bytes", "attn_broadcast_schedule",
           "dual_domain_attn_broadcast", "VinfError",
           "library_path", "load", "VINF_F32", "VINF_BF16"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libvinf.so")

VINF_OK, VINF_ERR_INVALID_ARG, VINF_ERR_UNSUPPORTED, VINF_ERR_WORKSPACE, VINF_ERR_HIP = range(5)
VINF_F32, VINF_BF16 = 0, 1

_lib = None


class VinfError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libvinf.so (built by video_diffusion_temporal_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run `python -m video_diffusion_temporal_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.vinf_groupnorm_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.vinf_groupnorm_workspace_bytes.restype = sz
        L.vinf_groupnorm_global.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.vinf_temporal_conv3.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.vinf_dual_domain_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        L.vinf_groupnorm_clip_sums.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.vinf_groupnorm_clip_apply.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
        L.vinf_dda_clip_halo.argtypes = [i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.vinf_dual_domain_attn_clip.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, f, i, vp]
        L.vinf_groupnorm_stats.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.vinf_temporal_conv3_gn_workspace_bytes.argtypes = [i, i]
        L.vinf_temporal_conv3_gn_workspace_bytes.restype = sz
        L.vinf_temporal_conv3_gn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, vp, sz, vp]
        for fn in ("vinf_groupnorm_global", "vinf_temporal_conv3", "vinf_dual_domain_attn", "vinf_groupnorm_clip_sums",
                   "vinf_groupnorm_clip_apply", "vinf_dda_clip_halo", "vinf_dual_domain_attn_clip",
                   "vinf_groupnorm_stats", "vinf_temporal_conv3_gn"):
            getattr(L, fn).restype = ctypes.c_int
        L.vinf_qkv_project.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.vinf_projected_dual_domain_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        L.vinf_groupnorm_global_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.vinf_groupnorm_global_noalloc.restype = ctypes.c_int
        L.vinf_attn_broadcast_schedule.argtypes = [i, i, ctypes.c_char_p]
        L.vinf_attn_broadcast_schedule.restype = ctypes.c_int
        L.vinf_status_string.argtypes = [i]
        L.vinf_status_string.restype = ctypes.c_char_p
        L.vinf_last_error.argtypes = []
        L.vinf_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != VINF_OK:
        raise VinfError(fn, status, load().vinf_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return VINF_BF16
    if t.dtype == torch.float32:
        return VINF_F32
    raise TypeError(f"libvinf tensors are float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (channels-last [F,H,W,C] storage)")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _fhwc(x: torch.Tensor):
    if x.dim() != 4:
        raise ValueError(f"expected a [F,H,W,C] tensor, got shape {tuple(x.shape)}")
    return tuple(int(s) for s in x.shape)


def _same_device(t: torch.Tensor, x: torch.Tensor, name: str) -> None:
    if t.device != x.device:
        raise ValueError(f"{name} is on {t.device}, x on {x.device}")


def _out_like(out: torch.Tensor | None, x: torch.Tensor, name: str = "out") -> torch.Tensor:
    """A caller-supplied output tensor must be exactly x's shape, dtype and
    device and contiguous: the library only sees its pointer and writes x's
    size through it."""
    if out is None:
        return torch.empty_like(x)
    _dev(out, name)
    _same_device(out, x, name)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError(f"{name} must be {tuple(x.shape)} of {x.dtype}, got {tuple(out.shape)} of {out.dtype}")
    return out


def _vec(t: torch.Tensor | None, x: torch.Tensor, name: str, n: int,
         dtype: torch.dtype = torch.float32) -> torch.Tensor | None:
    """An optional per-channel or per-group vector: n contiguous values of dtype
    on x's device (the library reads or writes exactly n values)."""
    if t is None:
        return None
    _dev(t, name)
    _same_device(t, x, name)
    if t.dtype != dtype or t.numel() != n:
        raise ValueError(f"{name} must hold {n} values of {dtype}, got {t.numel()} of {t.dtype}")
    return t


def _vec_out(t: torch.Tensor | None, x: torch.Tensor, name: str, n: int) -> torch.Tensor:
    if t is None:
        return torch.empty(n, device=x.device, dtype=torch.float32)
    return _vec(t, x, name, n)


def _ws(workspace: torch.Tensor, x: torch.Tensor) -> int:
    """Bytes of a caller-supplied workspace on x's device."""
    _dev(workspace, "workspace")
    _same_device(workspace, x, "workspace")
    return workspace.numel() * workspace.element_size()


def groupnorm_workspace_bytes(F: int, H: int, W: int, C: int, groups: int, dtype: torch.dtype) -> int:
    code = VINF_BF16 if dtype == torch.bfloat16 else VINF_F32
    return int(load().vinf_groupnorm_workspace_bytes(F, H, W, C, groups, code))


def groupnorm_global(x: torch.Tensor, groups: int, eps: float = 1e-5, gamma: torch.Tensor | None = None,
                     beta: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     mean_out: torch.Tensor | None = None, rstd_out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None):
    """GroupNorm with whole-video statistics.  Returns (y, mean[groups], rstd[groups])."""
    _dev(x, "x")
    F, H, W, C = _fhwc(x)
    groups = int(groups)
    y = _out_like(out, x)
    mean = _vec_out(mean_out, x, "mean_out", groups)
    rstd = _vec_out(rstd_out, x, "rstd_out", groups)
    _vec(gamma, x, "gamma", C)
    _vec(beta, x, "beta", C)
    need = groupnorm_workspace_bytes(F, H, W, C, groups, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    ws_bytes = _ws(workspace, x)
    st = load().vinf_groupnorm_global(_ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), _ptr(mean), _ptr(rstd), F, H, W, C,
                                       groups, float(eps), _dtype_code(x), _ptr(workspace), ws_bytes,
                                       _stream(x.device, stream))
    _check("vinf_groupnorm_global", st)
    return y, mean, rstd


def _ctx(ctx_pre, ctx_post, x: torch.Tensor) -> None:
    F, H, W, C = _fhwc(x)
    for name, c in (("ctx_pre", ctx_pre), ("ctx_post", ctx_post)):
        if c is not None:
            _dev(c, name)
            _same_device(c, x, name)
            if c.numel() != H * W * C or c.dtype != x.dtype:
                raise ValueError(f"{name} must hold [H,W,C] = {H * W * C} values of {x.dtype}")


def groupnorm_global_noalloc(x: torch.Tensor, groups: int, eps: float = 1e-5, gamma: torch.Tensor | None = None,
                             beta: torch.Tensor | None = None, out: torch.Tensor | None = None,
                             mean_out: torch.Tensor | None = None, rstd_out: torch.Tensor | None = None, stream=None):
    """groupnorm_global with the library's static scratch as its workspace (no
    workspace argument, nothing allocated by the library).  Calls that overlap
    on one GPU race.  Returns (y, mean[groups], rstd[groups])."""
    _dev(x, "x")
    F, H, W, C = _fhwc(x)
    groups = int(groups)
    y = _out_like(out, x)
    mean = _vec_out(mean_out, x, "mean_out", groups)
    rstd = _vec_out(rstd_out, x, "rstd_out", groups)
    _vec(gamma, x, "gamma", C)
    _vec(beta, x, "beta", C)
    st = load().vinf_groupnorm_global_noalloc(_ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), _ptr(mean), _ptr(rstd), F, H,
                                              W, C, groups, float(eps), _dtype_code(x), _stream(x.device, stream))
    _check("vinf_groupnorm_global_noalloc", st)
    return y, mean, rstd


def temporal_conv3(x: torch.Tensor, weight: torch.Tensor, ctx_pre: torch.Tensor | None = None,
                   ctx_post: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Kernel-3 temporal conv with context padding; weight is [3, C_out, C_in]."""
    _dev(x, "x")
    _dev(weight, "weight")
    F, H, W, C = _fhwc(x)
    if tuple(weight.shape) != (3, C, C) or weight.dtype != x.dtype:
        raise ValueError(f"weight must be [3,{C},{C}] of {x.dtype}")
    _same_device(weight, x, "weight")
    _ctx(ctx_pre, ctx_post, x)
    _vec(bias, x, "bias", C)
    y = _out_like(out, x)
    st = load().vinf_temporal_conv3(_ptr(x), _ptr(ctx_pre), _ptr(ctx_post), _ptr(weight), _ptr(bias), _ptr(y), F, H,
                                     W, C, _dtype_code(x), _stream(x.device, stream))
    _check("vinf_temporal_conv3", st)
    return y


def dual_domain_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                     head_dim: int = 64, n_local: int = 16, n_global: int = 16, scale: float = 0.0,
                     stream=None) -> torch.Tensor:
    """Dual-domain temporal attention over [F,H,W,C] q/k/v (already projected)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name)
        _same_device(t, q, name)
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k and v must share shape and dtype")
    F, H, W, C = _fhwc(q)
    o = _out_like(out, q)
    st = load().vinf_dual_domain_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), F, H, W, C, head_dim, n_local, n_global,
                                       float(scale), _dtype_code(q), _stream(q.device, stream))
    _check("vinf_dual_domain_attn", st)
    return o


def qkv_project(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                out: tuple[torch.Tensor, torch.Tensor, torch.Tensor] | None = None,
                stream=None) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(q, k, v): the three C x C maps of weight [3, C_out, C_in] (bias [3, C]
    float32 or None) applied to every token of x [F, H, W, C]."""
    _dev(x, "x")
    _dev(weight, "weight")
    F, H, W, C = _fhwc(x)
    if tuple(weight.shape) != (3, C, C) or weight.dtype != x.dtype:
        raise ValueError(f"weight must be [3,{C},{C}] of {x.dtype}")
    _same_device(weight, x, "weight")
    _vec(bias, x, "bias", 3 * C)
    if out is None:
        out = tuple(torch.empty_like(x) for _ in range(3))
    if len(out) != 3:
        raise ValueError("out must be a (q, k, v) triple")
    q, k, v = (_out_like(t, x, n) for t, n in zip(out, "qkv"))
    st = load().vinf_qkv_project(_ptr(x), _ptr(weight), _ptr(bias), _ptr(q), _ptr(k), _ptr(v), F, H, W, C,
                                 _dtype_code(x), _stream(x.device, stream))
    _check("vinf_qkv_project", st)
    return q, k, v


def projected_dual_domain_attn(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                               out: torch.Tensor | None = None, qkv: tuple | None = None, head_dim: int = 64,
                               n_local: int = 16, n_global: int = 16, scale: float = 0.0,
                               stream=None) -> torch.Tensor:
    """Dual-domain attention over the projected tokens of x: vinf_qkv_project
    then vinf_dual_domain_attn on one stream.  qkv: optional (q, k, v) buffers
    shaped like x."""
    q, k, v = qkv_project(x, weight, bias, out=qkv, stream=stream)
    return dual_domain_attn(q, k, v, out=out, head_dim=head_dim, n_local=n_local, n_global=n_global, scale=scale,
                            stream=stream)


def projected_dual_domain_attn_fused(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                                     out: torch.Tensor | None = None, head_dim: int = 64, scale: float = 0.0,
                                     stream=None) -> torch.Tensor:
    """The same result as projected_dual_domain_attn (full key set, bf16), in one
    launch that never writes q, k and v (vinf_projected_dual_domain_attn)."""
    _dev(x, "x")
    _dev(weight, "weight")
    F, H, W, C = _fhwc(x)
    if tuple(weight.shape) != (3, C, C) or weight.dtype != x.dtype:
        raise ValueError(f"weight must be [3,{C},{C}] of {x.dtype}")
    _same_device(weight, x, "weight")
    _vec(bias, x, "bias", 3 * C)
    o = _out_like(out, x)
    st = load().vinf_projected_dual_domain_attn(_ptr(x), _ptr(weight), _ptr(bias), _ptr(o), F, H, W, C, head_dim,
                                                16, 16, float(scale), _dtype_code(x), _stream(x.device, stream))
    _check("vinf_projected_dual_domain_attn", st)
    return o


def _workspace(x: torch.Tensor, groups: int, workspace):
    F, H, W, C = _fhwc(x)
    need = groupnorm_workspace_bytes(F, H, W, C, groups, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    return workspace, _ws(workspace, x)


def _f64(t: torch.Tensor | None, name: str, groups: int, x: torch.Tensor | None = None):
    if t is None:
        return None
    _dev(t, name)
    if x is not None:
        _same_device(t, x, name)
    if t.dtype != torch.float64 or t.numel() != groups:
        raise ValueError(f"{name} must be float64 [{groups}]")
    return t


def groupnorm_clip_sums(x: torch.Tensor, groups: int, F_total: int, mean_sums: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """One clip's float64 group sums: of x (mean_sums None) or of (x - mean)^2
    with mean = mean_sums / N_g, where mean_sums holds the first sums of all
    clips added together and N_g counts the whole video's F_total frames."""
    _dev(x, "x")
    F, H, W, C = _fhwc(x)
    groups = int(groups)
    _f64(mean_sums, "mean_sums", groups, x)
    sums = torch.empty(groups, device=x.device, dtype=torch.float64) if out is None else _f64(out, "out", groups, x)
    workspace, ws_bytes = _workspace(x, groups, workspace)
    st = load().vinf_groupnorm_clip_sums(_ptr(x), _ptr(mean_sums), _ptr(sums), F, H, W, C, groups, int(F_total),
                                          _dtype_code(x), _ptr(workspace), ws_bytes, _stream(x.device, stream))
    _check("vinf_groupnorm_clip_sums", st)
    return sums


def groupnorm_clip_apply(x: torch.Tensor, groups: int, F_total: int, sums: torch.Tensor, sq_sums: torch.Tensor,
                         eps: float = 1e-5, gamma: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, mean_out: torch.Tensor | None = None,
                         rstd_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stats_only: bool = False, stream=None):
    """Normalise one clip with the statistics of the all-clip sums.  Returns (y, mean, rstd);
    with stats_only=True only the statistics are computed (y is None)."""
    _dev(x, "x")
    F, H, W, C = _fhwc(x)
    groups = int(groups)
    if sums is None or sq_sums is None:
        raise ValueError("sums and sq_sums are required")
    _f64(sums, "sums", groups, x)
    _f64(sq_sums, "sq_sums", groups, x)
    y = None if stats_only else _out_like(out, x)
    mean = _vec_out(mean_out, x, "mean_out", groups)
    rstd = _vec_out(rstd_out, x, "rstd_out", groups)
    _vec(gamma, x, "gamma", C)
    _vec(beta, x, "beta", C)
    workspace, ws_bytes = _workspace(x, groups, workspace)
    st = load().vinf_groupnorm_clip_apply(None if stats_only else _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta),
                                           _ptr(sums), _ptr(sq_sums), _ptr(mean), _ptr(rstd), F, H, W, C, groups,
                                           int(F_total), float(eps), _dtype_code(x), _ptr(workspace), ws_bytes,
                                           _stream(x.device, stream))
    _check("vinf_groupnorm_clip_apply", st)
    return y, mean, rstd


def groupnorm_stats(x: torch.Tensor, groups: int, eps: float = 1e-5, mean_out: torch.Tensor | None = None,
                    rstd_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Whole-video GroupNorm statistics only (the two sweeps).  Returns (mean[groups], rstd[groups])."""
    _dev(x, "x")
    F, H, W, C = _fhwc(x)
    groups = int(groups)
    mean = _vec_out(mean_out, x, "mean_out", groups)
    rstd = _vec_out(rstd_out, x, "rstd_out", groups)
    workspace, ws_bytes = _workspace(x, groups, workspace)
    st = load().vinf_groupnorm_stats(_ptr(x), _ptr(mean), _ptr(rstd), F, H, W, C, groups, float(eps), _dtype_code(x),
                                     _ptr(workspace), ws_bytes, _stream(x.device, stream))
    _check("vinf_groupnorm_stats", st)
    return mean, rstd


def temporal_conv3_gn_workspace_bytes(C: int, dtype: torch.dtype) -> int:
    return int(load().vinf_temporal_conv3_gn_workspace_bytes(C, VINF_BF16 if dtype == torch.bfloat16 else VINF_F32))


def temporal_conv3_gn(x: torch.Tensor, weight: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor,
                      gamma: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                      ctx_pre: torch.Tensor | None = None, ctx_post: torch.Tensor | None = None,
                      bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """conv3(GroupNorm(x)) with the given statistics (mean, rstd: float32 [groups]); x and
    the context frames are raw (not normalised).  Bit for bit groupnorm apply + temporal_conv3."""
    _dev(x, "x")
    _dev(weight, "weight")
    F, H, W, C = _fhwc(x)
    if tuple(weight.shape) != (3, C, C) or weight.dtype != x.dtype:
        raise ValueError(f"weight must be [3,{C},{C}] of {x.dtype}")
    _same_device(weight, x, "weight")
    _ctx(ctx_pre, ctx_post, x)
    for name, v in (("mean", mean), ("rstd", rstd)):
        _dev(v, name)
        if v.dtype != torch.float32 or v.dim() != 1:
            raise ValueError(f"{name} must be float32 [groups]")
    groups = int(mean.numel())
    _vec(rstd, x, "rstd", groups)
    _vec(mean, x, "mean", groups)
    _vec(gamma, x, "gamma", C)
    _vec(beta, x, "beta", C)
    _vec(bias, x, "bias", C)
    y = _out_like(out, x)
    need = temporal_conv3_gn_workspace_bytes(C, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    ws_bytes = _ws(workspace, x)
    st = load().vinf_temporal_conv3_gn(_ptr(x), _ptr(ctx_pre), _ptr(ctx_post), _ptr(weight), _ptr(bias), _ptr(mean),
                                       _ptr(rstd), _ptr(gamma), _ptr(beta), groups, _ptr(y), F, H, W, C,
                                       _dtype_code(x), _ptr(workspace), ws_bytes, _stream(x.device, stream))
    _check("vinf_temporal_conv3_gn", st)
    return y


def dda_clip_halo(F_total: int, f0: int, Fc: int, n_local: int = 16) -> tuple[int, int]:
    """Frames before and after the clip [f0, f0+Fc) that its local windows reach."""
    pre, post = ctypes.c_int(), ctypes.c_int()
    st = load().vinf_dda_clip_halo(int(F_total), int(f0), int(Fc), int(n_local), ctypes.byref(pre),
                                   ctypes.byref(post))
    _check("vinf_dda_clip_halo", st)
    return pre.value, post.value


def dual_domain_attn_clip(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, F_total: int, f0: int, n_pre: int,
                          n_post: int, k_global: torch.Tensor | None = None, v_global: torch.Tensor | None = None,
                          out: torch.Tensor | None = None, head_dim: int = 64, n_local: int = 16,
                          n_global: int = 16, scale: float = 0.0, stream=None) -> torch.Tensor:
    """Attention of query frames f0 .. f0+Fc-1 (q: [Fc,H,W,C]) of an F_total-frame
    video; k, v: [n_pre+Fc+n_post, H, W, C] (the clip with its context);
    k_global, v_global: [n_global, H, W, C] frames floor(i*F_total/16) or None."""
    _dev(q, "q")
    Fc, H, W, C = _fhwc(q)
    for name, t in (("k", k), ("v", v)):
        _dev(t, name)
        _same_device(t, q, name)
        if tuple(t.shape) != (n_pre + Fc + n_post, H, W, C) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [{n_pre + Fc + n_post},{H},{W},{C}] of {q.dtype}")
    for name, t in (("k_global", k_global), ("v_global", v_global)):
        if t is not None:
            _dev(t, name)
            _same_device(t, q, name)
            if tuple(t.shape) != (n_global, H, W, C) or t.dtype != q.dtype:
                raise ValueError(f"{name} must be [{n_global},{H},{W},{C}] of {q.dtype}")
    o = _out_like(out, q)
    st = load().vinf_dual_domain_attn_clip(_ptr(q), _ptr(k), _ptr(v), _ptr(k_global), _ptr(v_global), _ptr(o),
                                            int(F_total), int(f0), Fc, int(n_pre), int(n_post), H, W, C, head_dim,
                                            n_local, n_global, float(scale), _dtype_code(q),
                                            _stream(q.device, stream))
    _check("vinf_dual_domain_attn_clip", st)
    return o


def attn_broadcast_schedule(n_steps: int, range_: int) -> list[int]:
    """1 for a diffusion step that computes its temporal attention, 0 for one that reuses the latest output."""
    buf = ctypes.create_string_buffer(max(int(n_steps), 1))
    st = load().vinf_attn_broadcast_schedule(int(n_steps), int(range_), buf)
    _check("vinf_attn_broadcast_schedule", st)
    return list(buf.raw[:n_steps])


def dual_domain_attn_broadcast(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, step: int,
                               schedule, **kw) -> torch.Tensor:
    """Diffusion step `step` of a broadcast schedule: on a computing step, the
    attention of q, k, v into `out`; on a reuse step nothing is launched and
    `out` keeps the latest computed output."""
    if schedule[step]:
        dual_domain_attn(q, k, v, out=out, **kw)
    return out
