"""The C ABI without a GPU: the library loads, exports what include/vinf.h
declares, and rejects bad arguments on the host before any HIP call.

The pointers passed here are fake addresses: every call below fails
validation, which runs before anything touches the device.
"""
import ctypes
import os
import re

import pytest

import video_diffusion_temporal_amd as vinf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = range(5)
F32, BF16 = 0, 1

# 256-byte aligned fake device addresses, far apart
A, B, Cp, D, E, Fp, G = (0x10000000000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "vinf.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vinf_[a-z0-9_]+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert os.path.exists(vinf.library_path)
    vinf.load()


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"vinf_groupnorm_global", "vinf_temporal_conv3", "vinf_dual_domain_attn",
                          "vinf_groupnorm_workspace_bytes", "vinf_status_string", "vinf_last_error",
                          "vinf_groupnorm_clip_sums", "vinf_groupnorm_clip_apply", "vinf_dda_clip_halo",
                          "vinf_dual_domain_attn_clip", "vinf_qkv_project", "vinf_projected_dual_domain_attn"}
    lib = ctypes.CDLL(vinf.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    L = vinf.load()
    for s in range(5):
        assert L.vinf_status_string(s)
    assert L.vinf_status_string(99) == b"unknown status"


def test_groupnorm_workspace_bytes():
    L = vinf.load()
    n = L.vinf_groupnorm_workspace_bytes(1024, 64, 40, 320, 32, BF16)
    assert n >= 2048 * 320 * 4 + 2 * 32 * 4
    assert n % 256 == 0
    assert L.vinf_groupnorm_workspace_bytes(16, 8, 5, 64, 8, F32) > 0
    assert L.vinf_groupnorm_workspace_bytes(16, 8, 5, 64, 7, F32) == 0  # C % groups
    assert L.vinf_groupnorm_workspace_bytes(0, 8, 5, 64, 8, F32) == 0
    # fewer rows than blocks: the block count shrinks with the tensor
    assert L.vinf_groupnorm_workspace_bytes(1, 1, 1, 64, 8, F32) < n


def attn(**kw):
    a = dict(q=A, k=B, v=Cp, o=D, F=16, H=8, W=5, C=64, hd=64, nl=16, ng=16, scale=0.0, dt=BF16)
    a.update(kw)
    L = vinf.load()
    return L.vinf_dual_domain_attn(a["q"], a["k"], a["v"], a["o"], a["F"], a["H"], a["W"], a["C"], a["hd"], a["nl"],
                                   a["ng"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(q=A + 8), INVALID), (dict(o=D + 2), INVALID),
    (dict(F=0), INVALID), (dict(H=-1), INVALID), (dict(W=0), INVALID), (dict(C=0), INVALID),
    (dict(C=96), INVALID),                       # not a multiple of head_dim
    (dict(hd=32, C=64), UNSUPPORTED), (dict(nl=8), UNSUPPORTED), (dict(ng=32), UNSUPPORTED),
    (dict(nl=0, ng=0), UNSUPPORTED), (dict(nl=-16), UNSUPPORTED),
    (dict(C=68), UNSUPPORTED),                   # not a multiple of 8 (bf16 vectors)
    (dict(dt=7), INVALID),
    (dict(o=A), INVALID), (dict(o=B + 256), INVALID),  # o overlaps q / k
    (dict(scale=float("nan")), INVALID),
    (dict(F=1, H=1024, W=1 << 20, C=128), UNSUPPORTED),   # 2^31 (location, head) strips
])
def test_attention_rejects(kw, status):
    assert attn(**kw) == status
    assert vinf.load().vinf_last_error()


def conv(**kw):
    a = dict(x=A, pre=None, post=None, w=B, bias=None, y=Cp, F=16, H=8, W=5, C=64, dt=BF16)
    a.update(kw)
    return vinf.load().vinf_temporal_conv3(a["x"], a["pre"], a["post"], a["w"], a["bias"], a["y"], a["F"], a["H"],
                                           a["W"], a["C"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(x=A + 4), INVALID), (dict(pre=D + 8), INVALID), (dict(post=E + 1), INVALID), (dict(bias=Fp + 2), INVALID),
    (dict(F=0), INVALID), (dict(C=-8), INVALID),
    (dict(C=48), UNSUPPORTED),                    # bf16 needs C % 32 == 0
    (dict(C=6, dt=F32), UNSUPPORTED),             # f32 needs C % 4 == 0
    (dict(y=A), INVALID), (dict(y=A + 16 * 40 * 64 * 2 - 16), INVALID),   # y overlaps x
    (dict(y=B), INVALID), (dict(pre=D, y=D + 64), INVALID),            # y overlaps weight / ctx
])
def test_conv_rejects(kw, status):
    assert conv(**kw) == status


def proj(**kw):
    a = dict(x=A, w=B, bias=None, q=Cp, k=D, v=E, F=16, H=8, W=5, C=64, dt=BF16)
    a.update(kw)
    return vinf.load().vinf_qkv_project(a["x"], a["w"], a["bias"], a["q"], a["k"], a["v"], a["F"], a["H"], a["W"],
                                        a["C"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(q=None), INVALID), (dict(k=None), INVALID),
    (dict(v=None), INVALID),
    (dict(x=A + 4), INVALID), (dict(q=Cp + 8), INVALID), (dict(v=E + 2), INVALID), (dict(bias=Fp + 2), INVALID),
    (dict(F=0), INVALID), (dict(H=0), INVALID), (dict(C=-32), INVALID), (dict(dt=5), INVALID),
    (dict(C=48), UNSUPPORTED),                    # bf16 needs C % 32 == 0
    (dict(C=6, dt=F32), UNSUPPORTED),             # f32 needs C % 4 == 0
    (dict(q=A), INVALID), (dict(k=A + 16 * 40 * 64 * 2 - 16), INVALID),   # an output overlaps x
    (dict(v=B + 64), INVALID), (dict(bias=Fp, k=Fp + 128), INVALID),    # an output overlaps weight / bias
    (dict(k=Cp), INVALID), (dict(v=Cp + 256), INVALID), (dict(v=D + 512), INVALID),   # outputs overlap
])
def test_qkv_project_rejects(kw, status):
    assert proj(**kw) == status
    assert vinf.load().vinf_last_error()


def pattn(**kw):
    a = dict(x=A, w=B, bias=None, o=Cp, F=16, H=8, W=5, C=64, hd=64, nl=16, ng=16, scale=0.0, dt=BF16)
    a.update(kw)
    return vinf.load().vinf_projected_dual_domain_attn(a["x"], a["w"], a["bias"], a["o"], a["F"], a["H"], a["W"],
                                                       a["C"], a["hd"], a["nl"], a["ng"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(o=None), INVALID),
    (dict(x=A + 4), INVALID), (dict(o=Cp + 8), INVALID), (dict(bias=D + 2), INVALID),
    (dict(F=0), INVALID), (dict(H=0), INVALID), (dict(dt=5), INVALID),
    (dict(C=96), INVALID),                        # not a multiple of head_dim
    (dict(hd=32), UNSUPPORTED),
    (dict(dt=F32), UNSUPPORTED),                  # bf16 only
    (dict(nl=0), UNSUPPORTED), (dict(ng=0), UNSUPPORTED),   # the full key set only
    (dict(scale=float("nan")), INVALID),
    (dict(o=A), INVALID), (dict(o=A + 16 * 40 * 64 * 2 - 16), INVALID),   # o overlaps x
    (dict(o=B + 64), INVALID), (dict(bias=D, o=D + 128), INVALID),       # o overlaps weight / bias
])
def test_projected_attention_rejects(kw, status):
    assert pattn(**kw) == status
    assert vinf.load().vinf_last_error()


def gn(**kw):
    L = vinf.load()
    a = dict(x=A, y=B, gamma=None, beta=None, mean=None, rstd=None, F=16, H=8, W=5, C=64, G=8, eps=1e-5, dt=F32,
             ws=Cp, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.vinf_groupnorm_workspace_bytes(a["F"], a["H"], a["W"], max(a["C"], 8), 8, a["dt"] if a["dt"] in (0, 1) else 0)
    return L.vinf_groupnorm_global(a["x"], a["y"], a["gamma"], a["beta"], a["mean"], a["rstd"], a["F"], a["H"],
                                   a["W"], a["C"], a["G"], a["eps"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(x=A + 2), INVALID), (dict(gamma=D + 1), INVALID),
    (dict(mean=E + 2), INVALID), (dict(G=7), INVALID), (dict(G=0), INVALID), (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(F=0), INVALID), (dict(dt=3), INVALID),
    (dict(C=12, dt=BF16, G=4), UNSUPPORTED),      # bf16 vectors need C % 8
    (dict(C=8200, G=8, dt=F32), UNSUPPORTED),     # beyond 1024 vectors per row
    (dict(y=A + 16), INVALID),                    # partial overlap (y == x is allowed)
    (dict(ws=None), WORKSPACE), (dict(wsb=16), WORKSPACE), (dict(ws=Cp + 16), WORKSPACE),
    (dict(ws=A), INVALID),                        # workspace overlaps x
    (dict(mean=A + 64), INVALID),                 # statistics inside x
])
def test_groupnorm_rejects(kw, status):
    assert gn(**kw) == status


def test_python_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros(2, 2, 2, 64)
    with pytest.raises(TypeError):
        vinf.dual_domain_attn(x, x, x)
    with pytest.raises(TypeError):
        vinf.temporal_conv3(x, torch.zeros(3, 64, 64))
    with pytest.raises(TypeError):
        vinf.groupnorm_global(x, 8)
    with pytest.raises(TypeError):
        vinf.qkv_project(x, torch.zeros(3, 64, 64))
    with pytest.raises(TypeError):
        vinf.projected_dual_domain_attn_fused(x, torch.zeros(3, 64, 64))


# ------------------------------------------------------------ clip forms

def test_clip_halo_matches_the_key_frames():
    # Brute force over the oracle's key lists: the first and last local key of
    # the clip's queries.
    import oracle
    for F in (1, 5, 15, 16, 17, 40, 300):
        for f0 in range(0, F, max(1, F // 7)):
            for Fc in sorted({1, 2, 7, 16, 33, F - f0}):
                if Fc < 1 or f0 + Fc > F:
                    continue
                keys = [j for t in range(f0, f0 + Fc) for j in oracle.dda_keys(F, t, 16, 0)]
                assert vinf.dda_clip_halo(F, f0, Fc) == (f0 - min(keys), max(0, max(keys) + 1 - (f0 + Fc))), \
                    (F, f0, Fc)
                assert vinf.dda_clip_halo(F, f0, Fc, 0) == (0, 0)
    assert vinf.dda_clip_halo(2300, 864, 288) == (8, 7)


@pytest.mark.parametrize("args", [(0, 0, 1, 16), (10, 5, 6, 16), (10, -1, 2, 16), (10, 0, 0, 16), (10, 0, 2, -1)])
def test_clip_halo_rejects(args):
    with pytest.raises(vinf.VinfError):
        vinf.dda_clip_halo(*args)


def attn_clip(**kw):
    # F_total=100, clip [40, 60) with the minimal context 8 / 7
    a = dict(q=A, k=B, v=Cp, kg=D, vg=E, o=Fp, Ft=100, f0=40, Fc=20, pre=8, post=7, H=8, W=5, C=64, hd=64, nl=16,
             ng=16, scale=0.0, dt=BF16)
    a.update(kw)
    return vinf.load().vinf_dual_domain_attn_clip(a["q"], a["k"], a["v"], a["kg"], a["vg"], a["o"], a["Ft"], a["f0"],
                                                  a["Fc"], a["pre"], a["post"], a["H"], a["W"], a["C"], a["hd"],
                                                  a["nl"], a["ng"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(o=None), INVALID), (dict(kg=D + 8), INVALID),
    (dict(kg=None), INVALID),                     # one of k_global / v_global
    (dict(kg=None, vg=None), INVALID),            # global frames not inside k/v
    (dict(pre=7), INVALID), (dict(post=6), INVALID),   # context shorter than the windows reach
    (dict(f0=90, Fc=20), INVALID), (dict(f0=-1), INVALID), (dict(Fc=0), INVALID),
    (dict(f0=5, pre=8), INVALID),                 # context before frame 0
    (dict(f0=90, Fc=5, post=7), INVALID),         # context past the last frame
    (dict(pre=-1), INVALID),
    (dict(nl=8), UNSUPPORTED), (dict(nl=0, ng=0), UNSUPPORTED), (dict(hd=32), UNSUPPORTED),
    (dict(o=B + 64), INVALID), (dict(o=D), INVALID),   # o overlaps k / k_global
    (dict(scale=float("nan")), INVALID), (dict(dt=5), INVALID),
])
def test_attention_clip_rejects(kw, status):
    assert attn_clip(**kw) == status
    assert vinf.load().vinf_last_error()


def gn_clip_sums(**kw):
    L = vinf.load()
    a = dict(x=A, ms=None, sums=B, F=16, H=8, W=5, C=64, G=8, Ft=64, dt=F32, ws=Cp, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.vinf_groupnorm_workspace_bytes(16, 8, 5, 64, 8, F32)
    return L.vinf_groupnorm_clip_sums(a["x"], a["ms"], a["sums"], a["F"], a["H"], a["W"], a["C"], a["G"], a["Ft"],
                                      a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(sums=None), INVALID), (dict(sums=B + 4), INVALID), (dict(ms=D + 4), INVALID),
    (dict(Ft=15), INVALID), (dict(G=7), INVALID), (dict(F=0), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=8), WORKSPACE),
    (dict(sums=A + 256), INVALID), (dict(ms=B), INVALID),   # sums inside x / equal to mean_sums
])
def test_groupnorm_clip_sums_rejects(kw, status):
    assert gn_clip_sums(**kw) == status


def gn_clip_apply(**kw):
    L = vinf.load()
    a = dict(x=A, y=B, gamma=None, beta=None, s1=D, s2=E, mean=None, rstd=None, F=16, H=8, W=5, C=64, G=8, Ft=64,
             eps=1e-5, dt=F32, ws=Cp, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.vinf_groupnorm_workspace_bytes(16, 8, 5, 64, 8, F32)
    return L.vinf_groupnorm_clip_apply(a["x"], a["y"], a["gamma"], a["beta"], a["s1"], a["s2"], a["mean"], a["rstd"],
                                       a["F"], a["H"], a["W"], a["C"], a["G"], a["Ft"], a["eps"], a["dt"], a["ws"],
                                       a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(y=None), INVALID), (dict(s1=None), INVALID), (dict(s2=None), INVALID), (dict(s2=E + 2), INVALID),
    (dict(Ft=3), INVALID), (dict(eps=-1.0), INVALID), (dict(y=A + 16), INVALID), (dict(mean=B + 64), INVALID),
    (dict(wsb=16), WORKSPACE),
])
def test_groupnorm_clip_apply_rejects(kw, status):
    assert gn_clip_apply(**kw) == status


# ------------------------------------------------- GroupNorm folded into the conv

def gn_stats(**kw):
    L = vinf.load()
    a = dict(x=A, mean=B, rstd=B + 256, F=16, H=8, W=5, C=64, G=8, eps=1e-5, dt=F32, ws=Cp, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.vinf_groupnorm_workspace_bytes(16, 8, 5, 64, 8, F32)
    return L.vinf_groupnorm_stats(a["x"], a["mean"], a["rstd"], a["F"], a["H"], a["W"], a["C"], a["G"], a["eps"],
                                  a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(mean=None), INVALID), (dict(rstd=None), INVALID), (dict(mean=B + 2), INVALID),
    (dict(G=7), INVALID), (dict(eps=-1.0), INVALID), (dict(F=0), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=16), WORKSPACE),
    (dict(mean=A + 64), INVALID), (dict(rstd=B + 16), INVALID),   # inside x / overlapping mean
])
def test_groupnorm_stats_rejects(kw, status):
    assert gn_stats(**kw) == status


def test_conv3_gn_workspace_bytes():
    L = vinf.load()
    n = L.vinf_temporal_conv3_gn_workspace_bytes(320, BF16)
    assert n >= 2 * 320 * 4 and n % 256 == 0   # the per-channel a and b tables
    assert L.vinf_temporal_conv3_gn_workspace_bytes(320, F32) == n
    assert L.vinf_temporal_conv3_gn_workspace_bytes(0, BF16) == 0
    assert L.vinf_temporal_conv3_gn_workspace_bytes(64, 9) == 0


def conv_gn(**kw):
    L = vinf.load()
    a = dict(x=A, pre=None, post=None, w=B, bias=None, mean=D, rstd=D + 256, gamma=None, beta=None, G=8, y=Cp,
             F=16, H=8, W=5, C=64, dt=BF16, ws=E, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.vinf_temporal_conv3_gn_workspace_bytes(a["C"], BF16)
    return L.vinf_temporal_conv3_gn(a["x"], a["pre"], a["post"], a["w"], a["bias"], a["mean"], a["rstd"],
                                    a["gamma"], a["beta"], a["G"], a["y"], a["F"], a["H"], a["W"], a["C"], a["dt"],
                                    a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID), (dict(mean=None), INVALID),
    (dict(rstd=None), INVALID), (dict(rstd=D + 2), INVALID), (dict(gamma=Fp + 1), INVALID),
    (dict(G=7), INVALID), (dict(G=0), INVALID), (dict(F=0), INVALID),
    (dict(C=48, G=8), UNSUPPORTED),                 # bf16 MFMA tiles need C % 32
    (dict(ws=None), WORKSPACE), (dict(wsb=8), WORKSPACE), (dict(ws=E + 16), WORKSPACE),
    (dict(y=A), INVALID), (dict(y=B + 64), INVALID),   # y overlaps x / the weights
    (dict(ws=B), INVALID), (dict(ws=Cp + 256), INVALID),   # workspace overlaps the weights / y
    (dict(mean=Cp + 64), INVALID),                 # statistics inside y
    (dict(F=1, H=2048, W=1639, C=320, G=32), UNSUPPORTED),   # one frame over 2 GiB (rejected before any launch)
])
def test_conv3_gn_rejects(kw, status):
    assert conv_gn(**kw) == status


# ----------------------------------------------- attention output reuse schedule

def test_broadcast_schedule_matches_the_oracle():
    import numpy as np
    import oracle
    for n in list(range(1, 50)) + [128, 1000]:
        for r in (1, 2, 3, 4, 9, 100):
            assert vinf.attn_broadcast_schedule(n, r) == list(oracle.broadcast_schedule(n, r)), (n, r)
    s = vinf.attn_broadcast_schedule(30, 3)
    assert sum(s) == 16 and s[:5] == [1, 1, 1, 1, 1] and s[5:7] == [0, 0]


@pytest.mark.parametrize("n,r", [(0, 2), (-1, 2), (10, 0), (10, -3)])
def test_broadcast_schedule_rejects(n, r):
    buf = ctypes.create_string_buffer(16)
    assert vinf.load().vinf_attn_broadcast_schedule(n, r, buf) == INVALID
    assert vinf.load().vinf_attn_broadcast_schedule(10, 2, None) == INVALID


# ------------------------------------------ allocation-free GroupNorm entry point

def gn_noalloc(**kw):
    a = dict(x=A, y=B, gamma=None, beta=None, mean=None, rstd=None, F=16, H=8, W=5, C=64, G=8, eps=1e-5, dt=BF16)
    a.update(kw)
    return vinf.load().vinf_groupnorm_global_noalloc(a["x"], a["y"], a["gamma"], a["beta"], a["mean"], a["rstd"],
                                                     a["F"], a["H"], a["W"], a["C"], a["G"], a["eps"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(x=A + 4), INVALID), (dict(gamma=Cp + 2), INVALID),
    (dict(G=7), INVALID), (dict(F=0), INVALID), (dict(eps=-1.0), INVALID), (dict(dt=5), INVALID),
    (dict(y=A + 64), INVALID),                           # partial overlap (only y == x is allowed)
    (dict(mean=A + 128), INVALID),                       # statistics inside x
    (dict(C=16384, G=32), UNSUPPORTED),                  # wider than the GroupNorm kernels take
    # 2048 blocks x 4096 channels of fp32 partials = 32 MiB, more than the static scratch
    (dict(F=64, H=64, W=64, C=4096, G=32, y=A), UNSUPPORTED),
])
def test_groupnorm_noalloc_rejects(kw, status):
    assert gn_noalloc(**kw) == status


def test_groupnorm_noalloc_limit_message():
    assert gn_noalloc(F=64, H=64, W=64, C=4096, G=32, y=A) == UNSUPPORTED
    assert b"scratch" in vinf.load().vinf_last_error()
