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
                          "vinf_groupnorm_workspace_bytes", "vinf_status_string", "vinf_last_error"}
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
    (dict(C=68), UNSUPPORTED),                   # not a multiple of 8 (bf16 vectors)
    (dict(dt=7), INVALID),
    (dict(o=A), INVALID), (dict(o=B + 256), INVALID),  # o overlaps q / k
    (dict(scale=float("nan")), INVALID),
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
