"""The Python binding's own argument checks, on the CPU.

The C library sees only pointers, so a caller-supplied output, statistics
vector, affine vector, bias or workspace of the wrong size or dtype would be
read or written out of bounds on the device.  The binding therefore checks
every tensor it passes before it calls the library.  Here the GPU-tensor test
is relaxed to accept CPU tensors and the library is replaced by a recorder,
so each bad argument must raise before any library call is made, and the
matching good call must reach the library.
"""
import pytest
import torch

import video_diffusion_temporal_amd as vinf


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 1024 if name.endswith("_workspace_bytes") else 0
        return fn


@pytest.fixture
def lib(monkeypatch):
    rec = Recorder()

    def dev(t, name):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t

    monkeypatch.setattr(vinf, "load", lambda: rec)
    monkeypatch.setattr(vinf, "_dev", dev)
    monkeypatch.setattr(vinf, "_stream", lambda device, stream: 0)
    return rec


F, H, W, C, G = 4, 2, 3, 128, 8
BF = torch.bfloat16


def x_():
    return torch.zeros(F, H, W, C, dtype=BF)


def f32(n):
    return torch.zeros(n, dtype=torch.float32)


def launched(rec):
    return [c for c in rec.calls if not c.endswith("_workspace_bytes")]


BAD_OUT = {
    "smaller": lambda: torch.zeros(F - 1, H, W, C, dtype=BF),
    "other dtype": lambda: torch.zeros(F, H, W, C, dtype=torch.float32),
    "flat": lambda: torch.zeros(F * H * W * C, dtype=BF),
    "strided": lambda: torch.zeros(F, H, W, 2 * C, dtype=BF)[..., :C],
}


@pytest.mark.parametrize("bad", sorted(BAD_OUT))
@pytest.mark.parametrize("call", ["groupnorm_global", "temporal_conv3", "dual_domain_attn", "temporal_conv3_gn",
                                  "groupnorm_clip_apply", "dual_domain_attn_clip", "qkv_project",
                                  "projected_dual_domain_attn_fused"])
def test_bad_output_tensor_raises_before_launch(lib, call, bad):
    x = x_()
    out = BAD_OUT[bad]()
    wt = torch.zeros(3, C, C, dtype=BF)
    with pytest.raises(ValueError):
        if call == "groupnorm_global":
            vinf.groupnorm_global(x, G, out=out)
        elif call == "temporal_conv3":
            vinf.temporal_conv3(x, wt, out=out)
        elif call == "dual_domain_attn":
            vinf.dual_domain_attn(x, x, x, out=out)
        elif call == "temporal_conv3_gn":
            vinf.temporal_conv3_gn(x, wt, f32(G), f32(G), out=out)
        elif call == "groupnorm_clip_apply":
            s = torch.zeros(G, dtype=torch.float64)
            vinf.groupnorm_clip_apply(x, G, F, s, s, out=out)
        elif call == "dual_domain_attn_clip":
            vinf.dual_domain_attn_clip(x, x, x, F, 0, 0, 0, out=out)
        elif call == "projected_dual_domain_attn_fused":
            vinf.projected_dual_domain_attn_fused(x, wt, out=out)
        else:
            vinf.qkv_project(x, wt, out=(x_(), out, x_()))
    assert launched(lib) == []


@pytest.mark.parametrize("field,value", [
    ("mean_out", lambda: f32(G - 1)), ("rstd_out", lambda: f32(G + 1)),
    ("mean_out", lambda: torch.zeros(G, dtype=torch.float64)), ("rstd_out", lambda: torch.zeros(G, dtype=BF)),
    ("gamma", lambda: f32(C - 8)), ("beta", lambda: torch.zeros(C, dtype=BF)),
])
def test_groupnorm_global_vectors(lib, field, value):
    with pytest.raises(ValueError):
        vinf.groupnorm_global(x_(), G, **{field: value()})
    assert launched(lib) == []


@pytest.mark.parametrize("field,value", [
    ("mean_out", lambda: f32(G - 1)), ("rstd_out", lambda: torch.zeros(G, dtype=torch.float64)),
])
def test_groupnorm_stats_vectors(lib, field, value):
    with pytest.raises(ValueError):
        vinf.groupnorm_stats(x_(), G, **{field: value()})
    assert launched(lib) == []


@pytest.mark.parametrize("field,value", [
    ("mean_out", lambda: f32(G - 1)), ("rstd_out", lambda: f32(2 * G)),
    ("gamma", lambda: f32(C + 1)), ("beta", lambda: torch.zeros(C, dtype=torch.float64)),
    ("sums", lambda: torch.zeros(G - 1, dtype=torch.float64)), ("sq_sums", lambda: f32(G)),
])
def test_groupnorm_clip_apply_vectors(lib, field, value):
    s = torch.zeros(G, dtype=torch.float64)
    kw = dict(sums=s, sq_sums=s)
    kw[field] = value()
    sums, sq = kw.pop("sums"), kw.pop("sq_sums")
    with pytest.raises(ValueError):
        vinf.groupnorm_clip_apply(x_(), G, F, sums, sq, **kw)
    assert launched(lib) == []


@pytest.mark.parametrize("field,value", [
    ("gamma", lambda: f32(C // 2)), ("beta", lambda: torch.zeros(C, dtype=BF)), ("bias", lambda: f32(C - 1)),
    ("bias", lambda: torch.zeros(C, dtype=torch.float64)), ("rstd", lambda: f32(G - 1)),
    ("ctx_pre", lambda: torch.zeros(H, W, C - 8, dtype=BF)), ("ctx_post", lambda: torch.zeros(H, W, C)),
])
def test_conv3_gn_vectors(lib, field, value):
    kw = dict(mean=f32(G), rstd=f32(G))
    kw[field] = value()
    mean, rstd = kw.pop("mean"), kw.pop("rstd")
    with pytest.raises(ValueError):
        vinf.temporal_conv3_gn(x_(), torch.zeros(3, C, C, dtype=BF), mean, rstd, **kw)
    assert launched(lib) == []


@pytest.mark.parametrize("field,value", [
    ("bias", lambda: f32(C - 1)), ("bias", lambda: torch.zeros(C, dtype=BF)),
    ("ctx_pre", lambda: torch.zeros(H, W, C + 8, dtype=BF)),
])
def test_conv3_vectors(lib, field, value):
    with pytest.raises(ValueError):
        vinf.temporal_conv3(x_(), torch.zeros(3, C, C, dtype=BF), **{field: value()})
    assert launched(lib) == []


def test_qkv_project_bias(lib):
    with pytest.raises(ValueError):
        vinf.qkv_project(x_(), torch.zeros(3, C, C, dtype=BF), bias=f32(C))
    with pytest.raises(ValueError):
        vinf.projected_dual_domain_attn_fused(x_(), torch.zeros(3, C, C, dtype=BF), bias=f32(C))
    with pytest.raises(ValueError):
        vinf.projected_dual_domain_attn_fused(x_(), torch.zeros(3, C, C, dtype=torch.float32))
    assert launched(lib) == []


def test_groupnorm_clip_sums_out(lib):
    with pytest.raises(ValueError):
        vinf.groupnorm_clip_sums(x_(), G, F, out=torch.zeros(G, dtype=torch.float32))
    assert launched(lib) == []


def test_good_arguments_reach_the_library(lib):
    x = x_()
    wt = torch.zeros(3, C, C, dtype=BF)
    s = torch.zeros(G, dtype=torch.float64)
    vinf.groupnorm_global(x, G, gamma=f32(C), beta=f32(C), out=x_(), mean_out=f32(G), rstd_out=f32(G))
    vinf.groupnorm_stats(x, G, mean_out=f32(G), rstd_out=f32(G))
    vinf.temporal_conv3(x, wt, ctx_pre=torch.zeros(H, W, C, dtype=BF), bias=f32(C), out=x_())
    vinf.temporal_conv3_gn(x, wt, f32(G), f32(G), gamma=f32(C), beta=f32(C), bias=f32(C), out=x_())
    vinf.dual_domain_attn(x, x, x, out=x_())
    vinf.qkv_project(x, wt, bias=f32(3 * C), out=(x_(), x_(), x_()))
    vinf.groupnorm_clip_sums(x, G, F, out=torch.zeros(G, dtype=torch.float64))
    vinf.groupnorm_clip_apply(x, G, F, s, s, gamma=f32(C), out=x_(), mean_out=f32(G), rstd_out=f32(G))
    vinf.dual_domain_attn_clip(x, x, x, F, 0, 0, 0, out=x_())
    vinf.projected_dual_domain_attn_fused(x, wt, bias=f32(3 * C), out=x_())
    assert launched(lib) == ["vinf_groupnorm_global", "vinf_groupnorm_stats", "vinf_temporal_conv3",
                             "vinf_temporal_conv3_gn", "vinf_dual_domain_attn", "vinf_qkv_project",
                             "vinf_groupnorm_clip_sums", "vinf_groupnorm_clip_apply", "vinf_dual_domain_attn_clip",
                             "vinf_projected_dual_domain_attn"]
