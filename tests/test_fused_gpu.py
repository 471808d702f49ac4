"""GroupNorm applied inside the temporal conv, on the GPU through the C ABI.

vinf_temporal_conv3_gn computes conv3(GroupNorm(x)) without writing the
normalised tensor: the conv normalises each x tile in LDS exactly as the
GroupNorm apply writes it (fp32 fmaf, rounded to the I/O type).  So the
fused call must equal GroupNorm apply + conv bit for bit, and the oracle
reference is its conv over the rounded GroupNorm output (context frames
normalised with the same statistics and rounded alike).  Clips with raw
context frames reproduce the whole-video call bit for bit, and the full chain
(statistics -> fused conv -> attention) at the workload sizes equals the
unfused chain bit for bit and meets the bar against the oracle chain.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, check_end_to_end, check_stats, dev, fetch, sample_locs, upload

pytestmark = pytest.mark.gpu

BF, FP = synth.BF16, synth.F32


def rnd(shape, seed, dt, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, dt, scale).reshape(shape)


def widen(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 values that are exactly bf16 -> uint16 bits."""
    return (np.asarray(a).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dt", [BF, FP])
def test_groupnorm_stats_equal_the_full_call(dt):
    F, H, W, C, G = 37, 7, 9, 320, 32
    announce(f"groupnorm stats only F={F} C={C} G={G} dt={dt}")
    x = upload(rnd((F, H, W, C), 4000, dt))
    _, m, r = vinf.groupnorm_global(x, G)
    m2, r2 = vinf.groupnorm_stats(x, G)
    assert torch.equal(m, m2) and torch.equal(r, r2)


@pytest.mark.parametrize("F,H,W,C,G,dt,ctx,bias,affine", [
    (37, 5, 7, 320, 32, BF, False, False, False),  # ragged frame and location tiles
    (33, 4, 5, 256, 32, BF, True, True, True),
    (20, 3, 6, 128, 16, BF, False, True, True),
    (5, 4, 4, 64, 8, BF, True, False, True),
    (1, 3, 3, 64, 8, BF, False, True, False),      # one frame: both taps of it read pads
    (1, 3, 3, 64, 8, BF, True, True, True),
    (2, 2, 2, 32, 4, BF, False, False, True),
    (48, 16, 95, 32, 8, BF, True, True, True),     # 285 tiles: workgroups walk several, with pads
    (70, 16, 59, 32, 8, BF, True, False, True),    # 295 tiles, ragged last frame block, with pads
    (17, 4, 3, 96, 8, FP, True, True, True),
    (9, 2, 5, 32, 4, FP, False, False, False),
])
def test_conv3_gn_vs_oracle(F, H, W, C, G, dt, ctx, bias, affine):
    announce(f"conv3_gn F={F} H={H} W={W} C={C} G={G} dt={dt} ctx={ctx} bias={bias} affine={affine}")
    # an offset mean, so that the fold's mean term matters
    x = synth.normal(F * H * W * C, 4100 + F + C, dt, 1.5, H * W * C, 0.05).reshape(F, H, W, C)
    x = (widen(x) + 3.0).astype(np.float32)
    if dt == BF:
        x = to_bf16_bits(torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())
    w = rnd((3, C, C), 4200 + C, dt, (1.0 / (3 * C)) ** 0.5)
    pre = rnd((H, W, C), 4300, dt) if ctx else None
    post = rnd((H, W, C), 4301, dt) if ctx else None
    gamma = np.linspace(0.5, 1.5, C).astype(np.float32) if affine else None
    beta = np.linspace(-0.25, 0.25, C).astype(np.float32) if affine else None
    b = np.linspace(-0.1, 0.1, C).astype(np.float32) if bias else None
    xd = upload(x)
    mean, rstd = vinf.groupnorm_stats(xd, G)
    tg = lambda a: None if a is None else torch.from_numpy(a).to(dev())
    y = vinf.temporal_conv3_gn(xd, upload(w), mean, rstd, tg(gamma), tg(beta),
                               None if pre is None else upload(pre), None if post is None else upload(post), tg(b))
    g64 = None if gamma is None else gamma.astype(np.float64)
    b64 = None if beta is None else beta.astype(np.float64)
    gn, rm, rr = oracle.groupnorm(x, G, 1e-5, g64, b64)
    check_stats(mean, rstd, rm, rr, "stats")
    rnd_dt = np.vectorize(lambda v: oracle.round_to(v, dt))

    def as_dt(v):  # rounded float64 values -> the oracle's input type
        return to_bf16_bits(v) if dt == BF else v.astype(np.float32)

    def norm(c):  # a context frame normalised with the video's statistics, rounded like the tensor
        if c is None:
            return None
        v = (widen(c).reshape(H * W, C) - np.repeat(rm, C // G)) * np.repeat(rr, C // G)
        if g64 is not None:
            v = v * g64 + b64
        return as_dt(rnd_dt(v))

    ref = oracle.conv3(as_dt(rnd_dt(gn)), w, norm(pre), norm(post), None if b is None else b.astype(np.float64))
    check(fetch(y), ref, dt, "y")
    if not ctx:  # without context frames: bit for bit the unfused pair of calls
        g, _, _ = vinf.groupnorm_global(xd, G, 1e-5, tg(gamma), tg(beta))
        assert np.array_equal(bits(y), bits(vinf.temporal_conv3(g, upload(w), bias=tg(b))))


@pytest.mark.parametrize("F,C,G", [(72, 320, 32), (72, 256, 32), (72, 128, 16), (72, 64, 8), (72, 32, 8),
                                   (40, 640, 32), (24, 1280, 32)])
def test_conv3_gn_many_tiles_bitwise(F, C, G):
    """31 x 29 locations and 72 frames make 285 tiles (both axes ragged; 342
    and 456 at C = 640 and 1280, where two and four channel tiles share each
    staged x tile), more than there are workgroups, so a workgroup normalises
    the next tile's first slice while it multiplies the previous tile's last
    one.  Every tiling the bf16 conv picks for these C must still equal
    GroupNorm apply + conv bit for bit."""
    H, W = 31, 29
    announce(f"conv3_gn many tiles F={F} H={H} W={W} C={C} G={G}")
    x = upload(rnd((F, H, W, C), 4600 + C, BF, 2.0))
    w = upload(rnd((3, C, C), 4700 + C, BF, (1.0 / (3 * C)) ** 0.5))
    tg = lambda a: torch.from_numpy(a).to(dev())
    gamma = tg(np.linspace(0.5, 1.5, C).astype(np.float32))
    beta = tg(np.linspace(-0.25, 0.25, C).astype(np.float32))
    b = tg(np.linspace(-0.1, 0.1, C).astype(np.float32))
    mean, rstd = vinf.groupnorm_stats(x, G)
    y = vinf.temporal_conv3_gn(x, w, mean, rstd, gamma, beta, None, None, b)
    g, _, _ = vinf.groupnorm_global(x, G, 1e-5, gamma, beta)
    assert torch.equal(y.view(torch.int16), vinf.temporal_conv3(g, w, bias=b).view(torch.int16))


@pytest.mark.parametrize("dt", [BF, FP])
def test_conv3_gn_clip_equals_whole_bitwise(dt):
    F, H, W, C, G = 70, 3, 4, 128, 16
    announce(f"conv3_gn clips vs whole F={F} C={C} dt={dt}")
    x = upload(rnd((F, H, W, C), 4400, dt))
    w = upload(rnd((3, C, C), 4401, dt, (1.0 / (3 * C)) ** 0.5))
    gamma = torch.linspace(0.5, 1.5, C, device=dev())
    beta = torch.linspace(-0.25, 0.25, C, device=dev())
    bias = torch.linspace(-0.1, 0.1, C, device=dev())
    mean, rstd = vinf.groupnorm_stats(x, G)
    whole = bits(vinf.temporal_conv3_gn(x, w, mean, rstd, gamma, beta, bias=bias))
    for a, b in [(0, 16), (16, 17), (17, 50), (50, 70)]:
        y = vinf.temporal_conv3_gn(x[a:b], w, mean, rstd, gamma, beta, x[a - 1] if a > 0 else None,
                                   x[b] if b < F else None, bias)
        assert np.array_equal(bits(y), whole[a:b]), (a, b)


def test_fused_clip_pipeline():
    # The clip-parallel form of the fused path: per-clip sums, aggregated,
    # statistics from the totals, then the fused conv of each clip with raw
    # context frames; against the whole-video fused call.
    F, H, W, C, G = 61, 4, 5, 320, 32
    announce(f"fused clip pipeline F={F} C={C}")
    x = upload(synth.normal(F * H * W * C, 4500, BF, 1.0, H * W * C, 2.0 / F).reshape(F, H, W, C))
    w = upload(rnd((3, C, C), 4501, BF, (1.0 / (3 * C)) ** 0.5))
    clips = [(0, 13), (13, 40), (40, 61)]
    s1 = sum(vinf.groupnorm_clip_sums(x[a:b], G, F) for a, b in clips)
    s2 = sum(vinf.groupnorm_clip_sums(x[a:b], G, F, s1) for a, b in clips)
    _, m, r = vinf.groupnorm_clip_apply(x[0:13], G, F, s1, s2, stats_only=True)
    m2, r2 = vinf.groupnorm_stats(x, G)
    check_stats(m, r, m2.cpu().numpy().astype(np.float64), r2.cpu().numpy().astype(np.float64), "clip stats")
    whole = fetch(vinf.temporal_conv3_gn(x, w, m, r))
    parts = [fetch(vinf.temporal_conv3_gn(x[a:b], w, m, r, ctx_pre=x[a - 1] if a > 0 else None,
                                          ctx_post=x[b] if b < F else None)) for a, b in clips]
    assert np.array_equal(np.concatenate(parts), whole)


def run_fused_chain(cfgno):
    """Statistics -> fused conv -> attention (Q = K = V) at a workload's size.

    (1) bit for bit the unfused chain (GroupNorm apply -> conv -> attention)
    on the same inputs; (2) the fused conv against the oracle's conv of its
    rounded GroupNorm output at the bar; (3) the attention against the
    oracle's attention over the GPU's own conv output at the bar; (4) end to
    end against the oracle chain: mean-abs at the bar, max-abs at the bar
    where both sides rounded every conv value the attention reads alike, and
    elsewhere the bar plus the bound on how far one-step rounding differences
    move the attention (helpers.check_end_to_end)."""
    c = synth.CONFIGS[cfgno]
    F, H, W, C, G, dt = c["F"], c["H"], c["W"], c["C"], c["G"], c["dtype"]
    S = H * W
    locs = sample_locs(S, 8, seed=cfgno)
    announce(f"{c['name']}: fused chain groupnorm stats -> conv3_gn -> attention")
    x = synth.make_tensor(cfgno, synth.X_GN, F, H, W, C, dt)
    w = synth.make_conv_weight(cfgno, C, dt)
    xd, wd = upload(x), upload(w)
    mean, rstd = vinf.groupnorm_stats(xd, G)
    cv = vinf.temporal_conv3_gn(xd, wd, mean, rstd)
    o = vinf.dual_domain_attn(cv, cv, cv)
    g, mean_u, rstd_u = vinf.groupnorm_global(xd, G)
    del xd
    cv_u = vinf.temporal_conv3(g, wd)
    del g
    assert torch.equal(mean, mean_u) and torch.equal(rstd, rstd_u)
    assert torch.equal(cv.view(torch.int16), cv_u.view(torch.int16)), "fused conv differs from groupnorm + conv"
    del cv_u
    o_u = vinf.dual_domain_attn(cv, cv, cv)
    assert torch.equal(o.view(torch.int16), o_u.view(torch.int16))
    del o_u
    cs, os_ = fetch(cv, locs), fetch(o, locs)
    del cv, o
    out, _, cv_r, _, cv_x, rm, rr = oracle.chain(x, w, G, locs=locs, exact=True)
    check_stats(mean, rstd, rm, rr, "fused chain stats")
    check(cs, cv_x, dt, "fused conv3 vs the oracle's conv")
    cb = to_bf16_bits(cs)
    o_on_gpu_conv = oracle.dda(cb, cb, cb)
    check(os_, o_on_gpu_conv, dt, "attention over the fused conv output")
    check_end_to_end(os_, out, o_on_gpu_conv, cv_r, cs, dt, "fused chain")


@pytest.mark.parametrize("cfgno", [5, 6])
def test_workload_fused_chain(cfgno):
    run_fused_chain(cfgno)
