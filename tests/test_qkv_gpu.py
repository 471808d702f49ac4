"""Q/K/V projection and the attention over the projected tokens, on the GPU
through the C ABI, against the oracle.

The bf16 projection runs the conv's MFMA kernel with one tap; its three maps
are three output tiles of one launch.  Checks: every element against the
oracle's exact projection at the bar (ragged frame and location tiles, every
tile width the kernel has), identity maps bit for bit, and the attention over
the projected tokens in two stages (projection vs the oracle; attention over
the GPU's own Q/K/V vs the oracle's attention), as the chain tests do.

The fused call (projection inside the attention's work items) must give the
two calls' result bit for bit: it rounds the same fp32 sums, accumulated in
the same order, to the same bf16 q, k and v.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, dev, fetch, sample_locs, upload

pytestmark = pytest.mark.gpu

BF, FP = synth.BF16, synth.F32


def rnd(shape, seed, dt, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, dt, scale).reshape(shape)


def to_bf16_bits(a):
    return (np.asarray(a).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("F,H,W,C,dt,bias", [
    (37, 5, 7, 320, BF, False),   # ragged frame and location tiles, 5x4 waves of 80 channels
    (33, 4, 5, 256, BF, True),
    (20, 3, 6, 128, BF, True),
    (5, 4, 4, 64, BF, False),
    (1, 3, 3, 64, BF, True),
    (2, 2, 2, 32, BF, True),      # the narrowest tile (32 channels)
    (3, 5, 5, 640, BF, False),    # two N tiles per output
    (4, 2, 3, 1280, BF, True),    # four N tiles per output (twelve per launch)
    (7, 3, 5, 96, BF, True),      # C / 32 odd: one slice per barrier
    (17, 4, 3, 96, FP, True),
    (9, 2, 5, 32, FP, False),
])
def test_qkv_project_vs_oracle(F, H, W, C, dt, bias):
    announce(f"qkv_project F={F} H={H} W={W} C={C} dt={dt} bias={bias}")
    x = rnd((F, H, W, C), 6000 + F + C, dt)
    w = rnd((3, C, C), 6100 + C, dt, (1.0 / C) ** 0.5)
    b = np.linspace(-0.3, 0.3, 3 * C).astype(np.float32).reshape(3, C) if bias else None
    q, k, v = vinf.qkv_project(upload(x), upload(w), None if b is None else torch.from_numpy(b).to(dev()))
    ref = oracle.qkv_project(x, w, None if b is None else b.astype(np.float64))
    for p, t in enumerate((q, k, v)):
        check(fetch(t), ref[p], dt, "qkv"[p])


@pytest.mark.parametrize("dt", [BF, FP])
def test_identity_maps_are_exact(dt):
    F, H, W, C = 19, 3, 7, 320
    announce(f"qkv_project identity maps F={F} C={C} dt={dt}")
    x = upload(rnd((F, H, W, C), 6200, dt))
    tdt = torch.bfloat16 if dt == BF else torch.float32
    w = torch.stack([torch.eye(C, device=dev())] * 3).to(tdt)
    for t in vinf.qkv_project(x, w):
        assert np.array_equal(bits(t), bits(x))


def test_outputs_in_one_buffer():
    # Q, K and V as three slices of one [3, F, H, W, C] allocation.
    F, H, W, C = 21, 4, 4, 128
    announce(f"qkv_project into one buffer F={F} C={C}")
    x = upload(rnd((F, H, W, C), 6300, BF))
    w = upload(rnd((3, C, C), 6301, BF, (1.0 / C) ** 0.5))
    buf = torch.empty((3, F, H, W, C), device=dev(), dtype=torch.bfloat16)
    vinf.qkv_project(x, w, out=(buf[0], buf[1], buf[2]))
    for a, b in zip(vinf.qkv_project(x, w), buf):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("F,H,W,C,dt", [
    (600, 2, 3, 128, BF),   # several attention items per strip, ragged tail
    (40, 4, 5, 320, BF),
    (16, 3, 3, 64, FP),
])
def test_projected_attention_vs_oracle(F, H, W, C, dt):
    announce(f"projected attention F={F} H={H} W={W} C={C} dt={dt}")
    x = rnd((F, H, W, C), 6400 + F, dt)
    w = rnd((3, C, C), 6401 + C, dt, (1.0 / C) ** 0.5)
    b = np.linspace(-0.2, 0.2, 3 * C).astype(np.float32).reshape(3, C)
    xd, wd, bd = upload(x), upload(w), torch.from_numpy(b).to(dev())
    q, k, v = vinf.qkv_project(xd, wd, bd)
    o = vinf.projected_dual_domain_attn(xd, wd, bd)
    assert np.array_equal(bits(o), bits(vinf.dual_domain_attn(q, k, v)))
    ref_o, ref_qkv = oracle.qkv_dda(x, w, b.astype(np.float64), intermediates=True)
    exact = oracle.qkv_project(x, w, b.astype(np.float64))
    for p, t in enumerate((q, k, v)):
        check(fetch(t), exact[p], dt, "qkv"[p] + " vs the oracle's projection")
    gq, gk, gv = (fetch(t).reshape(F, H, W, C) for t in (q, k, v))
    if dt == BF:
        gq, gk, gv = (to_bf16_bits(a) for a in (gq, gk, gv))
    else:
        gq, gk, gv = (a.astype(np.float32) for a in (gq, gk, gv))
    check(fetch(o), oracle.dda(gq, gk, gv), dt, "attention over the GPU's q, k, v")
    err = np.abs(fetch(o) - ref_o)
    announce(f"  (end to end against the oracle's own rounding of q, k, v: max-abs {err.max():.3e} "
             f"mean-abs {err.mean():.3e})")


def test_projected_attention_at_workload_size():
    # F=1024 at 64x40x320 with projection weights of variance 1/C: sampled
    # locations against the oracle, in the same two stages.
    cfg = 6
    F, H, W, C = 1024, 64, 40, 320
    announce(f"projected attention at workload size F={F} {H}x{W}x{C} bf16")
    x = synth.make_tensor(cfg, synth.X_CONV, F, H, W, C, BF)
    w = synth.make_qkv_weight(cfg, C, BF)
    xd, wd = upload(x), upload(w)
    q, k, v = vinf.qkv_project(xd, wd)
    o = vinf.dual_domain_attn(q, k, v)
    locs = sample_locs(H * W, 6, seed=11)
    xs = x.reshape(F, H * W, C)[:, locs].reshape(F, len(locs), 1, C)
    exact = oracle.qkv_project(xs, w)
    cols = [fetch(t, locs) for t in (q, k, v)]
    for p in range(3):
        check(cols[p], exact[p], BF, "qkv"[p] + " (sampled locations)")
    gq, gk, gv = (to_bf16_bits(c).reshape(F, len(locs), 1, C) for c in cols)
    check(fetch(o, locs), oracle.dda(gq, gk, gv), BF, "attention over the GPU's q, k, v (sampled locations)")


@pytest.mark.parametrize("F,H,W,C,bias", [
    (37, 5, 7, 320, True),     # one partial 256-frame item per strip
    (300, 2, 3, 128, False),   # a full and a partial item per strip
    (513, 1, 2, 64, True),     # three items per strip, one query in the last
    (5, 2, 2, 64, True),       # F < 16: every frame is local context, rows past F are zeros
    (16, 3, 3, 192, False),    # F = 16: one window, global frames 0 .. 15
    (40, 4, 5, 640, True),     # ten heads
    (23, 2, 3, 1280, False),   # twenty heads, 40 slices of 32 channels
    (1, 3, 2, 128, True),      # one frame: its window and every global row are frame 0
])
def test_fused_projected_attention(F, H, W, C, bias):
    announce(f"fused projected attention F={F} H={H} W={W} C={C} bias={bias}")
    x = rnd((F, H, W, C), 6500 + F, BF)
    w = rnd((3, C, C), 6501 + C, BF, (1.0 / C) ** 0.5)
    b = np.linspace(-0.2, 0.2, 3 * C).astype(np.float32).reshape(3, C) if bias else None
    xd, wd = upload(x), upload(w)
    bd = None if b is None else torch.from_numpy(b).to(dev())
    o = vinf.projected_dual_domain_attn_fused(xd, wd, bd)
    q, k, v = vinf.qkv_project(xd, wd, bd)
    assert np.array_equal(bits(o), bits(vinf.dual_domain_attn(q, k, v))), "fused != qkv_project + attention"
    gq, gk, gv = (to_bf16_bits(fetch(t).reshape(F, H, W, C)) for t in (q, k, v))
    check(fetch(o), oracle.dda(gq, gk, gv), BF, "fused: attention over the projected q, k, v vs the oracle")
    exact = oracle.qkv_project(x, w, None if b is None else b.astype(np.float64))
    check(fetch(k), exact[1], BF, "k vs the oracle's projection")


def test_fused_projected_attention_at_workload_size():
    F, H, W, C = 1024, 64, 40, 320
    announce(f"fused projected attention at workload size F={F} {H}x{W}x{C} bf16")
    cfg = 6
    xd = upload(synth.make_tensor(cfg, synth.X_CONV, F, H, W, C, BF))
    wd = upload(synth.make_qkv_weight(cfg, C, BF))
    b = torch.linspace(-0.1, 0.1, 3 * C, device=dev())
    o = vinf.projected_dual_domain_attn_fused(xd, wd, b)
    ref = vinf.projected_dual_domain_attn(xd, wd, b)
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), "fused != qkv_project + attention"
