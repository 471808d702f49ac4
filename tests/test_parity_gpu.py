"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small shapes compare every output element and span several workgroup tiles
with ragged tails; the full workloads compare sampled spatial locations (the
oracle computes those columns exactly: conv and attention never mix
locations, and the GroupNorm statistics are compared as well).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, check_end_to_end, check_stats, fetch, sample_locs, upload

pytestmark = pytest.mark.gpu

BF, FP = synth.BF16, synth.F32


def rnd(shape, seed, dt, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, dt, scale).reshape(shape)


# ------------------------------------------------------------------ GroupNorm

@pytest.mark.parametrize("F,H,W,C,G,dt", [
    (16, 8, 5, 64, 8, FP),          # the tiny float32 workload
    (37, 7, 9, 320, 32, BF),        # ragged rows, C/G = 10
    (5, 3, 3, 640, 32, BF),
    (3, 1, 1, 1280, 32, BF),        # fewer rows than one block's row slots
    (1, 1, 1, 8, 1, BF),            # a single voxel row
    (9, 4, 4, 2048, 16, BF),        # 256 vectors per row
    (2, 3, 2, 4096, 8, BF),         # 512 vectors per row (one row slot per block)
    (11, 5, 3, 12, 3, FP),          # C/G = 4
])
def test_groupnorm_small(F, H, W, C, G, dt):
    announce(f"groupnorm F={F} H={H} W={W} C={C} G={G} dt={dt}")
    x = rnd((F, H, W, C), 1000 + C + F, dt)
    # |y| stays below 8, where one bf16 half-ulp (2^-6) is under the 2e-2 bar
    gamma = np.linspace(0.5, 1.25, C).astype(np.float32)
    beta = np.linspace(-0.5, 0.5, C).astype(np.float32)
    y, mean, rstd = vinf.groupnorm_global(upload(x), G, 1e-5, torch.from_numpy(gamma).cuda(),
                                          torch.from_numpy(beta).cuda())
    ref, rm, rr = oracle.groupnorm(x, G, 1e-5, gamma.astype(np.float64), beta.astype(np.float64))
    check(fetch(y), ref, dt, "y")
    check_stats(mean, rstd, rm, rr, "stats")


def test_groupnorm_in_place_and_deterministic():
    F, H, W, C, G = 33, 6, 6, 320, 32
    x = rnd((F, H, W, C), 77, BF)
    xd = upload(x)
    y1, m1, r1 = vinf.groupnorm_global(xd, G)
    y2, m2, r2 = vinf.groupnorm_global(xd, G)
    assert np.array_equal(bits(y1), bits(y2)) and torch.equal(m1, m2) and torch.equal(r1, r2)
    xi = xd.clone()
    y3, _, _ = vinf.groupnorm_global(xi, G, out=xi)
    assert y3.data_ptr() == xi.data_ptr()
    assert np.array_equal(bits(xi), bits(y1))


def test_groupnorm_drifting_mean():
    # Per-frame offset 0.3 t/F: the global mean is far from zero relative to
    # the per-voxel noise in late frames; two passes keep the variance exact.
    F, H, W, C, G = 2300, 2, 2, 64, 8
    x = synth.make_tensor(9, synth.X_GN, F, H, W, C, BF, slope=0.3)
    y, mean, rstd = vinf.groupnorm_global(upload(x), G)
    ref, rm, rr = oracle.groupnorm(x, G)
    check(fetch(y), ref, BF, "y")
    check_stats(mean, rstd, rm, rr, "stats")


# ------------------------------------------------------------- temporal conv

@pytest.mark.parametrize("F,H,W,C,dt,ctx,bias", [
    (16, 8, 5, 64, FP, False, False),     # the tiny float32 workload
    (37, 7, 9, 320, BF, False, False),    # ragged frame (8) and location (16) tiles, 2 N tiles of 160
    (19, 3, 7, 320, BF, True, True),
    (9, 5, 5, 128, BF, True, False),      # N tile 128
    (10, 4, 5, 64, BF, False, True),      # N tile 64
    (7, 3, 3, 96, BF, True, True),        # N tile 32
    (1, 4, 4, 640, BF, True, False),      # a single frame: both pads used
    (2, 1, 1, 1280, BF, False, False),
    (13, 2, 3, 40, FP, True, True),
])
def test_conv_small(F, H, W, C, dt, ctx, bias):
    announce(f"conv F={F} H={H} W={W} C={C} dt={dt} ctx={ctx} bias={bias}")
    x = rnd((F, H, W, C), 2000 + C + F, dt)
    w = rnd((3, C, C), 2100 + C, dt, 1 / math.sqrt(3 * C))
    pre = rnd((H, W, C), 2200 + C, dt) if ctx else None
    post = rnd((H, W, C), 2300 + C, dt) if ctx else None
    b = np.linspace(-0.3, 0.3, C).astype(np.float32) if bias else None
    y = vinf.temporal_conv3(upload(x), upload(w), None if pre is None else upload(pre),
                            None if post is None else upload(post), None if b is None else torch.from_numpy(b).cuda())
    ref = oracle.conv3(x, w, pre, post, None if b is None else b.astype(np.float64))
    check(fetch(y), ref, dt, "y")


def bf16_eye_taps(C, tap):
    w = np.zeros((3, C, C), np.float32)
    w[tap] = np.eye(C, dtype=np.float32)
    return (w.view(np.uint32) >> 16).astype(np.uint16)


def test_conv_identity_and_shift_bitwise():
    F, H, W, C = 21, 5, 7, 320
    x = rnd((F, H, W, C), 31, BF)
    pre, post = rnd((H, W, C), 32, BF), rnd((H, W, C), 33, BF)
    xd, pd, qd = upload(x), upload(pre), upload(post)
    y = vinf.temporal_conv3(xd, upload(bf16_eye_taps(C, 1)), pd, qd)
    assert np.array_equal(bits(y), x)
    y = vinf.temporal_conv3(xd, upload(bf16_eye_taps(C, 0)), pd, qd)   # y[f] = x[f-1], y[0] = ctx_pre
    yb = bits(y)
    assert np.array_equal(yb[1:], x[:-1]) and np.array_equal(yb[0], pre)
    y = vinf.temporal_conv3(xd, upload(bf16_eye_taps(C, 2)))           # y[f] = x[f+1], zero after the end
    yb = bits(y)
    assert np.array_equal(yb[:-1], x[1:]) and not yb[-1].any()


def test_conv_clip_split_equals_whole_bitwise():
    # The clip-parallel view on one GPU: each clip padded with its neighbours'
    # edge frames reproduces the whole-video result exactly.
    F, H, W, C = 40, 4, 6, 320
    x = rnd((F, H, W, C), 41, BF)
    w = rnd((3, C, C), 42, BF, 1 / math.sqrt(3 * C))
    xd, wd = upload(x), upload(w)
    whole = bits(vinf.temporal_conv3(xd, wd))
    for a, b in [(0, 13), (13, 29), (29, 40)]:
        pre = xd[a - 1].contiguous() if a > 0 else None
        post = xd[b].contiguous() if b < F else None
        part = vinf.temporal_conv3(xd[a:b].contiguous(), wd, pre, post)
        assert np.array_equal(bits(part), whole[a:b])


def test_conv_deterministic():
    F, H, W, C = 17, 6, 6, 640
    x, w = upload(rnd((F, H, W, C), 51, BF)), upload(rnd((3, C, C), 52, BF, 0.02))
    assert np.array_equal(bits(vinf.temporal_conv3(x, w)), bits(vinf.temporal_conv3(x, w)))


# --------------------------------------------------- dual-domain attention

@pytest.mark.parametrize("F,H,W,C,dt", [
    (16, 8, 5, 64, FP),      # the tiny float32 workload
    (1, 2, 3, 64, BF),
    (5, 3, 2, 128, BF),      # F < 16: local context = all frames, repeated global frames
    (16, 4, 4, 320, BF),
    (17, 3, 3, 64, BF),
    (40, 2, 5, 192, BF),
    (300, 2, 2, 320, BF),    # two query blocks of 256, ragged second block
    (513, 1, 3, 128, BF),    # three blocks, one query in the last
    (70, 3, 1, 128, FP),
    (256, 20, 20, 320, BF),  # 2000 whole-strip items: several per half
    (400, 16, 16, 128, BF),  # the same with a ragged second block (144 queries)
    # remainder packing at its boundaries (F = 256 + r): r = 36 fills four strips' slices, r = 37 takes two,
    # r = 104 fills two, r = 105 is a partial whole-strip item; F = 255 is one partial item per strip
    (292, 2, 3, 128, BF),
    (293, 2, 3, 128, BF),
    (360, 2, 2, 128, BF),
    (361, 2, 2, 128, BF),
    (255, 3, 2, 64, BF),
])
def test_attention_small(F, H, W, C, dt):
    announce(f"attention F={F} H={H} W={W} C={C} dt={dt}")
    q, k, v = (rnd((F, H, W, C), 3000 + 10 * i + F, dt) for i in range(3))
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v))
    check(fetch(o), oracle.dda(q, k, v), dt, "o")


def test_attention_closed_forms_on_gpu():
    F, H, W, C = 200, 2, 3, 128
    q, v = rnd((F, H, W, C), 61, BF), rnd((F, H, W, C), 62, BF)
    kc = np.broadcast_to(rnd((1, H, W, C), 63, BF), (F, H, W, C)).copy()
    o = fetch(vinf.dual_domain_attn(upload(q), upload(kc), upload(v)))
    vf = synth.bf16_bits_to_f32(v).reshape(F, H * W, C).astype(np.float64)
    for t in (0, 7, 8, 9, 100, 191, 192, 199):
        keys = oracle.dda_keys(F, t)
        check(o[t:t + 1], vf[keys].mean(axis=0, keepdims=True), BF, f"constant-K mean of V, t={t}")
    vc = np.broadcast_to(v[:1], v.shape).copy()
    o = fetch(vinf.dual_domain_attn(upload(q), upload(kc), upload(vc)))
    check(o, np.broadcast_to(vf[:1], o.shape), BF, "constant V")


def test_attention_scale_and_determinism():
    F, H, W, C = 64, 2, 2, 128
    q, k, v = (upload(rnd((F, H, W, C), 70 + i, BF)) for i in range(3))
    o1 = vinf.dual_domain_attn(q, k, v)
    o2 = vinf.dual_domain_attn(q, k, v, scale=0.125)
    assert np.array_equal(bits(o1), bits(o2))
    o3 = vinf.dual_domain_attn(q, k, v, scale=0.05)
    ref = oracle.dda(*(bits(t) for t in (q, k, v)), scale=0.05)
    check(fetch(o3), ref, BF, "scale 0.05")


@pytest.mark.parametrize("F,H,W,C", [(1024, 8, 5, 320), (300, 7, 3, 128), (2300, 2, 3, 192), (40, 5, 4, 64)])
def test_attention_item_orders_agree(F, H, W, C):
    """One tensor passed as q, k and v (the chain's case) takes the chunk-major
    item order; the same values in three buffers take the strip-major ranges.
    Each item is computed once in either order, so the outputs agree bit for
    bit; so do the one-sided key sets, which take the strip-major ranges both
    times, and both full-key outputs match the oracle at sampled locations."""
    announce(f"attention item orders F={F} H={H} W={W} C={C}")
    xh = rnd((F, H, W, C), 91, BF)
    x = upload(xh)
    k, v = x.clone(), x.clone()
    o1 = vinf.dual_domain_attn(x, x, x)
    o2 = vinf.dual_domain_attn(x, k, v)
    assert np.array_equal(bits(o1), bits(o2))
    for nl, ng in ((16, 0), (0, 16)):
        a1 = vinf.dual_domain_attn(x, x, x, n_local=nl, n_global=ng)
        a2 = vinf.dual_domain_attn(x, k, v, n_local=nl, n_global=ng)
        assert np.array_equal(bits(a1), bits(a2))
    locs = sample_locs(H * W, 3, seed=F)
    check(fetch(o1, locs), oracle.dda(xh, xh, xh, locs=locs), BF, "item orders, sampled")


# ------------------------------------------------------------- full workloads

CFG = synth.CONFIGS


def run_modules(cfgno):
    """Every module on its own seeded inputs at full size, sampled locations checked."""
    c = CFG[cfgno]
    F, H, W, C, G, dt = c["F"], c["H"], c["W"], c["C"], c["G"], c["dtype"]
    S = H * W
    locs = sample_locs(S, 8, seed=cfgno)
    announce(f"{c['name']}: groupnorm")
    x = synth.make_tensor(cfgno, synth.X_GN, F, H, W, C, dt, c["slope"])
    y, mean, rstd = vinf.groupnorm_global(upload(x), G)
    ref, rm, rr = oracle.groupnorm(x, G, locs=locs)
    check(fetch(y, locs), ref, dt, "groupnorm")
    check_stats(mean, rstd, rm, rr, "groupnorm stats")
    del x, y
    announce(f"{c['name']}: temporal conv")
    x = synth.make_tensor(cfgno, synth.X_CONV, F, H, W, C, dt, c["slope"])
    w = synth.make_conv_weight(cfgno, C, dt)
    y = vinf.temporal_conv3(upload(x), upload(w))
    check(fetch(y, locs), oracle.conv3(x, w, locs=locs), dt, "conv3")
    del x, y
    announce(f"{c['name']}: dual-domain attention")
    q, k, v = (synth.make_tensor(cfgno, tid, F, H, W, C, dt, c["slope"]) for tid in (synth.Q, synth.K, synth.V))
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v))
    check(fetch(o, locs), oracle.dda(q, k, v, locs=locs), dt, "attention")


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 values that are exactly bf16 -> uint16 bits."""
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_step(r: np.ndarray, d: np.ndarray) -> np.ndarray:
    """The bf16 neighbour of bf16 values r in direction d (+1 up, -1 down)."""
    b = to_bf16_bits(r).astype(np.int64)
    key = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF) + d
    nb = np.where(key >= 0, key, 0x8000 | (-key)).astype(np.uint32)
    return (nb << 16).view(np.float32).astype(np.float64)


def rounds_from(got: np.ndarray, exact: np.ndarray, eps: np.ndarray) -> np.ndarray:
    """Is bf16 value `got` the nearest rounding of some value within eps of
    `exact`?  (Its rounding interval meets [exact - eps, exact + eps].)"""
    lo = got - 0.5 * (got - bf16_step(got, -1))
    hi = got + 0.5 * (bf16_step(got, 1) - got)
    return (lo <= exact + eps) & (hi >= exact - eps)


U32 = 2.0 ** -24  # fp32 unit roundoff


def conv_abs_sum(xr: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_k sum_ci |W[k][co][ci]| |x[f+k-1, s, ci]| (zero pads) -- scales the fp32 error bound."""
    F, S, C = xr.shape
    ax = np.abs(xr).reshape(F, S * 1, C)
    pad = np.zeros((1, S, C))
    xp = np.concatenate([pad, ax, pad])
    aw = np.abs(synth.bf16_bits_to_f32(w).astype(np.float64).reshape(3, C, C))
    return sum(xp[k:k + F].reshape(-1, C) @ aw[k].T for k in range(3)).reshape(F, S, C)


def run_chain(cfgno):
    """GroupNorm -> conv3 -> attention with Q = K = V.

    Each module's output is a bf16 tensor, so both sides round the two
    intermediates, the kernels from fp32 and the oracle from fp64.  Where the
    exact value lies within the kernel's fp32 error of a rounding boundary,
    more than one bf16 value is a correct result.  The test checks (1) every
    stage of the full-size GPU chain against the oracle's exact values at the
    bar; (2) the GPU conv and attention on the oracle's own rounded
    intermediates at the bar; (3) that each GPU intermediate is the rounding
    of a value within a stated fp32 error bound of the exact one; (4) the
    final output at the bar against the oracle's attention over that
    validated intermediate; (5) the final output end to end against the
    oracle chain: mean-abs at the bar, max-abs at the bar where both sides
    rounded every conv value the attention reads alike, and elsewhere the
    bar plus the bound on how far those one-step differences move the
    attention (helpers.check_end_to_end)."""
    c = CFG[cfgno]
    F, H, W, C, G, dt = c["F"], c["H"], c["W"], c["C"], c["G"], c["dtype"]
    S = H * W
    locs = sample_locs(S, 8, seed=cfgno)
    nl = locs.size
    announce(f"{c['name']}: chain groupnorm -> conv3 -> attention")
    x = synth.make_tensor(cfgno, synth.X_GN, F, H, W, C, dt)
    w = synth.make_conv_weight(cfgno, C, dt)
    xd, wd = upload(x), upload(w)
    g, mean, rstd = vinf.groupnorm_global(xd, G)
    del xd
    cv = vinf.temporal_conv3(g, wd)
    gs = fetch(g, locs)
    del g
    o = vinf.dual_domain_attn(cv, cv, cv)
    cs, os_ = fetch(cv, locs), fetch(o, locs)
    del cv, o
    out, gn_r, cv_r, gn_x, cv_x, rm, rr = oracle.chain(x, w, G, locs=locs, exact=True)
    xs = synth.bf16_bits_to_f32(x.reshape(F, S, C)[:, locs]).astype(np.float64)
    del x
    check_stats(mean, rstd, rm, rr, "chain groupnorm stats")

    # (1) stages against the oracle's exact values
    check(gs, gn_x, dt, "chain groupnorm")
    check(cs, cv_x, dt, "chain conv3")

    # (2) GPU conv / attention on the oracle's rounded intermediates
    gcol = upload(to_bf16_bits(gn_r).reshape(F, 1, nl, C))
    check(fetch(vinf.temporal_conv3(gcol, wd)), oracle.conv3(to_bf16_bits(gn_r), w), dt, "conv3 on oracle input")
    ccol = upload(to_bf16_bits(cv_r).reshape(F, 1, nl, C))
    check(fetch(vinf.dual_domain_attn(ccol, ccol, ccol)), out, dt, "attention on oracle input")
    del gcol, ccol

    # (3) GPU intermediates are correct roundings of values within the
    # kernels' fp32 error of the exact ones.  groupnorm: y = x*a + b in fp32
    # with a, b rounded from the statistics -> a few ulp of |x*a| + |b|.
    mg = np.repeat(rm, C // G)
    rg = np.repeat(rr, C // G)
    eps_g = 8 * U32 * (np.abs(xs * rg) + np.abs(mg * rg))
    assert np.all(rounds_from(gs, gn_x, eps_g)), "groupnorm output is not a rounding of its value"
    # conv: fp32 accumulation of 3C products in MFMA blocks of 32 (at most
    # 3C/32 + 2 roundings of partial sums bounded by sum |w x|), plus the exact
    # effect of the groupnorm values the GPU rounded the other way.
    eps_c = (3 * C // 32 + 2) * U32 * conv_abs_sum(gn_r, w) + conv_abs_sum(np.abs(gs - gn_r), w)
    assert np.all(rounds_from(cs, cv_x, eps_c)), "conv3 output is not a rounding of its value"
    announce(f"  intermediates rounded differently from the oracle: groupnorm {int((gs != gn_r).sum())}, "
             f"conv3 {int((cs != cv_r).sum())} of {cs.size}")

    # (4) final output over the validated intermediate
    cb = to_bf16_bits(cs)
    o_on_gpu_conv = oracle.dda(cb, cb, cb)
    check(os_, o_on_gpu_conv, dt, "chain attention")

    # (5) end to end against the oracle chain itself
    check_end_to_end(os_, out, o_on_gpu_conv, cv_r, cs, dt, "chain")



@pytest.mark.parametrize("cfgno", [1, 2, 3, 4])
def test_workload_modules(cfgno):
    run_modules(cfgno)


@pytest.mark.parametrize("cfgno", [5, 6])
def test_workload_chain(cfgno):
    run_chain(cfgno)
