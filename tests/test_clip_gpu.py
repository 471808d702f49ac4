"""Clip-parallel forms and attention ablations on the GPU, through the C ABI.

A clip plus its context must give the whole video's result for its frames:
bit for bit for attention (each query's arithmetic does not depend on where
the clip starts) and for GroupNorm when one clip covers the video; within the
parity bar (against the oracle) when the group sums of several clips are
added.  The ablation variants (local context only, global context only) are
checked against the oracle element by element.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, check_stats, dev, fetch, sample_locs, upload

pytestmark = pytest.mark.gpu

BF, FP = synth.BF16, synth.F32


def rnd(shape, seed, dt, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, dt, scale).reshape(shape)


def global_rows(F, G=16):
    return [i * F // G for i in range(G)]


# ------------------------------------------------------- attention, clips

# F = 600: three work items of 256 query frames per strip, the last ragged;
# clips shorter than a window, at both ends, and spanning item boundaries;
# clip lengths 361 (a ragged second whole-strip item) and 292 (a remainder of
# 36 queries per strip, four strips to an item).
CLIPS_600 = [(0, 9), (9, 300), (300, 555), (555, 597), (597, 600), (255, 257), (0, 600), (100, 461), (200, 492)]


@pytest.mark.parametrize("dt", [BF, FP])
def test_attention_clip_equals_whole_bitwise(dt):
    F, H, W, C = 600, 4, 5, 128
    announce(f"attention clip vs whole F={F} H={H} W={W} C={C} dt={dt}")
    q, k, v = (upload(rnd((F, H, W, C), 3000 + i, dt)) for i in range(3))
    whole = bits(vinf.dual_domain_attn(q, k, v))
    gi = torch.tensor(global_rows(F), device=dev())
    kg, vg = k.index_select(0, gi).contiguous(), v.index_select(0, gi).contiguous()
    for f0, f1 in CLIPS_600:
        Fc = f1 - f0
        pre, post = vinf.dda_clip_halo(F, f0, Fc)
        ks, vs = k[f0 - pre:f1 + post], v[f0 - pre:f1 + post]
        o = vinf.dual_domain_attn_clip(q[f0:f1], ks, vs, F, f0, pre, post, kg, vg)
        assert np.array_equal(bits(o), whole[f0:f1]), (f0, f1, "external global rows")
        # global rows read in place: the context buffers hold the whole video
        o = vinf.dual_domain_attn_clip(q[f0:f1], k, v, F, f0, f0, F - f1)
        assert np.array_equal(bits(o), whole[f0:f1]), (f0, f1, "global rows in place")


@pytest.mark.parametrize("dt", [BF, FP])
def test_attention_clip_external_globals_vs_oracle(dt):
    # Global rows that differ from the clip buffer's frames (the gathered
    # global context of other devices): every output element vs the oracle.
    F, H, W, C = 700, 3, 4, 128
    f0, f1 = 250, 530
    announce(f"attention clip external globals F={F} clip=[{f0},{f1}) dt={dt}")
    pre, post = vinf.dda_clip_halo(F, f0, f1 - f0)
    assert (pre, post) == (8, 7)
    n_ext = pre + (f1 - f0) + post
    q = rnd((f1 - f0, H, W, C), 3100, dt)
    k, v = rnd((n_ext, H, W, C), 3101, dt), rnd((n_ext, H, W, C), 3102, dt)
    kg, vg = rnd((16, H, W, C), 3103, dt), rnd((16, H, W, C), 3104, dt)
    o = vinf.dual_domain_attn_clip(upload(q), upload(k), upload(v), F, f0, pre, post, upload(kg), upload(vg))
    ref = oracle.dda_clip(q, k, v, F, f0, f0 - pre, kg, vg)
    check(fetch(o), ref, dt, "o")


def test_attention_clip_at_workload_size():
    # One of eight clips of a 2300-frame video at 64x40x320, with its 8 + 7
    # context frames and the 16 global rows: bit for bit against the
    # whole-video call, sampled locations against the oracle.
    F, H, W, C = 2300, 64, 40, 320
    f0, Fc = 864, 288
    announce(f"attention clip at workload size F={F} clip=[{f0},{f0 + Fc}) {H}x{W}x{C} bf16")
    g = torch.Generator(device=dev())
    g.manual_seed(2300)
    q, k, v = (torch.randn((F, H, W, C), generator=g, device=dev()).to(torch.bfloat16) for _ in range(3))
    pre, post = vinf.dda_clip_halo(F, f0, Fc)
    gi = torch.tensor(global_rows(F), device=dev())
    kg, vg = k.index_select(0, gi).contiguous(), v.index_select(0, gi).contiguous()
    o = vinf.dual_domain_attn_clip(q[f0:f0 + Fc], k[f0 - pre:f0 + Fc + post], v[f0 - pre:f0 + Fc + post], F, f0,
                                   pre, post, kg, vg)
    whole = vinf.dual_domain_attn(q, k, v)
    assert torch.equal(o.view(torch.int16), whole[f0:f0 + Fc].view(torch.int16))
    del whole
    locs = sample_locs(H * W, 6, seed=5)
    li = torch.as_tensor(locs, device=dev())

    def cols(t):
        a = t.reshape(t.shape[0], H * W, C)[:, li].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        return a.reshape(t.shape[0], len(locs), 1, C)

    ref = oracle.dda_clip(cols(q[f0:f0 + Fc]), cols(k[f0 - pre:f0 + Fc + post]), cols(v[f0 - pre:f0 + Fc + post]),
                          F, f0, f0 - pre, cols(kg), cols(vg))
    check(fetch(o, locs), ref, BF, "o (sampled locations)")


# ------------------------------------------------- attention, ablations

@pytest.mark.parametrize("nl,ng", [(16, 0), (0, 16)])
@pytest.mark.parametrize("F,H,W,C,dt", [
    (600, 3, 4, 128, BF),    # several items per strip, ragged tail
    (256, 20, 20, 128, BF),  # 800 whole-strip items: several per half
    (292, 2, 3, 64, BF),     # remainder of 36 queries per strip: four strips per item
    (300, 2, 3, 192, FP),
    (17, 4, 4, 64, BF),      # one window short of a full item
    (5, 3, 3, 64, BF),       # fewer frames than a window
    (1, 2, 2, 64, FP),
])
def test_attention_ablation_vs_oracle(nl, ng, F, H, W, C, dt):
    announce(f"attention n_local={nl} n_global={ng} F={F} H={H} W={W} C={C} dt={dt}")
    q, k, v = (rnd((F, H, W, C), 3200 + F + i, dt) for i in range(3))
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v), n_local=nl, n_global=ng)
    ref = oracle.dda(q, k, v, n_local=nl, n_global=ng)
    check(fetch(o), ref, dt, "o")


@pytest.mark.parametrize("nl,ng", [(16, 0), (0, 16)])
def test_attention_ablation_clip_equals_whole_bitwise(nl, ng):
    F, H, W, C = 600, 2, 4, 128
    announce(f"attention ablation clips n_local={nl} n_global={ng} F={F}")
    q, k, v = (upload(rnd((F, H, W, C), 3300 + i, BF)) for i in range(3))
    whole = bits(vinf.dual_domain_attn(q, k, v, n_local=nl, n_global=ng))
    gi = torch.tensor(global_rows(F), device=dev())
    kg, vg = k.index_select(0, gi).contiguous(), v.index_select(0, gi).contiguous()
    for f0, f1 in CLIPS_600:
        pre, post = vinf.dda_clip_halo(F, f0, f1 - f0, nl)
        globs = (kg, vg) if ng else (None, None)
        o = vinf.dual_domain_attn_clip(q[f0:f1], k[f0 - pre:f1 + post], v[f0 - pre:f1 + post], F, f0, pre, post,
                                       *globs, n_local=nl, n_global=ng)
        assert np.array_equal(bits(o), whole[f0:f1]), (f0, f1)


# ------------------------------------------------------- GroupNorm, clips

@pytest.mark.parametrize("dt", [BF, FP])
def test_groupnorm_one_clip_is_whole_bitwise(dt):
    F, H, W, C, G = 37, 7, 9, 320, 32
    announce(f"groupnorm one clip vs whole F={F} C={C} G={G} dt={dt}")
    x = upload(rnd((F, H, W, C), 3400, dt))
    gamma = torch.linspace(0.5, 1.25, C, device=dev())
    beta = torch.linspace(-0.5, 0.5, C, device=dev())
    y, m, r = vinf.groupnorm_global(x, G, 1e-5, gamma, beta)
    s1 = vinf.groupnorm_clip_sums(x, G, F)
    s2 = vinf.groupnorm_clip_sums(x, G, F, s1)
    y2, m2, r2 = vinf.groupnorm_clip_apply(x, G, F, s1, s2, 1e-5, gamma, beta)
    assert np.array_equal(bits(y), bits(y2))
    assert torch.equal(m, m2) and torch.equal(r, r2)


@pytest.mark.parametrize("dt", [BF, FP])
def test_groupnorm_clips_with_aggregated_sums(dt):
    # Three clips of a drifting-mean video (so that a clip's own statistics
    # are wrong for it); their sums added on the device stand in for the
    # all-reduce across devices.
    F, H, W, C, G = 61, 6, 5, 320, 32
    announce(f"groupnorm three clips F={F} C={C} G={G} dt={dt}")
    xh = synth.normal(F * H * W * C, 3500, dt, 1.0, H * W * C, 2.0 / F).reshape(F, H, W, C)
    x = upload(xh)
    clips = [(0, 13), (13, 40), (40, 61)]
    s1 = sum(vinf.groupnorm_clip_sums(x[a:b], G, F) for a, b in clips)
    s2 = sum(vinf.groupnorm_clip_sums(x[a:b], G, F, s1) for a, b in clips)
    ys, stats = [], []
    for a, b in clips:
        y, m, r = vinf.groupnorm_clip_apply(x[a:b], G, F, s1, s2)
        ys.append(fetch(y))
        stats.append((m, r))
    ref, rm, rr = oracle.groupnorm(xh, G)
    check(np.concatenate(ys), ref, dt, "y")
    for m, r in stats:
        check_stats(m, r, rm, rr, "stats")
    # the first clip's own mean sits below the global one
    own = vinf.groupnorm_clip_sums(x[0:13], G, 13).cpu().numpy() / (13 * H * W * C // G)
    assert np.all(own < rm - 0.5)
    # in place
    xi = x[13:40].clone()
    vinf.groupnorm_clip_apply(xi, G, F, s1, s2, out=xi)
    assert np.array_equal(bits(xi), bits(vinf.groupnorm_clip_apply(x[13:40], G, F, s1, s2)[0]))
