"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes the oracle to a closed form, a hand-derived fixture under
tests/golden/, brute force on tiny inputs, or an independent library routine
(torch CPU float64), chosen so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def randn(shape, seed, dtype=synth.F32, scale=1.0):
    n = int(np.prod(shape))
    return synth.normal(n, seed, dtype, scale).reshape(shape)


def grid(a):
    """Round to multiples of 1/64 in [-4, 4]: small integer combinations stay exact in float32."""
    return (np.clip(np.round(a * 64), -256, 256) / 64).astype(np.float32)


def widen(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


# ---------------------------------------------------------------- GroupNorm

def test_gn_hand_example():
    g = gold("gn_tiny.json")
    x = np.array(g["x"], dtype=np.float32).reshape(2, 1, 4)
    mean, var, rstd = oracle.gn_stats(x, g["G"], g["eps"])
    assert np.array_equal(mean, g["mean"]) and np.array_equal(var, g["var"])
    y, _, _ = oracle.groupnorm(x, g["G"], g["eps"])
    xv = np.array(g["x"], dtype=np.float64)
    for c in range(4):
        gi = c // 2
        expect = (xv[:, c] - g["mean"][gi]) / math.sqrt(g["var"][gi] + g["eps"])
        assert np.allclose(y[:, 0, c], expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("F,S,C,G,dt", [(16, 40, 64, 8, synth.F32), (7, 13, 96, 32, synth.BF16),
                                         (3, 5, 40, 4, synth.BF16), (1, 1, 8, 1, synth.F32)])
def test_gn_matches_torch_group_norm(F, S, C, G, dt):
    x = randn((F, S, C), 11 + F, dt)
    gamma = np.linspace(0.5, 1.5, C)
    beta = np.linspace(-1, 1, C)
    y, mean, rstd = oracle.groupnorm(x, G, 1e-5, gamma, beta)
    xt = torch.from_numpy(widen(x).astype(np.float64)).reshape(F * S, C).T.reshape(1, C, F * S)
    ref = torch.nn.functional.group_norm(xt, G, torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-5)
    ref = ref.reshape(C, F, S).permute(1, 2, 0).numpy()
    assert np.abs(y - ref).max() < 1e-12


def test_gn_closed_forms():
    # Output group mean is 0 and output group variance is v/(v+eps), v the
    # population variance of the input group (numpy's np.var).
    F, S, C, G, eps = 9, 11, 48, 6, 0.3
    x = randn((F, S, C), 5, synth.BF16)
    y, _, _ = oracle.groupnorm(x, G, eps)
    xf = widen(x).astype(np.float64)
    for g in range(G):
        cs = slice(g * C // G, (g + 1) * C // G)
        v = np.var(xf[:, :, cs])
        assert abs(y[:, :, cs].mean()) < 1e-14
        assert abs(np.var(y[:, :, cs]) - v / (v + eps)) < 1e-13


def test_gn_affine_invariance():
    # x -> a*x + b_g with eps -> a^2 eps leaves y unchanged (a power of two keeps inputs exact).
    F, S, C, G = 5, 6, 32, 4
    # inputs on a 1/64 grid in [-4, 4] so that 4*x + b is exact in float32
    x = grid(randn((F, S, C), 7, synth.F32))
    b = np.repeat(np.array([3.0, -1.5, 0.25, 8.0], dtype=np.float32), C // G)
    x2 = (4.0 * x + b).astype(np.float32)
    y1, _, _ = oracle.groupnorm(x, G, 1e-3)
    y2, _, _ = oracle.groupnorm(x2, G, 16e-3)
    assert np.abs(y1 - y2).max() < 1e-12


def test_gn_global_not_per_frame():
    # Per-frame offset 0.3*t/F (the long-video drift case): the global mean is
    # 0.3*(F-1)/(2F) up to noise and the global variance is 1 + 0.09*(F^2-1)/(12F^2).
    F, S, C, G = 2300, 4, 16, 2
    x = synth.normal(F * S * C, 99, synth.F32, 1.0, S * C, 0.3 / F).reshape(F, S, C)
    mean, var, _ = oracle.gn_stats(x, G)
    n = F * S * C // G
    assert np.all(np.abs(mean - 0.3 * (F - 1) / (2 * F)) < 5 / math.sqrt(n))
    assert np.all(np.abs(var - (1 + 0.09 * (F * F - 1) / (12 * F * F))) < 10 * math.sqrt(2 / n))


def test_gn_location_subset_is_exact():
    F, S, C, G = 6, 10, 32, 4
    x = randn((F, S, C), 3, synth.BF16)
    yall, _, _ = oracle.groupnorm(x, G)
    locs = [9, 0, 4]
    ysub, _, _ = oracle.groupnorm(x, G, locs=locs)
    assert np.array_equal(ysub, yall[:, locs, :])


# ------------------------------------------------------------ temporal conv

def test_conv_hand_example():
    g = gold("conv_tiny.json")
    x = np.array(g["x"], dtype=np.float32).reshape(3, 1, 1)
    w = np.array(g["w"], dtype=np.float32).reshape(3, 1, 1)
    assert np.array_equal(oracle.conv3(x, w)[:, 0, 0], g["y_zero_pad"])
    pre = np.array([g["ctx_pre"]], dtype=np.float32).reshape(1, 1)
    post = np.array([g["ctx_post"]], dtype=np.float32).reshape(1, 1)
    assert np.array_equal(oracle.conv3(x, w, pre, post)[:, 0, 0], g["y_ctx"])


@pytest.mark.parametrize("F,S,C,dt,ctx", [(16, 40, 64, synth.F32, False), (9, 7, 24, synth.BF16, True),
                                           (1, 3, 16, synth.F32, True), (2, 2, 8, synth.BF16, False)])
def test_conv_matches_torch_conv1d(F, S, C, dt, ctx):
    x = randn((F, S, C), 21, dt)
    w = randn((3, C, C), 22, dt, 1 / math.sqrt(3 * C))
    pre = randn((S, C), 23, dt) if ctx else None
    post = randn((S, C), 24, dt) if ctx else None
    bias = np.linspace(-0.5, 0.5, C)
    y = oracle.conv3(x, w, pre, post, bias)
    xs = torch.from_numpy(widen(x).astype(np.float64)).permute(1, 2, 0)  # [S, C, F]
    z = torch.zeros(S, C, 1, dtype=torch.float64)
    left = torch.from_numpy(widen(pre).astype(np.float64)).reshape(S, C, 1) if ctx else z
    right = torch.from_numpy(widen(post).astype(np.float64)).reshape(S, C, 1) if ctx else z
    xp = torch.cat([left, xs, right], dim=2)
    wt = torch.from_numpy(widen(w).astype(np.float64)).permute(1, 2, 0).contiguous()  # [C_out, C_in, 3]
    ref = torch.nn.functional.conv1d(xp, wt, torch.from_numpy(bias)).permute(2, 0, 1).numpy()
    assert np.abs(y - ref).max() < 1e-11


def test_conv_identity_and_shift_kernels():
    F, S, C = 7, 5, 16
    x = randn((F, S, C), 31, synth.BF16)
    pre, post = randn((S, C), 32, synth.BF16), randn((S, C), 33, synth.BF16)
    eye = np.eye(C, dtype=np.float32)
    zero = np.zeros((C, C), np.float32)
    xf, pf, qf = (widen(a).astype(np.float64) for a in (x, pre, post))

    def bf(w):  # exact bf16 bits of 0/1 matrices
        return (w.view(np.uint32) >> 16).astype(np.uint16)

    y = oracle.conv3(x, bf(np.stack([zero, eye, zero])), pre, post)
    assert np.array_equal(y, xf)
    y = oracle.conv3(x, bf(np.stack([eye, zero, zero])), pre, post)  # tap 0 reads frame f-1
    assert np.array_equal(y[1:], xf[:-1]) and np.array_equal(y[0], pf)
    y = oracle.conv3(x, bf(np.stack([zero, zero, eye])), pre, post)  # tap 2 reads frame f+1
    assert np.array_equal(y[:-1], xf[1:]) and np.array_equal(y[-1], qf)
    y = oracle.conv3(x, bf(np.stack([eye, zero, zero])))  # no context: zero padding
    assert np.array_equal(y[0], np.zeros((S, C)))


def test_conv_weight_orientation():
    # W[k][c_out][c_in]: a single nonzero W[1][a][b] = 1 copies input channel b to output channel a.
    F, S, C = 4, 3, 8
    x = randn((F, S, C), 41, synth.F32)
    w = np.zeros((3, C, C), np.float32)
    w[1, 2, 5] = 1.0
    y = oracle.conv3(x, w)
    assert np.array_equal(y[:, :, 2], x[:, :, 5].astype(np.float64))
    assert np.count_nonzero(np.delete(y, 2, axis=2)) == 0


def test_conv_linearity():
    F, S, C = 6, 4, 16
    x1, x2 = grid(randn((F, S, C), 51)), grid(randn((F, S, C), 52))
    w = randn((3, C, C), 53, synth.F32, 0.1)
    y = oracle.conv3((2 * x1 - x2).astype(np.float32), w)
    assert np.abs(y - (2 * oracle.conv3(x1, w) - oracle.conv3(x2, w))).max() < 1e-12


def test_conv_clip_split_equals_whole():
    # Cutting the video into clips and padding each with its neighbours' edge
    # frames gives the whole-video result (clip parallelism).
    F, S, C = 12, 3, 16
    x = randn((F, S, C), 61, synth.BF16)
    w = randn((3, C, C), 62, synth.BF16, 0.2)
    whole = oracle.conv3(x, w)
    parts = []
    for a, b in [(0, 5), (5, 9), (9, 12)]:
        pre = x[a - 1] if a > 0 else None
        post = x[b] if b < F else None
        parts.append(oracle.conv3(x[a:b], w, pre, post))
    assert np.array_equal(np.concatenate(parts), whole)


# ------------------------------------------------- dual-domain attention

def key_multiset(F, t, L=16, G=16):
    """Independent construction of the key frames of query t: the window of
    min(L,F) consecutive in-range frames whose start is nearest to t - L//2,
    followed by the frames i*F//G."""
    n = min(L, F)
    starts = range(0, F - n + 1)
    st = min(starts, key=lambda s: abs(s - (t - L // 2)))
    return list(range(st, st + n)) + [i * F // G for i in range(G)]


def test_dda_key_frames_hand_tables():
    g = gold("dda_key_frames.json")
    for case in g["cases"]:
        F = case["F"]
        n = case.get("local_len", 16)
        for t, st in case["local_start"]:
            keys = oracle.dda_keys(F, t)
            assert list(keys) == list(range(st, st + n)) + case["global"], (F, t)
            assert list(keys) == key_multiset(F, t), (F, t)


def test_dda_key_frames_all_queries():
    for F in list(range(1, 40)) + [127, 128, 129, 1024, 2300]:
        for t in range(F):
            assert list(oracle.dda_keys(F, t)) == key_multiset(F, t)


def test_dda_hand_example_equal_scores():
    g = gold("dda_tiny.json")
    F, d = g["F"], g["head_dim"]
    q = np.zeros((F, 1, d), np.float32)
    k = randn((F, 1, d), 71)
    v = np.stack([np.full((1, d), t + 1.0, np.float32) for t in range(F)])
    o = oracle.dda(q, k, v, head_dim=d)
    assert np.abs(o - g["expected_o"]).max() < 1e-14
    counts = np.bincount(key_multiset(F, 0), minlength=F)
    assert list(counts) == g["multiplicity"]


def test_dda_hand_example_score_ratio():
    c = gold("dda_tiny.json")["case2"]
    F, d = c["F"], 64
    q = np.zeros((F, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((F, 1, d), np.float32)
    k[0, 0, 0] = c["k0_dim0"]
    v = np.zeros((F, 1, d), np.float32)
    v[0] = 3.0
    o = oracle.dda(q, k, v)  # scale 1/sqrt(64) = 1/8
    assert np.abs(o - c["expected_o"]).max() < 1e-6  # k0 is ln2*8 rounded to float32


def sdpa_multiset(q, k, v, scale):
    """torch scaled_dot_product_attention (fp64) with additive mask log(multiplicity)."""
    F, S, C = q.shape
    H = C // 64
    mult = np.zeros((F, F))
    for t in range(F):
        for j in key_multiset(F, t):
            mult[t, j] += 1
    with np.errstate(divide="ignore"):
        mask = torch.from_numpy(np.log(mult))
    def heads(a):
        return torch.from_numpy(widen(a).astype(np.float64)).reshape(F, S, H, 64).permute(1, 2, 0, 3)
    o = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v), attn_mask=mask,
                                                         scale=scale)
    return o.permute(2, 0, 1, 3).reshape(F, S, C).numpy()


@pytest.mark.parametrize("F", [1, 2, 3, 5, 16, 17, 23, 40, 70])
def test_dda_matches_sdpa_with_multiplicity_mask(F):
    S, C = 3, 128
    q, k, v = (randn((F, S, C), 80 + i, synth.BF16) for i in range(3))
    o = oracle.dda(q, k, v)
    assert np.abs(o - sdpa_multiset(q, k, v, 0.125)).max() < 1e-12


@pytest.mark.parametrize("F", [1, 2, 4, 8, 16])
def test_dda_equals_full_attention_when_uniform(F):
    # F in {1,2,4,8,16}: every frame has the same multiplicity 1 + 16/F, so the
    # method equals plain full temporal attention.
    S, C = 2, 64
    q, k, v = (randn((F, S, C), 90 + i) for i in range(3))
    o = oracle.dda(q, k, v)
    def heads(a):
        return torch.from_numpy(a.astype(np.float64)).permute(1, 0, 2)  # [S, F, C] one head
    ref = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v)).permute(1, 0, 2).numpy()
    assert np.abs(o - ref).max() < 1e-12
    # brute force, plain numpy
    qd, kd, vd = (a.astype(np.float64) for a in (q, k, v))
    for s in range(S):
        sc = qd[:, s] @ kd[:, s].T / 8.0
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.abs(o[:, s] - p @ vd[:, s]).max() < 1e-12


def test_dda_closed_forms():
    F, S, C = 50, 3, 128
    q, k, v = (randn((F, S, C), 100 + i) for i in range(3))
    # K constant over frames: all scores equal -> mean of V over the key multiset.
    kc = np.broadcast_to(k[:1], k.shape).copy()
    o = oracle.dda(q, kc, v)
    for t in (0, 8, 9, 25, 41, 42, 49):
        keys = key_multiset(F, t)
        assert np.abs(o[t] - v[keys].astype(np.float64).mean(axis=0)).max() < 1e-13
    # V constant over frames: o = V.
    vc = np.broadcast_to(v[:1], v.shape).copy()
    o = oracle.dda(q, k, vc)
    assert np.abs(o - vc[0].astype(np.float64)).max() < 1e-13
    # Same vector added to every key row: scores shift per query, o unchanged.
    c = randn((1, S, C), 104)
    o1 = oracle.dda(q, k, v)
    o2 = oracle.dda(q, (k + c).astype(np.float32), v)
    assert np.abs(o1 - o2).max() < 1e-6  # k + c is rounded to float32
    # Linear in V.
    v, v2 = grid(v), grid(randn((F, S, C), 105))
    o1 = oracle.dda(q, k, v)
    o3 = oracle.dda(q, k, (2 * v - v2).astype(np.float32))
    assert np.abs(o3 - (2 * o1 - oracle.dda(q, k, v2))).max() < 1e-12


def test_dda_dominant_key():
    # One global frame's key made huge along q: its value takes over.
    F, S, C = 64, 1, 64
    q = np.ones((F, S, C), np.float32)
    k = randn((F, S, C), 110, scale=0.01)
    v = randn((F, S, C), 111)
    k[32] = 100.0  # frame 32 = floor(8*64/16), a global frame of every query
    o = oracle.dda(q, k, v)
    assert np.abs(o - v[32].astype(np.float64)).max() < 1e-12


def test_dda_scale_argument():
    F, S, C = 20, 2, 64
    q, k, v = (randn((F, S, C), 120 + i) for i in range(3))
    o_def = oracle.dda(q, k, v)
    o_exp = oracle.dda(q, k, v, scale=0.125)
    assert np.array_equal(o_def, o_exp)
    o2 = oracle.dda((2 * q).astype(np.float32), k, v, scale=0.0625)
    assert np.abs(o2 - o_def).max() < 1e-13


# ------------------------------------------------------------------ chain

def test_chain_composes_the_three_modules():
    F, S, C, G = 20, 6, 128, 8
    x = randn((F, S, C), 130, synth.BF16)
    w = randn((3, C, C), 131, synth.BF16, 1 / math.sqrt(3 * C))
    out, gn, cv, mean, rstd = oracle.chain(x, w, G, intermediates=True)
    y, _, _ = oracle.groupnorm(x, G)
    gn_ref = np.vectorize(lambda a: oracle.round_to(a, synth.BF16))(y)
    assert np.array_equal(gn, gn_ref)
    bits = (gn.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    cv_ref = np.vectorize(lambda a: oracle.round_to(a, synth.BF16))(oracle.conv3(bits, w))
    assert np.array_equal(cv, cv_ref)
    cb = (cv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(out, oracle.dda(cb, cb, cb))
    locs = [5, 1]
    out_s, _, _ = oracle.chain(x, w, G, locs=locs)
    assert np.array_equal(out_s, out[:, locs])
    # the exact (pre-rounding) intermediates
    _, gn2, cv2, gx, cx, _, _ = oracle.chain(x, w, G, exact=True)
    assert np.array_equal(gx, y) and np.array_equal(gn2, gn) and np.array_equal(cv2, cv)
    assert np.array_equal(cx, oracle.conv3(bits, w))


def test_round_to_bf16_matches_torch():
    vals = synth.normal(4096, 140, synth.F32, 3.0).astype(np.float64)  # float32-exact: one rounding step
    ours = np.array([oracle.round_to(v, synth.BF16) for v in vals])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
