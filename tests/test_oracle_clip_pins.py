"""Pins of the oracle's clip-parallel routines and attention ablations (CPU only).

The clip routines are fixed to the whole-video routines through the property
clip parallelism rests on (a clip plus its context gives the whole video's
result for its frames), to numpy brute force built from an independent key
construction, and to closed forms.  The ablations (local context only, global
context only) are fixed to torch's attention with an explicit mask.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def randn(shape, seed, dtype=synth.F32, scale=1.0):
    n = int(np.prod(shape))
    return synth.normal(n, seed, dtype, scale).reshape(shape)


def widen(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def local_frames(F, t, L=16):
    """The window of min(L,F) consecutive in-range frames whose start is
    nearest to t - L//2 (built without the oracle's clamp)."""
    n = min(L, F)
    if n == 0:
        return []
    st = min(range(0, F - n + 1), key=lambda s: abs(s - (t - L // 2)))
    return list(range(st, st + n))


def global_frames(F, G=16):
    return [i * F // G for i in range(G)]


def needed(F, f0, Fc, L=16):
    """First and last local key frame of the clip's queries."""
    fr = [j for t in range(f0, f0 + Fc) for j in local_frames(F, t, L)]
    return min(fr), max(fr)


# ------------------------------------------------- attention, clip form

CLIPS = [(0, 9), (9, 40), (40, 62), (62, 70)]


def test_dda_clip_split_equals_whole():
    F, S, C = 70, 3, 128
    q, k, v = (randn((F, S, C), 150 + i, synth.BF16) for i in range(3))
    whole = oracle.dda(q, k, v)
    gi = global_frames(F)
    for f0, f1 in CLIPS:
        lo, hi = needed(F, f0, f1 - f0)
        o = oracle.dda_clip(q[f0:f1], k[lo:hi + 1], v[lo:hi + 1], F, f0, lo, k[gi], v[gi])
        assert np.array_equal(o, whole[f0:f1]), (f0, f1)
        # global rows read in place from buffers that hold the whole video
        o2 = oracle.dda_clip(q[f0:f1], k, v, F, f0, 0)
        assert np.array_equal(o2, whole[f0:f1]), (f0, f1)


def test_dda_clip_external_globals_brute_force():
    # Global rows that are not the clip buffer's own frames: the result must
    # take them from k_glob / v_glob, the local rows from the halo buffer.
    F, S, C = 300, 2, 64
    f0, f1 = 120, 150
    q, k, v = (randn((F, S, C), 160 + i) for i in range(3))
    kg, vg = randn((16, S, C), 163), randn((16, S, C), 164)
    lo, hi = needed(F, f0, f1 - f0)
    assert (lo, hi) == (f0 - 8, f1 + 6)
    o = oracle.dda_clip(q[f0:f1], k[lo:hi + 1], v[lo:hi + 1], F, f0, lo, kg, vg)
    for t in range(f0, f1):
        loc = local_frames(F, t)
        for s in range(S):
            K = np.concatenate([k[loc, s], kg[:, s]]).astype(np.float64)
            V = np.concatenate([v[loc, s], vg[:, s]]).astype(np.float64)
            sc = K @ q[t, s].astype(np.float64) / 8.0
            p = np.exp(sc - sc.max())
            ref = p @ V / p.sum()
            assert np.abs(o[t - f0, s] - ref).max() < 1e-12, (t, s)


def test_dda_clip_at_video_ends_and_short_clips():
    # Clips shorter than the window and clips at either end: the window is
    # shifted inward, so the halo can exceed 8 before / 7 after.
    F, S, C = 40, 2, 64
    q, k, v = (randn((F, S, C), 170 + i) for i in range(3))
    whole = oracle.dda(q, k, v)
    gi = global_frames(F)
    for f0, f1 in [(0, 1), (0, 3), (5, 6), (37, 40), (39, 40), (20, 21)]:
        lo, hi = needed(F, f0, f1 - f0)
        o = oracle.dda_clip(q[f0:f1], k[lo:hi + 1], v[lo:hi + 1], F, f0, lo, k[gi], v[gi])
        assert np.array_equal(o, whole[f0:f1]), (f0, f1)
    assert needed(F, 39, 1) == (24, 39)  # 15 frames before the query
    assert needed(F, 0, 1) == (0, 15)    # 15 frames after


def test_dda_clip_rejects_missing_context():
    F, S, C = 100, 1, 64
    q, k, v = (randn((F, S, C), 180 + i) for i in range(3))
    f0, f1 = 40, 60
    lo, hi = needed(F, f0, f1 - f0)
    gi = global_frames(F)
    with pytest.raises(ValueError, match="rc=3"):  # one frame short before
        oracle.dda_clip(q[f0:f1], k[lo + 1:hi + 1], v[lo + 1:hi + 1], F, f0, lo + 1, k[gi], v[gi])
    with pytest.raises(ValueError, match="rc=3"):  # one frame short after
        oracle.dda_clip(q[f0:f1], k[lo:hi], v[lo:hi], F, f0, lo, k[gi], v[gi])
    with pytest.raises(ValueError, match="rc=3"):  # global rows not supplied and not in the buffer
        oracle.dda_clip(q[f0:f1], k[lo:hi + 1], v[lo:hi + 1], F, f0, lo)
    # the local-only ablation needs no global rows at all
    o = oracle.dda_clip(q[f0:f1], k[lo:hi + 1], v[lo:hi + 1], F, f0, lo, n_global=0)
    assert np.array_equal(o, oracle.dda(q, k, v, n_global=0)[f0:f1])


# --------------------------------------------- attention, ablation variants

def sdpa_masked(q, k, v, allowed):
    """torch attention (fp64, one head of 64 per 64 channels) with a 0/1 mask [F, F]."""
    F, S, C = q.shape
    H = C // 64
    with np.errstate(divide="ignore"):
        mask = torch.from_numpy(np.log(allowed.astype(np.float64)))

    def heads(a):
        return torch.from_numpy(widen(a).astype(np.float64)).reshape(F, S, H, 64).permute(1, 2, 0, 3)

    o = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v), attn_mask=mask, scale=0.125)
    return o.permute(2, 0, 1, 3).reshape(F, S, C).numpy()


@pytest.mark.parametrize("F", [1, 5, 16, 17, 40])
def test_dda_local_only_is_sliding_window_attention(F):
    S, C = 2, 128
    q, k, v = (randn((F, S, C), 190 + i, synth.BF16) for i in range(3))
    allowed = np.zeros((F, F))
    for t in range(F):
        allowed[t, local_frames(F, t)] = 1
    o = oracle.dda(q, k, v, n_global=0)
    assert np.abs(o - sdpa_masked(q, k, v, allowed)).max() < 1e-12


@pytest.mark.parametrize("F", [1, 5, 16, 40])
def test_dda_global_only_attends_the_sampled_frames(F):
    # Every query sees the same 16 rows (with repeats when F < 16), so the
    # key multiplicity enters as log(count) in the mask.
    S, C = 2, 64
    q, k, v = (randn((F, S, C), 200 + i) for i in range(3))
    counts = np.bincount(global_frames(F), minlength=F).astype(np.float64)
    allowed = np.broadcast_to(counts, (F, F))
    o = oracle.dda(q, k, v, n_local=0)
    assert np.abs(o - sdpa_masked(q, k, v, allowed)).max() < 1e-12


# ------------------------------------------------- GroupNorm, clip form

def test_gn_clip_sums_brute_force_and_closed_form():
    F, S, C, G = 7, 5, 48, 6
    x = randn((F, S, C), 210, synth.BF16)
    xf = widen(x).astype(np.float64).reshape(F * S, G, C // G)
    s1 = oracle.gn_clip_sums(x, G)
    assert np.allclose(s1, xf.sum(axis=(0, 2)), rtol=1e-13, atol=1e-12)
    mean = np.linspace(-0.5, 0.5, G)
    s2 = oracle.gn_clip_sums(x, G, mean)
    assert np.allclose(s2, ((xf - mean[None, :, None]) ** 2).sum(axis=(0, 2)), rtol=1e-13, atol=0)
    c = np.full((F, S, C), 1.5, np.float32)
    n = F * S * C // G
    assert np.array_equal(oracle.gn_clip_sums(c, G), np.full(G, 1.5 * n))
    assert np.array_equal(oracle.gn_clip_sums(c, G, np.full(G, 1.5)), np.zeros(G))


def test_gn_clip_sums_aggregate_to_whole_video_stats():
    # Sum of the clips' first sums / N_g = the global mean; sum of the clips'
    # second sums (about that global mean) / N_g = the global variance.
    F, S, C, G = 23, 4, 64, 8
    x = synth.normal(F * S * C, 211, synth.BF16, 1.0, S * C, 0.3).reshape(F, S, C)  # drift 0.3 per frame
    mean, var, _ = oracle.gn_stats(x, G)
    n = F * S * C // G
    clips = [(0, 5), (5, 17), (17, 23)]
    s1 = sum(oracle.gn_clip_sums(x[a:b], G) for a, b in clips)
    assert np.abs(s1 / n - mean).max() < 1e-15
    s2 = sum(oracle.gn_clip_sums(x[a:b], G, mean) for a, b in clips)
    assert np.abs(s2 / n - var).max() < 1e-14
    # a clip's own mean is not the global one (frames 0..4 sit below it)
    m0 = oracle.gn_clip_sums(x[0:5], G) / (5 * S * C // G)
    assert np.all(m0 < mean)


# ------------------------------------------------ float64 (exact) inputs

def test_float64_inputs_match_the_narrow_types():
    # A float64 array holding the same values as a float32 or bf16 one gives
    # identical results: the type only changes how values are read.
    F, S, C, G = 19, 3, 64, 8
    for dt in (synth.F32, synth.BF16):
        x = randn((F, S, C), 220 + dt, dt)
        x64 = widen(x).astype(np.float64)
        w = randn((3, C, C), 222 + dt, dt, 0.1)
        w64 = widen(w).astype(np.float64)
        assert np.array_equal(oracle.conv3(x64, w64), oracle.conv3(x, w))
        assert np.array_equal(oracle.dda(x64, x64, x64), oracle.dda(x, x, x))
        for a, b in zip(oracle.gn_stats(x64, G), oracle.gn_stats(x, G)):
            assert np.array_equal(a, b)


def test_conv_of_exact_groupnorm_brute_force():
    # The reference of a conv that consumes an unrounded GroupNorm output:
    # the oracle's conv over float64 input against a numpy sum of three
    # shifted matrix products.
    F, S, C, G = 11, 4, 32, 4
    x = randn((F, S, C), 230, synth.BF16)
    gn, _, _ = oracle.groupnorm(x, G)                 # float64 [F, S, C]
    w = randn((3, C, C), 231, synth.BF16, 0.2)
    wf = widen(w).astype(np.float64)
    pad = np.zeros((F + 2, S, C))
    pad[1:-1] = gn
    ref = sum(pad[k:k + F] @ wf[k].T for k in range(3))
    assert np.abs(oracle.conv3(gn, wf) - ref).max() < 1e-12


def test_chain_without_groupnorm_rounding_composes_the_modules():
    # The fused reading: the conv reads the exact GroupNorm output, only the
    # conv output is rounded before the attention.
    import math
    F, S, C, G = 20, 6, 128, 8
    x = randn((F, S, C), 240, synth.BF16)
    w = randn((3, C, C), 241, synth.BF16, 1 / math.sqrt(3 * C))
    out, gn, cv, mean, rstd = oracle.chain(x, w, G, intermediates=True, round_gn=False)
    y, m2, r2 = oracle.groupnorm(x, G)
    assert np.array_equal(gn, y) and np.array_equal(mean, m2) and np.array_equal(rstd, r2)
    cx = oracle.conv3(y, widen(w).astype(np.float64))
    cv_ref = np.vectorize(lambda a: oracle.round_to(a, synth.BF16))(cx)
    assert np.array_equal(cv, cv_ref)
    cb = (cv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(out, oracle.dda(cb, cb, cb))
    # the rounded reading differs from it only through the GroupNorm rounding
    out_r, gn_r, _, _, _ = oracle.chain(x, w, G, intermediates=True)
    assert not np.array_equal(gn_r, gn) and np.abs(gn_r - gn).max() <= 2.0 ** -8 * np.abs(gn).max()


# ------------------------------------- reuse of attention outputs across steps

def test_broadcast_schedule_hand_tables():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "broadcast_schedule.json")))
    for c in g["cases"]:
        got = oracle.broadcast_schedule(c["n_steps"], c["range"])
        assert list(np.nonzero(got)[0]) == c["compute"], c


def broadcast_by_walking(n, r):
    """Independent construction from the prose: walk the steps, broadcasting a
    computed output to the next r - 1 steps while inside the stable middle."""
    edge = n * 15 // 100
    out, since = [], None
    for i in range(n):
        if i < edge or i >= n - edge:
            out.append(1)
            since = None
            continue
        if since is None or since == r - 1:
            out.append(1)
            since = 0
        else:
            out.append(0)
            since += 1
    return out


def test_broadcast_schedule_brute_force_and_counts():
    for n in list(range(1, 60)) + [100, 250]:
        edge = n * 15 // 100
        for r in (1, 2, 3, 4, 5, 7, 60):
            got = oracle.broadcast_schedule(n, r)
            assert list(got) == broadcast_by_walking(n, r), (n, r)
            # every edge step computes; the middle computes ceil(middle / r) times
            assert got[:edge].all() and got[n - edge:].all()
            assert int(got.sum()) == 2 * edge + -(-(n - 2 * edge) // r)
    assert oracle.broadcast_schedule(30, 1).all()
    with pytest.raises(ValueError):
        oracle.broadcast_schedule(0, 2)
    with pytest.raises(ValueError):
        oracle.broadcast_schedule(10, 0)
