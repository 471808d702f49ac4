"""Pins of the oracle's Q/K/V projection and of projection -> attention (CPU only).

The projection is fixed to a hand-worked token (tests/golden/qkv_tiny.json),
to closed forms (identity, bias only, a channel permutation that is not its
own transpose, distinct maps per output) and to numpy's matmul in fp64.  The
composition with the attention is fixed to the oracle's attention through
weights whose effect on the attention has a closed form: identity maps,
a power-of-two query scale (the attention's score scale), a permuted value map
(a permutation of the output), and zero keys (the mean of the values over the
key multiset, from an independent key construction).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def randn(shape, seed, dtype=synth.F32, scale=1.0):
    n = int(np.prod(shape))
    return synth.normal(n, seed, dtype, scale).reshape(shape)


def widen(a):
    return (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def as_dt(a64, dt):
    """float64 values exact in dt -> an array of dt."""
    a = np.asarray(a64, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16) if dt == synth.BF16 else a


def cyclic_within_heads(C, shift=1, dh=64):
    """Permutation matrix P with (P x)[c] = x[head(c) + (c + shift) % dh]: a
    channel permutation inside each head, not its own transpose."""
    P = np.zeros((C, C))
    for c in range(C):
        h = c - c % dh
        P[c, h + (c % dh + shift) % dh] = 1.0
    return P


def test_golden_tiny_token():
    g = json.load(open(os.path.join(GOLD, "qkv_tiny.json")))
    x = np.array(g["x"], dtype=np.float32).reshape(1, 1, 1, 2)
    w = np.array(g["w"], dtype=np.float32)
    out = oracle.qkv_project(x, w, np.array(g["bias"]))
    assert np.array_equal(out.reshape(3, 2), np.array(g["qkv"], dtype=np.float64))


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16])
def test_identity_maps_give_the_tokens(dt):
    F, H, W, C = 7, 2, 3, 128
    x = randn((F, H, W, C), 500, dt)
    w = as_dt(np.stack([np.eye(C)] * 3), dt)
    out = oracle.qkv_project(x, w)
    for p in range(3):
        assert np.array_equal(out[p], widen(x).reshape(F, H * W, C))


def test_bias_only():
    F, S, C = 3, 4, 64
    x = randn((F, S, C), 501)
    bias = np.arange(3 * C, dtype=np.float64).reshape(3, C) / 7.0
    out = oracle.qkv_project(x, np.zeros((3, C, C), np.float32), bias)
    for p in range(3):
        assert np.array_equal(out[p], np.broadcast_to(bias[p], (F, S, C)))


def test_each_output_has_its_own_map_and_orientation():
    # Q = x, K = 2x, V = P x with P a permutation that differs from its
    # transpose: a transposed weight operand or a swapped output index fails.
    F, S, C = 5, 3, 128
    x = randn((F, S, C), 502)
    P = cyclic_within_heads(C, 3)
    assert not np.array_equal(P, P.T)
    w = np.stack([np.eye(C), 2 * np.eye(C), P]).astype(np.float32)
    out = oracle.qkv_project(x, w)
    x64 = widen(x)
    assert np.array_equal(out[0], x64)
    assert np.array_equal(out[1], 2 * x64)
    assert np.array_equal(out[2], x64 @ P.T)
    assert np.array_equal(out[2][..., 0], x64[..., 3])


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16])
def test_random_maps_vs_numpy(dt):
    F, H, W, C = 9, 3, 5, 192
    x = randn((F, H, W, C), 503, dt)
    w = randn((3, C, C), 504, dt, (1.0 / C) ** 0.5)
    bias = randn((3, C), 505) .astype(np.float64)
    locs = [0, 4, 14]
    out = oracle.qkv_project(x, w, bias, locs=locs)
    xs = widen(x).reshape(F, H * W, C)[:, locs]
    ref = np.stack([xs @ widen(w)[p].T + bias[p] for p in range(3)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------- projection -> attention

@pytest.mark.parametrize("dt", [synth.F32, synth.BF16])
def test_identity_maps_give_self_attention(dt):
    F, H, W, C = 40, 2, 2, 128
    x = randn((F, H, W, C), 510, dt)
    w = as_dt(np.stack([np.eye(C)] * 3), dt)
    o, qkv = oracle.qkv_dda(x, w, intermediates=True)
    assert np.array_equal(o, oracle.dda(x, x, x))
    for p in range(3):
        assert np.array_equal(qkv[p], widen(x).reshape(F, H * W, C))


def test_query_scale_is_the_score_scale():
    # Q = 2x (exact in bf16): the scores double, as with scale 2/sqrt(64).
    # K = 2x does the same, V = 2x instead doubles the output.
    F, S, C = 33, 3, 128
    x = randn((F, S, C), 511, synth.BF16)
    I = np.eye(C)
    ref = oracle.dda(x, x, x, scale=2.0 / 8.0)
    assert np.array_equal(oracle.qkv_dda(x, as_dt(np.stack([2 * I, I, I]), synth.BF16)), ref)
    assert np.array_equal(oracle.qkv_dda(x, as_dt(np.stack([I, 2 * I, I]), synth.BF16)), ref)
    assert np.array_equal(oracle.qkv_dda(x, as_dt(np.stack([I, I, 2 * I]), synth.BF16)), 2 * oracle.dda(x, x, x))
    assert not np.allclose(ref, oracle.dda(x, x, x), atol=1e-3)


def test_value_map_permutes_the_output():
    F, S, C = 24, 2, 128
    x = randn((F, S, C), 512)
    P = cyclic_within_heads(C, 5)
    o = oracle.qkv_dda(x, np.stack([np.eye(C), np.eye(C), P]).astype(np.float32))
    np.testing.assert_allclose(o, oracle.dda(x, x, x) @ P.T, rtol=0, atol=1e-12)


def test_zero_keys_average_the_values():
    # K = 0: every score is 0, so the output is the mean of V over the key
    # multiset (local window + uniform global frames, built here from the
    # reading, not from the oracle).
    F, S, C = 37, 2, 64
    x = randn((F, S, C), 513)
    wv = randn((C, C), 514, synth.F32, 0.125)
    w = np.stack([np.eye(C, dtype=np.float32), np.zeros((C, C), np.float32), wv])
    o = oracle.qkv_dda(x, w)
    v = np.vectorize(lambda a: oracle.round_to(a, synth.F32))(widen(x) @ widen(wv).T)
    for t in (0, 8, 20, 36):
        st = min(max(t - 8, 0), F - 16)
        keys = list(range(st, st + 16)) + [i * F // 16 for i in range(16)]
        np.testing.assert_allclose(o[t], v[keys].mean(axis=0), rtol=0, atol=1e-12)


def test_attention_reads_rounded_projections():
    F, S, C = 20, 2, 64
    x = randn((F, S, C), 515, synth.BF16)
    w = randn((3, C, C), 516, synth.BF16, 0.125)
    o, qkv = oracle.qkv_dda(x, w, intermediates=True)
    exact = oracle.qkv_project(x, w)
    for p in range(3):
        r = np.vectorize(lambda a: oracle.round_to(a, synth.BF16))(exact[p])
        assert np.array_equal(qkv[p], r)
        assert np.array_equal(widen(as_dt(r, synth.BF16)), r)  # each value is a bf16 value
    q, k, v = (as_dt(qkv[p], synth.BF16) for p in range(3))
    assert np.array_equal(o, oracle.dda(q, k, v))
