"""The per-element error terms of the ulp-level accuracy tests, pinned on the CPU.

tests/test_ulp_gpu.py asserts |kernel - exact| <= half a bf16 ulp (the output
rounding) + a term derived from each kernel's arithmetic (helpers.py).  Here
each term is checked against a simulation of that arithmetic in float64 (the
rounding steps the term accounts for, done exactly), and shown to be tight
enough that a kernel with a coarser step would fail it.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (U_BF16, attention_terms, conv_terms, groupnorm_terms, key_frames, ulp_bf16)


def widen(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def round_bits(x: np.ndarray, keep: int) -> np.ndarray:
    """Round float64 values to `keep` significand bits, nearest even (keep=8: bf16)."""
    m, e = np.frexp(x)
    scale = 2.0 ** keep
    return np.ldexp(np.round(m * scale) / scale, e)


def within(got, ref, term):
    half = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    return np.abs(got - ref) <= half + term


def simulated_attention(q, k, v, keep, scale=0.125):
    """Softmax weights rounded to `keep` bits and normalised by their own sum,
    output rounded to bf16 (the attention kernel's rounding steps)."""
    F, n, C = q.shape
    H = C // 64
    qh, kh, vh = (a.reshape(F, n, H, 64) for a in (q, k, v))
    out = np.empty_like(qh)
    for t in range(F):
        J = np.array(key_frames(t, F))
        s = scale * np.einsum("nhd,jnhd->jnh", qh[t], kh[J])
        w = round_bits(np.exp(s - s.max(axis=0, keepdims=True)), keep)
        out[t] = np.einsum("jnh,jnhd->nhd", w, vh[J]) / w.sum(axis=0)[..., None]
    return round_bits(out.reshape(F, n, C), 8)


@pytest.mark.parametrize("F,n,C,sc", [(40, 3, 128, 1.0), (17, 2, 64, 2.0), (300, 1, 192, 1.0)])
def test_attention_term(F, n, C, sc):
    q, k, v = (synth.normal(F * n * C, 700 + i + F, synth.BF16, sc).reshape(F, n, C) for i in range(3))
    o, term, smax = attention_terms(widen(q), widen(k), widen(v))
    assert smax < 1000
    assert np.abs(o - oracle.dda(q, k, v)).max() < 1e-10      # the exact output is the oracle's
    sim = simulated_attention(widen(q), widen(k), widen(v), keep=8)
    assert within(sim, o, term).all()                          # bf16 weights: inside the bound
    assert not within(sim, o, 0 * term).all()                  # ... and the term is needed
    coarse = simulated_attention(widen(q), widen(k), widen(v), keep=5)
    assert not within(coarse, o, term).all()                   # 5-bit weights would fail it


def test_conv_term():
    F, n, C = 24, 3, 96
    x = synth.normal(F * n * C, 801, synth.BF16, 1.0).reshape(F, n, C)
    w = synth.normal(3 * C * C, 802, synth.BF16, (1 / (3 * C)) ** 0.5).reshape(3, C, C)
    y = oracle.conv3(x, w)
    absum = oracle.conv3(x & np.uint16(0x7FFF), w & np.uint16(0x7FFF))
    term = conv_terms(absum, C)
    # fp32 accumulation of the 3C exact products in order, then bf16
    xf = np.concatenate([np.zeros((1, n, C)), widen(x), np.zeros((1, n, C))]).astype(np.float32)
    wf = widen(w).astype(np.float32)
    acc = np.zeros((F, n, C), np.float32)
    for kk in range(3):
        for ci in range(C):
            acc = acc + xf[kk:kk + F, :, ci:ci + 1] * wf[kk, :, ci][None, None, :]
    sim = round_bits(acc.astype(np.float64), 8)
    assert within(sim, y, term).all()
    # without the output rounding, the fp32 sum alone sits inside the term
    assert (np.abs(acc.astype(np.float64) - y) <= term).all()


def test_groupnorm_term():
    F, n, C, G = 30, 4, 64, 8
    x = widen(synth.normal(F * n * C, 901, synth.BF16, 1.5).reshape(F, n, C)) + 0.7
    xb = x.reshape(F * n, G, C // G)
    mean = xb.mean(axis=(0, 2))
    rstd = 1 / np.sqrt(xb.var(axis=(0, 2)) + 1e-5)
    y = (x - np.repeat(mean, C // G)) * np.repeat(rstd, C // G)
    # statistics off by the tolerated amounts, apply in fp32, output in bf16
    m_off = (mean + 1e-5).astype(np.float32).astype(np.float64)
    r_off = (rstd * (1 - 1e-5)).astype(np.float32).astype(np.float64)
    a = np.repeat(r_off, C // G).astype(np.float32)
    b = (-(np.repeat(m_off, C // G).astype(np.float32) * a)).astype(np.float32)
    yf = (x.astype(np.float32) * a + b).astype(np.float64)
    sim = round_bits(yf, 8)
    term = groupnorm_terms(x, mean, rstd, G)
    assert within(sim, y, term).all()
    # statistics off by ten times the tolerance leave it somewhere
    m_bad = (mean + 1e-3).astype(np.float32).astype(np.float64)
    yb = (x - np.repeat(m_bad, C // G)) * np.repeat(rstd, C // G)
    assert not within(round_bits(yb, 8), y, term).all()
