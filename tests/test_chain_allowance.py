"""The chain's end-to-end allowance, pinned on the CPU.

In the GroupNorm -> conv -> attention chain each module returns a bf16
tensor, so both the kernels (from fp32) and the oracle (from fp64) round the
conv output before the attention reads it.  Where the exact conv value lies
within the kernel's fp32 error of a rounding boundary, the two sides may pick
neighbouring bf16 values, and the attention carries that difference to the
end.  tests/helpers.flip_allowance bounds, per output element, how far the
attention can move when some of its input values move by one bf16 step.
Here that bound is checked against the oracle itself: attention over an input
with planted one-step changes stays within the bound of attention over the
original input, is unchanged wherever the bound is zero, and needs the
softmax term of the bound (the direct term alone is exceeded).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import flip_allowance, key_frames


def widen(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def step_bits(b: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Move bf16 bit patterns one representable value up (d=+1) or down (d=-1)."""
    b = b.astype(np.int64)
    key = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF) + d
    return np.where(key >= 0, key, 0x8000 | (-key)).astype(np.uint16)


@pytest.mark.parametrize("F,S,C,frac,scale_in", [
    (40, 6, 128, 0.01, 1.0),
    (24, 3, 64, 0.05, 2.5),     # larger values: one step moves the scores more
    (16, 4, 64, 0.002, 1.0),    # F = 16: every frame is a key of every query
    (300, 2, 64, 0.001, 1.0),
])
def test_flip_allowance_bounds_the_oracle(F, S, C, frac, scale_in):
    v = synth.normal(F * S * C, 9100 + F, synth.BF16, scale_in).reshape(F, S, C)
    rng = np.random.default_rng(F * 7 + C)
    mask = rng.random(v.shape) < frac
    d = np.where(rng.random(v.shape) < 0.5, -1, 1)
    vg = np.where(mask, step_bits(v, d), v)
    out = oracle.dda(v, v, v)
    out_g = oracle.dda(vg, vg, vg)
    allow = flip_allowance(out, widen(v), widen(vg))
    diff = np.abs(out_g - out)
    assert np.all(diff <= allow + 1e-12), float((diff - allow).max())
    assert np.all(diff[allow == 0] == 0)
    # With sparse changes (the chain's case: a few values of millions) the
    # bound stays within a modest factor of the worst change; dense changes of
    # large values make the softmax term's worst case loose.
    if frac <= 0.01:
        assert allow.max() <= 16 * diff.max() + 1e-9, (allow.max(), diff.max())
    # the softmax term is needed: the direct term alone is exceeded somewhere
    direct = np.zeros_like(out)
    dv = np.abs(widen(vg) - widen(v))
    for t in range(F):
        direct[t] = dv[sorted(set(key_frames(t, F)))].max(axis=0)
    assert (diff > direct + 1e-12).any()


def test_flip_allowance_is_zero_without_changes():
    F, S, C = 20, 3, 64
    v = synth.normal(F * S * C, 5, synth.BF16, 1.0).reshape(F, S, C)
    out = oracle.dda(v, v, v)
    assert not flip_allowance(out, widen(v), widen(v)).any()


def test_flip_allowance_reaches_only_the_queries_that_see_the_change():
    """One value changed in frame f, head 1: only queries whose key set holds
    frame f get a nonzero allowance, and only in head 1's channels."""
    F, S, C, f = 64, 2, 128, 40
    v = synth.normal(F * S * C, 6, synth.BF16, 1.0).reshape(F, S, C)
    vg = v.copy()
    vg[f, 1, 64 + 5] = step_bits(v[f, 1, 64 + 5:64 + 6], np.array([1]))[0]
    out = oracle.dda(v, v, v)
    allow = flip_allowance(out, widen(v), widen(vg))
    for t in range(F):
        sees = f in key_frames(t, F)
        assert bool(allow[t, 1, 64:].any()) == sees, t
        assert not allow[t, 1, :64].any() and not allow[t, 0].any()
