"""Accuracy of each bf16 kernel at the level of single ulps, on the GPU through the C ABI.

The parity bar (max-abs 2e-2) is loose next to bf16 resolution for small
outputs, so here every sampled output must lie within half a bf16 ulp (the
output rounding, which any correct bf16 result may carry) plus an error term
derived from the kernel's own arithmetic (helpers.attention_terms,
conv_terms, groupnorm_terms; pinned on the CPU in test_ulp_terms.py):

* attention: the softmax weights are rounded to bf16 and normalised by their
  own sum, so the output may move by (e^(2 eta) - 1) * sum_j pi_j |v_j - o|
  with eta = 2^-8 + 1e-4, plus fp32 sums;
* conv: fp32 accumulation of exact bf16 products, (3C + 2) 2^-24 sum |W||x|;
* GroupNorm: the apply in fp32 from statistics within the tolerances the
  statistics tests assert.

Inputs are the seeded workloads (sampled locations at full size) and small
ragged shapes (every output).
"""
import numpy as np
import pytest

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import (announce, attention_terms, check_stats, check_ulp, conv_terms, fetch, groupnorm_terms,
                     sample_locs, upload)

pytestmark = pytest.mark.gpu

BF = synth.BF16
CFG = synth.CONFIGS


def widen_locs(a: np.ndarray, locs) -> np.ndarray:
    """uint16 bf16 bits [F, H, W, C] -> float64 [F, n_locs, C]."""
    F = a.shape[0]
    C = a.shape[-1]
    a = a.reshape(F, -1, C)
    if locs is not None:
        a = a[:, locs]
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def attention_case(q, k, v, locs, what):
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v))
    got = fetch(o, locs)
    ref, term, smax = attention_terms(widen_locs(q, locs), widen_locs(k, locs), widen_locs(v, locs))
    assert smax < 1000, smax   # the premise of the score-error allowance
    check_ulp(got, ref, term, what)


def conv_case(x, w, locs, what):
    C = x.shape[-1]
    y = vinf.temporal_conv3(upload(x), upload(w))
    got = fetch(y, locs)
    ref = oracle.conv3(x, w, locs=locs)
    absum = oracle.conv3(x & np.uint16(0x7FFF), w & np.uint16(0x7FFF), locs=locs)
    check_ulp(got, ref, conv_terms(absum, C), what)


def groupnorm_case(x, G, locs, what):
    y, mean, rstd = vinf.groupnorm_global(upload(x), G)
    got = fetch(y, locs)
    ref, rm, rr = oracle.groupnorm(x, G, locs=locs)
    check_stats(mean, rstd, rm, rr, what + " stats")   # the premise of the apply term
    check_ulp(got, ref, groupnorm_terms(widen_locs(x, locs), rm, rr, G), what)


@pytest.mark.parametrize("cfgno", [2, 3, 4, 5, 6])
def test_workload_ulp(cfgno):
    c = CFG[cfgno]
    F, H, W, C, G = c["F"], c["H"], c["W"], c["C"], c["G"]
    locs = sample_locs(H * W, 8, seed=100 + cfgno)
    slope = c["slope"]
    announce(f"{c['name']}: ulp-level accuracy of groupnorm, conv3, attention")
    x = synth.make_tensor(cfgno, synth.X_GN, F, H, W, C, BF, slope)
    groupnorm_case(x, G, locs, "groupnorm")
    del x
    x = synth.make_tensor(cfgno, synth.X_CONV, F, H, W, C, BF, slope)
    conv_case(x, synth.make_conv_weight(cfgno, C, BF), locs, "conv3")
    del x
    if c["chain"]:   # the chain's attention reads one tensor as Q, K and V
        q = synth.make_tensor(cfgno, synth.Q, F, H, W, C, BF, slope)
        attention_case(q, q, q, locs, "attention (Q = K = V)")
    else:
        q, k, v = (synth.make_tensor(cfgno, t, F, H, W, C, BF, slope) for t in (synth.Q, synth.K, synth.V))
        attention_case(q, k, v, locs, "attention")


def rnd(shape, seed, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, BF, scale).reshape(shape)


@pytest.mark.parametrize("F,H,W,C", [(5, 3, 2, 128), (17, 3, 3, 64), (40, 2, 5, 192), (300, 2, 2, 320),
                                     (513, 1, 3, 128)])
def test_attention_small_ulp(F, H, W, C):
    announce(f"attention ulp F={F} {H}x{W} C={C}")
    q, k, v = (rnd((F, H, W, C), 5000 + 10 * i + F, 1.0 + 0.5 * i) for i in range(3))
    attention_case(q, k, v, None, "attention")


@pytest.mark.parametrize("F,H,W,C", [(37, 5, 7, 320), (33, 4, 5, 256), (1, 3, 3, 64), (70, 16, 59, 32)])
def test_conv_small_ulp(F, H, W, C):
    announce(f"conv3 ulp F={F} {H}x{W} C={C}")
    x = rnd((F, H, W, C), 6000 + F)
    w = rnd((3, C, C), 6001 + C, (1.0 / (3 * C)) ** 0.5)
    conv_case(x, w, None, "conv3")


@pytest.mark.parametrize("F,H,W,C,G", [(37, 7, 9, 320, 32), (9, 4, 4, 2048, 16), (3, 1, 1, 1280, 32)])
def test_groupnorm_small_ulp(F, H, W, C, G):
    announce(f"groupnorm ulp F={F} {H}x{W} C={C} G={G}")
    x = rnd((F, H, W, C), 7000 + F, 2.0)
    groupnorm_case(x, G, None, "groupnorm")
