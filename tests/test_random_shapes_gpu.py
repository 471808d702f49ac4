"""Seeded random shapes, every output element against the oracle, on the GPU through the C ABI.

The hand-picked parity shapes cover the tile and work-item boundaries one at a
time; these draw frame counts (biased towards multiples of 16 and 256 plus or
minus one), location grids and channel counts together, so that ragged frame,
location and channel tiles, partial attention items and remainder packings
meet in the same call.  Each case checks GroupNorm, the conv (and, on inputs
1.5 times larger, the conv at the level of single ulps), the conv with
GroupNorm applied inside (bit for bit against apply + conv) and the
attention.  The oracle's conv cost bounds F*H*W*C^2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, check_stats, check_ulp, conv_terms, fetch, upload

pytestmark = pytest.mark.gpu

BF = synth.BF16
N_CASES = 10
CONV_BUDGET = 2.0e9   # F * H * W * C^2, about a second of oracle conv


def draw(i: int):
    rng = np.random.default_rng(4200 + i)
    C = int(rng.choice([64, 128, 192, 256, 320, 384, 640]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16, 32) if C % g == 0]))
    base = int(rng.choice([1, 16, 256, 512]))
    F = max(1, base + int(rng.integers(-3, 4)) if rng.random() < 0.6 else int(rng.integers(1, 700)))
    smax = max(1, int(CONV_BUDGET / (F * C * C)))
    H = int(rng.integers(1, 10))
    W = int(rng.integers(1, max(2, min(10, smax // H + 1))))
    while H * W > smax and H > 1:
        H -= 1
    return F, H, W, C, G


CASES = [draw(i) for i in range(N_CASES)]


def rnd(shape, seed, scale=1.0):
    return synth.normal(int(np.prod(shape)), seed, BF, scale).reshape(shape)


@pytest.mark.parametrize("case", range(N_CASES), ids=[f"F{c[0]}_{c[1]}x{c[2]}_C{c[3]}_G{c[4]}" for c in CASES])
def test_random_shape(case):
    F, H, W, C, G = CASES[case]
    announce(f"random shape {case}: F={F} {H}x{W} C={C} G={G}")
    seed = 9000 + 10 * case
    # unit-variance inputs and outputs: with |y| >= 8 the bf16 output's own
    # rounding (half an ulp, up to 2^-5) would exceed the 2e-2 bar
    x = rnd((F, H, W, C), seed)
    w = rnd((3, C, C), seed + 1, (1.0 / (3 * C)) ** 0.5)

    y, mean, rstd = vinf.groupnorm_global(upload(x), G)
    ref, rm, rr = oracle.groupnorm(x, G)
    check_stats(mean, rstd, rm, rr, "groupnorm stats")
    check(fetch(y), ref, BF, "groupnorm")

    xd, wd = upload(x), upload(w)
    c = vinf.temporal_conv3(xd, wd)
    check(fetch(c), oracle.conv3(x, w), BF, "conv3")

    # at 1.5x the input scale some outputs pass 8, where half a bf16 ulp is 2^-5:
    # per element, half an ulp plus the fp32 accumulation term
    x15 = rnd((F, H, W, C), seed + 4, 1.5)
    c15 = fetch(vinf.temporal_conv3(upload(x15), wd))
    ref15 = oracle.conv3(x15, w)
    absum = oracle.conv3(x15 & np.uint16(0x7FFF), w & np.uint16(0x7FFF))
    check_ulp(c15, ref15, conv_terms(absum.reshape(ref15.shape), C), "conv3 at 1.5x scale (ulp level)")

    # GroupNorm inside the conv equals the apply followed by the conv, bit for bit
    ws = torch.empty(vinf.temporal_conv3_gn_workspace_bytes(C, torch.bfloat16), dtype=torch.uint8, device=xd.device)
    fused = vinf.temporal_conv3_gn(xd, wd, mean, rstd, workspace=ws)
    assert np.array_equal(bits(fused), bits(vinf.temporal_conv3(y, wd))), "conv3 with GroupNorm inside"

    q, k, v = x, rnd((F, H, W, C), seed + 2), rnd((F, H, W, C), seed + 3, 0.7)
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v))
    check(fetch(o), oracle.dda(q, k, v), BF, "attention")


FP = synth.F32
N_FP = 3
FP_CASES = [draw(100 + i) for i in range(N_FP)]


@pytest.mark.parametrize("case", range(N_FP), ids=[f"F{c[0]}_{c[1]}x{c[2]}_C{c[3]}_G{c[4]}" for c in FP_CASES])
def test_random_shape_f32(case):
    """The float32 kernels on seeded shapes, every element within 1e-4."""
    F, H, W, C, G = FP_CASES[case]
    announce(f"random shape f32 {case}: F={F} {H}x{W} C={C} G={G}")
    seed = 9500 + 10 * case
    x = synth.normal(F * H * W * C, seed, FP).reshape(F, H, W, C)
    w = synth.normal(3 * C * C, seed + 1, FP, (1.0 / (3 * C)) ** 0.5).reshape(3, C, C)
    y, mean, rstd = vinf.groupnorm_global(upload(x), G)
    ref, rm, rr = oracle.groupnorm(x, G)
    check_stats(mean, rstd, rm, rr, "groupnorm stats")
    check(fetch(y), ref, FP, "groupnorm")
    xd, wd = upload(x), upload(w)
    check(fetch(vinf.temporal_conv3(xd, wd)), oracle.conv3(x, w), FP, "conv3")
    ws = torch.empty(vinf.temporal_conv3_gn_workspace_bytes(C, torch.float32), dtype=torch.uint8, device=xd.device)
    fused = vinf.temporal_conv3_gn(xd, wd, mean, rstd, workspace=ws)
    assert np.array_equal(bits(fused), bits(vinf.temporal_conv3(y, wd))), "conv3 with GroupNorm inside"
    q = x
    k, v = (synth.normal(F * H * W * C, seed + 2 + i, FP).reshape(F, H, W, C) for i in range(2))
    o = vinf.dual_domain_attn(upload(q), upload(k), upload(v))
    check(fetch(o), oracle.dda(q, k, v), FP, "attention")
