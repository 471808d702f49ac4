"""Attention at the largest frame that its whole-strip stage addresses with 32-bit offsets, and one location past it.

A whole-strip work item stages its K and V rows through buffer loads whose
byte offsets count from the item's first frame in 32 bits, as long as 290
frame strides stay below 4 GiB (H*W*C <= 7,405,116 elements); larger frames
take 64-bit addresses.  Both shapes here have 160 frames, one head (C = 64)
and one item per location, so the last rows of an item sit more than 2^31
bytes past its first: offsets that a signed reading would get wrong.  The
locations repeat 97 seeded patterns (the data generation stays cheap); the
output is compared with the oracle at sampled locations, the last one
included.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, check, fetch, sample_locs, upload

pytestmark = pytest.mark.gpu

BF = synth.BF16
F, C, P = 160, 64, 97


def tiled(S: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """[F, S, C] bf16 bits: location s holds seeded pattern s % P."""
    pat = synth.normal(F * P * C, seed, BF, scale).reshape(F, P, C)
    return np.ascontiguousarray(np.tile(pat, (1, (S + P - 1) // P, 1))[:, :S])


@pytest.mark.parametrize("H,W", [(72, 1607), (2, 57853)], ids=["32-bit offsets, S*C=7405056", "64-bit, S*C=7405184"])
def test_attention_wide_frames(H, W):
    S = H * W
    announce(f"wide frame attention: F={F} {H}x{W} C={C} (S*C={S * C})")
    q, k, v = (tiled(S, 7100 + i, 0.7 if i == 2 else 1.0).reshape(F, H, W, C) for i in range(3))
    qd, kd, vd = upload(q), upload(k), upload(v)
    o = vinf.dual_domain_attn(qd, kd, vd)
    locs = sample_locs(S, 8, seed=S)
    got = fetch(o, locs)
    del qd, kd, vd, o
    torch.cuda.empty_cache()
    check(got, oracle.dda(q, k, v, locs=locs), BF, "attention at sampled locations")
