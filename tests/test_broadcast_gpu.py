"""Reuse of temporal-attention outputs across diffusion steps, on the GPU.

Over a 10-step schedule with range 3, every computing step must give the
attention of that step's inputs (bit for bit the plain call, and the oracle at
the bar), and every reuse step must leave the latest computed output in place.
"""
import numpy as np
import pytest

import oracle
import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, check, fetch, upload

pytestmark = pytest.mark.gpu


def test_broadcast_steps():
    F, H, W, C = 40, 2, 3, 128
    n, r = 10, 3
    sched = vinf.attn_broadcast_schedule(n, r)
    assert sched == [1, 1, 0, 0, 1, 0, 0, 1, 0, 1]
    announce(f"attention broadcast over {n} steps, range {r}: {sched}")
    out = upload(np.zeros((F, H, W, C), np.uint16))
    last = None
    for i in range(n):
        q, k, v = (synth.normal(F * H * W * C, 5000 + 3 * i + j, synth.BF16).reshape(F, H, W, C) for j in range(3))
        qd, kd, vd = upload(q), upload(k), upload(v)
        vinf.dual_domain_attn_broadcast(qd, kd, vd, out, i, sched)
        if sched[i]:
            assert np.array_equal(bits(out), bits(vinf.dual_domain_attn(qd, kd, vd))), i
            if i == 4:
                check(fetch(out), oracle.dda(q, k, v), synth.BF16, f"step {i}")
            last = bits(out)
        else:
            assert np.array_equal(bits(out), last), i
