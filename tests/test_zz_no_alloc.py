"""The allocation-free GroupNorm entry point, through the C ABI, on the GPU.

vinf_groupnorm_global_noalloc takes no workspace: its partial sums live in a
static device array of the library.  Its results must equal those of
vinf_groupnorm_global with a caller workspace bit for bit, on two calls in a
row (the second with a smaller input, which reuses the array the first one
left behind).  The host-side rejections are in test_abi.py.
"""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_temporal_amd as vinf
from helpers import announce, bits, upload

pytestmark = pytest.mark.gpu


def run_both(F, H, W, C, G, dt, seed):
    L = vinf.load()
    x = upload(synth.normal(F * H * W * C, seed, dt, 1.5).reshape(F, H, W, C))
    code = vinf.VINF_BF16 if dt == synth.BF16 else vinf.VINF_F32
    gamma = torch.linspace(0.5, 1.5, C, device=x.device)
    beta = torch.linspace(-0.25, 0.25, C, device=x.device)
    outs = []
    for noalloc in (False, True):
        y = torch.empty_like(x)
        mean = torch.empty(G, device=x.device)
        rstd = torch.empty(G, device=x.device)
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = L.vinf_groupnorm_global_noalloc(x.data_ptr(), y.data_ptr(), gamma.data_ptr(), beta.data_ptr(),
                                                 mean.data_ptr(), rstd.data_ptr(), F, H, W, C, G, 1e-5, code, stream)
        else:
            need = L.vinf_groupnorm_workspace_bytes(F, H, W, C, G, code)
            ws = torch.empty(need, device=x.device, dtype=torch.uint8)
            st = L.vinf_groupnorm_global(x.data_ptr(), y.data_ptr(), gamma.data_ptr(), beta.data_ptr(),
                                         mean.data_ptr(), rstd.data_ptr(), F, H, W, C, G, 1e-5, code, ws.data_ptr(),
                                         need, stream)
        assert st == 0, L.vinf_last_error().decode()
        torch.cuda.synchronize()
        outs.append((bits(y), bits(mean), bits(rstd)))
    for a, b, what in zip(outs[0], outs[1], ("y", "mean", "rstd")):
        assert np.array_equal(a, b), f"noalloc {what} differs from the workspace call"


def test_noalloc_equals_workspace_call_twice():
    announce("groupnorm noalloc: F=96 64x40 C=320 bf16, then F=9 5x7 C=64 fp32")
    run_both(96, 64, 40, 320, 32, synth.BF16, 11)   # 2048 partial blocks
    run_both(9, 5, 7, 64, 8, synth.F32, 12)          # fewer blocks than the first call left
    run_both(3, 2, 2, 1280, 32, synth.BF16, 13)      # wide rows, few blocks
