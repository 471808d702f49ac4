"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import torch

import synth

# Parity bars: bf16 I/O max-abs <= 2e-2 and mean-abs <= 2e-3; float32 I/O
# max-abs <= 1e-4 (hence mean-abs too).
TOL = {synth.BF16: (2e-2, 2e-3), synth.F32: (1e-4, 1e-4)}


def dev():
    return torch.device("cuda:0")


def upload(a: np.ndarray) -> torch.Tensor:
    """numpy float32 or uint16 bf16 bits -> device tensor of the same shape."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev())


def fetch(t: torch.Tensor, locs=None) -> np.ndarray:
    """Device [F,H,W,C] -> float64 numpy [F, n_locs, C] (all locations when locs is None)."""
    F, H, W, C = t.shape
    t = t.reshape(F, H * W, C)
    if locs is not None:
        t = t[:, torch.as_tensor(np.asarray(locs), device=t.device, dtype=torch.long)]
    return t.float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor (for bitwise comparisons)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def check(got: np.ndarray, ref: np.ndarray, dt: int, what: str):
    max_tol, mean_tol = TOL[dt]
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    print(f"  {what}: max-abs {mx:.3e} mean-abs {mn:.3e}", flush=True)
    assert mx <= max_tol and mn <= mean_tol, f"{what}: max-abs {mx:.3e} (<= {max_tol}), mean-abs {mn:.3e} (<= {mean_tol})"
    return mx, mn


def check_stats(mean_gpu, rstd_gpu, mean_ref, rstd_ref, what):
    mg = mean_gpu.cpu().numpy().astype(np.float64)
    rg = rstd_gpu.cpu().numpy().astype(np.float64)
    dm = np.abs(mg - mean_ref).max()
    dr = (np.abs(rg - rstd_ref) / rstd_ref).max()
    print(f"  {what}: |d mean| {dm:.2e}  |d rstd|/rstd {dr:.2e}", flush=True)
    assert dm <= 1e-5 and dr <= 1e-5, (what, dm, dr)


def sample_locs(S: int, n: int = 8, seed: int = 0) -> np.ndarray:
    """n spatial locations: the first, the last and n-2 seeded others."""
    if S <= n:
        return np.arange(S, dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, S - 1), size=n - 2, replace=False)
    return np.array(sorted({0, S - 1, *(int(m) for m in mid)}), dtype=np.int64)


def announce(msg: str):
    print(msg, flush=True)
