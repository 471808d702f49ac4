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


def key_frames(t: int, F: int, n_local: int = 16, n_global: int = 16) -> list:
    """Key frames of query frame t: the local window [st, st + min(16, F)),
    st = clamp(t - 8, 0, max(F - 16, 0)), then the global frames
    floor(i * F / 16) (Video-Infinity, dual-domain attention paragraph, as read
    for this library)."""
    nl = min(n_local, F)
    st = min(max(t - n_local // 2, 0), max(F - n_local, 0))
    loc = list(range(st, st + nl)) if n_local else []
    return loc + [(i * F) // n_global for i in range(n_global)]


def flip_allowance(out: np.ndarray, v_ref: np.ndarray, v_got: np.ndarray, scale: float = 0.125,
                   head_dim: int = 64) -> np.ndarray:
    """Per-element bound on how far attention over v_got (Q = K = V) may lie
    from attention over v_ref, the exact output `out` over v_ref being known.

    v_ref and v_got are [F, n, C] (the attention's input at n locations) and
    differ only where the two sides rounded an intermediate to different
    neighbouring bf16 values.  For an output o[t, s, c] of head h with key
    frames J(t), writing p, p' for the softmax weights over v_ref, v_got:
        o' - o = sum_j p'_j (v'_j[c] - v_j[c]) + sum_j (p'_j - p_j)(v_j[c] - o[c])
    The first sum is at most A = max_j |v'_j[c] - v_j[c]|.  Every score moves by
    at most M = max_j |s'_j - s_j| (s_j = scale * q_t . k_j over the head), so
    p'_j / p_j lies in [e^-2M, e^2M] and the second sum is at most
    B = (e^2M - 1) * max_j |v_j[c] - o[c]|.  Returns A + B (zero wherever no key
    row of the head changed)."""
    F, n, C = v_ref.shape
    heads = C // head_dim
    d = v_got - v_ref
    allow = np.zeros_like(out)
    changed = np.abs(d).reshape(F, n, heads, head_dim).max(axis=3) > 0   # [F, n, heads]
    for t in range(F):
        J = np.array(sorted(set(key_frames(t, F))))
        if not changed[J].any():
            continue
        A = np.abs(d[J]).max(axis=0)                                      # [n, C]
        qr = v_ref[t].reshape(n, heads, head_dim)
        qg = v_got[t].reshape(n, heads, head_dim)
        kr = v_ref[J].reshape(len(J), n, heads, head_dim)
        kg = v_got[J].reshape(len(J), n, heads, head_dim)
        ds = scale * np.abs((qg[None] * kg).sum(-1) - (qr[None] * kr).sum(-1))   # [J, n, heads]
        M = np.repeat(ds.max(axis=0), head_dim, axis=1)                   # [n, C]
        V = np.abs(v_ref[J] - out[t][None]).max(axis=0)                   # [n, C]
        allow[t] = A + np.expm1(2 * M) * V
    return allow


def check_end_to_end(got, out, o_on_gpu_conv, cv_r, cs, dt, what):
    """The chain's output against the oracle chain's.  Mean-abs within the
    bar everywhere.  Max-abs within the bar wherever every key row of the
    head holds the same conv values on both sides; elsewhere within the bar
    plus the bound (tests/helpers.flip_allowance) on how far the attention
    moves when conv values are one bf16 step apart -- the case where both
    roundings are correct.  The bound is checked on the oracle too."""
    max_tol, mean_tol = TOL[dt]
    allow = flip_allowance(out, cv_r, cs)
    moved = np.abs(o_on_gpu_conv - out)
    assert np.all(moved <= allow + 1e-9), f"{what}: the oracle moves beyond the bound ({(moved - allow).max():.3e})"
    err = np.abs(got - out)
    same = allow == 0
    rest = float(err[same].max()) if same.any() else 0.0
    announce(f"  {what} end to end: max-abs {err.max():.3e} mean-abs {err.mean():.3e}; "
             f"{int((~same).sum())} of {err.size} outputs see a conv value rounded the other way "
             f"(max-abs {err[~same].max() if (~same).any() else 0:.3e}, largest allowance "
             f"{max_tol + allow.max():.3e}); the rest max-abs {rest:.3e}")
    assert err.mean() <= mean_tol, f"{what}: end-to-end mean-abs {err.mean():.3e} (<= {mean_tol})"
    assert rest <= max_tol, f"{what}: end-to-end max-abs {rest:.3e} (<= {max_tol})"
    assert np.all(err <= max_tol + allow), f"{what}: end-to-end beyond the allowance ({(err - max_tol - allow).max():.3e})"


U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand, round to nearest even)
U_F32 = 2.0 ** -24


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    """The spacing of bf16 values at |a| (2^(e-7) for |a| in [2^e, 2^(e+1)))."""
    m, e = np.frexp(np.abs(a))   # |a| = m * 2^e, m in [0.5, 1)
    return np.where(a == 0, 0.0, np.ldexp(1.0, e - 8))


def check_ulp(got: np.ndarray, ref: np.ndarray, err_term: np.ndarray, what: str):
    """Per element |got - ref| <= half a bf16 ulp (the output rounding) plus
    the kernel's own error term."""
    half = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    err = np.abs(got - ref)
    slack = err - (half + err_term)
    within_half = float(np.mean(err <= half))
    print(f"  {what}: max |err| / (half-ulp + term) = {float((err / (half + err_term + 1e-300)).max()):.3f}; "
          f"{within_half:.4f} of outputs within half an ulp alone; largest term {float(err_term.max()):.2e}",
          flush=True)
    assert np.all(slack <= 0), (f"{what}: {int((slack > 0).sum())} outputs beyond half an ulp + the kernel term "
                                f"(worst excess {float(slack.max()):.3e})")


def attention_terms(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float = 0.125, head_dim: int = 64,
                    eps_w: float = 1e-4):
    """For attention over [F, n, C] float64 q, k, v (Q/K/V at n locations): the
    exact output o and the per-element error term of a kernel that rounds each
    softmax weight to bf16 and normalises by the sum of the rounded weights.

    Each rounded weight is p_j e^(eta_j) with |eta_j| <= U_BF16 + eps_w (eps_w
    covers the fp32 scores and exp2), so the normalised weights move by a
    factor within e^(+-2 eta) and the output by at most
        (e^(2 eta) - 1) * sum_j pi_j |v_j - o|        (pi: exact weights)
    plus the fp32 sums of 34 products and 17 weights and the final
    normalisation, at most 64 U_F32 (max_j |v_j| + |o|).  Also returns the
    largest score magnitude sum_d |q_d k_d| over the sample (eps_w holds while
    it stays below 1000)."""
    F, n, C = q.shape
    H = C // head_dim
    qh = q.reshape(F, n, H, head_dim)
    kh = k.reshape(F, n, H, head_dim)
    vh = v.reshape(F, n, H, head_dim)
    o = np.empty_like(qh)
    term = np.empty_like(qh)
    smax = 0.0
    eta = U_BF16 + eps_w
    for t in range(F):
        J = np.array(key_frames(t, F))                                     # 32 keys, repeats kept
        s = scale * np.einsum("nhd,jnhd->jnh", qh[t], kh[J])
        smax = max(smax, float(np.einsum("nhd,jnhd->jnh", np.abs(qh[t]), np.abs(kh[J])).max()))
        p = np.exp(s - s.max(axis=0, keepdims=True))
        pi = p / p.sum(axis=0, keepdims=True)                              # [32, n, H]
        ot = np.einsum("jnh,jnhd->nhd", pi, vh[J])
        spread = np.einsum("jnh,jnhd->nhd", pi, np.abs(vh[J] - ot[None]))
        vmax = np.abs(vh[J]).max(axis=0)
        o[t] = ot
        term[t] = np.expm1(2 * eta) * spread + 64 * U_F32 * (vmax + np.abs(ot))
    return o.reshape(F, n, C), term.reshape(F, n, C), smax


def conv_terms(x_abs_conv: np.ndarray, C: int) -> np.ndarray:
    """Error term of a kernel-3 conv accumulated in fp32 from exact bf16
    products: at most 3C + 2 roundings along any summation path, each within
    U_F32 of a partial sum bounded by sum |W| |x| (x_abs_conv: that sum, the
    conv of |x| with |W|)."""
    return (3 * C + 2) * U_F32 * x_abs_conv


def groupnorm_terms(x: np.ndarray, mean: np.ndarray, rstd: np.ndarray, G: int, d_mean: float = 1e-5,
                    d_rstd: float = 1e-5) -> np.ndarray:
    """Error term of y = fma(x, a, b) in fp32 with a = rstd_g and b = -mean_g a
    formed in fp32 from statistics within d_mean (absolute) and d_rstd
    (relative) of the exact ones (the stats tests assert those bounds):
        |x a + b - (x - mean) rstd| <= rstd (|x| (d_rstd + U) + d_mean + |mean| (d_rstd + 2U))
    plus the fma's own rounding, U |y|.  x: [F, n, C] float64; mean, rstd: [G]."""
    C = x.shape[-1]
    m = np.repeat(mean, C // G)
    r = np.repeat(rstd, C // G)
    y = (x - m) * r
    return r * (np.abs(x) * (d_rstd + U_F32) + d_mean + np.abs(m) * (d_rstd + 2 * U_F32)) + U_F32 * np.abs(y)
