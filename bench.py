"""Throughput of the Video-Infinity temporal module on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole temporal module over one synthetic latent:
GroupNorm with whole-video statistics -> kernel-3 temporal conv (zero pads at
the video ends) -> dual-domain attention with Q = K = V = the conv output, at
F=1024 frames, 64x40 locations, C=320 (5 heads of 64), bf16, 32 groups -- the
VideoCrafter2 latent shape at 512x320.  The GroupNorm normalisation is applied
inside the conv (statistics call + fused conv call, bit for bit the same
result), so the normalised tensor is never written; the chain that writes it
is timed too ("chain_unfused").  Inputs and every intermediate live in
HBM before the timed region starts; no allocation happens inside it.

Prints ONE JSON line: voxels/s (F*H*W per step), per-module times, the
roofline position of the dominant kernel (HIP events on the launch stream),
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
WORKLOAD = dict(name="m1024_chain_f1024_64x40x320_bf16", F=1024, H=64, W=40, C=320, G=32)
SEED_CONFIG = 6  # seeds of the F=1024 64x40x320 workload in synth.CONFIGS

# Which source file holds each kernel (for the traffic record's staleness check).
KERNEL_SOURCES = {
    "dda_bf16": "video_diffusion_temporal_amd/csrc/dual_domain_attn.hip",
    "conv3_bf16": "video_diffusion_temporal_amd/csrc/temporal_conv3.hip",
    "groupnorm": "video_diffusion_temporal_amd/csrc/groupnorm.hip",
}


def algorithmic_work(F, H, W, C, b=2):
    """Bytes / flops each module must move or compute (the method's own work)."""
    S = H * W
    vox = F * S
    return {
        # read q, k, v once, write o; plus the 16 global K and V rows per location
        "dda_bf16": dict(bound="hbm", bytes=vox * 4 * C * b + S * 32 * C * b, flops=vox * 128 * C),
        # 6 C^2 flops per voxel (3 taps x C_in x C_out x 2)
        "conv3_bf16": dict(bound="mfma", bytes=vox * 2 * C * b + 3 * C * C * b, flops=vox * 6 * C * C),
        # two statistic sweeps + apply: 3 reads and 1 write
        "groupnorm": dict(bound="hbm", bytes=vox * 4 * C * b, flops=vox * 8 * C),
        # the two statistic sweeps alone: 2 reads
        "groupnorm_stats": dict(bound="hbm", bytes=vox * 2 * C * b, flops=vox * 4 * C),
    }


def traffic_record(kernel):
    """HBM bytes per launch from profiles/traffic_<kernel>.json, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, KERNEL_SOURCES[kernel])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def host_threads():
    """Host threads this process may run on: its CPU affinity set, further
    limited by a cgroup CPU quota when one is set.  Returns (threads, detail)."""
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = nproc
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    threads = min(affinity, quota) if quota else affinity
    return threads, {"nproc": nproc, "affinity": affinity, "cgroup_quota_cpus": quota}


def cpu_baseline(F, C, G, side=16):
    """The oracle chain, as it stands, on F frames x side x side locations,
    over every host thread this process may use."""
    import numpy as np

    import oracle
    import synth

    H = W = side
    x = synth.make_tensor(SEED_CONFIG, synth.X_GN, F, H, W, C, synth.BF16)
    w = synth.make_conv_weight(SEED_CONFIG, C, synth.BF16)
    threads, detail = host_threads()
    t = time.perf_counter()
    oracle.chain(x, w, G, nthreads=threads)
    dt = time.perf_counter() - t
    vox = F * H * W
    return {"value": vox / dt, "unit": "voxels/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle chain (GroupNorm stats+apply, conv3, attention) in fp64 on F={F}, "
                      f"{H}x{W} locations, C={C}: {vox} voxels in {dt:.2f} s",
            "seconds": dt, "cpu_model": cpu_model(), "host": detail}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def percentiles(samples):
    """p10 / p50 / p90 (ms) of a list of per-step times."""
    import numpy as np

    a = np.asarray(samples, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def config3_calls(vinf, steps, stream):
    """Each call, and the step, at the per-level shape F=1024, 32x20 locations,
    C=640 (10 heads), bf16, 32 groups: timed alone, HIP events on the launch
    stream, seeded N(0,1) inputs."""
    import numpy as np
    import torch

    import synth

    F, H, W, C, G, cfg = 1024, 32, 20, 640, 32, 3
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    x = up(synth.make_tensor(cfg, synth.X_GN, F, H, W, C, synth.BF16))
    wt = up(synth.make_conv_weight(cfg, C, synth.BF16))
    q = up(synth.make_tensor(cfg, synth.Q, F, H, W, C, synth.BF16))
    k = up(synth.make_tensor(cfg, synth.K, F, H, W, C, synth.BF16))
    v = up(synth.make_tensor(cfg, synth.V, F, H, W, C, synth.BF16))
    y, o = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(G, device=dev)
    rstd = torch.empty(G, device=dev)
    ws = torch.empty(vinf.groupnorm_workspace_bytes(F, H, W, C, G, x.dtype), device=dev, dtype=torch.uint8)
    cws = torch.empty(vinf.temporal_conv3_gn_workspace_bytes(C, x.dtype), device=dev, dtype=torch.uint8)
    work = algorithmic_work(F, H, W, C)
    out = {"shape": f"F={F}, {H}x{W}, C={C}, bf16, groups={G}"}
    calls = [
        ("groupnorm", "hbm", lambda: vinf.groupnorm_global(x, G, out=y, mean_out=mean, rstd_out=rstd, workspace=ws,
                                                           stream=stream)),
        ("groupnorm_stats", "hbm", lambda: vinf.groupnorm_stats(x, G, mean_out=mean, rstd_out=rstd, workspace=ws,
                                                                stream=stream)),
        ("conv3_bf16", "mfma", lambda: vinf.temporal_conv3(x, wt, out=y, stream=stream)),
        ("conv3_gn_bf16", "mfma", lambda: vinf.temporal_conv3_gn(x, wt, mean, rstd, out=y, workspace=cws,
                                                                 stream=stream)),
        ("dda_bf16", "hbm", lambda: vinf.dual_domain_attn(q, k, v, out=o, stream=stream)),
    ]
    for name, bound, fn in calls:
        ms = timed(fn, steps, stream)
        wk = work["conv3_bf16" if name == "conv3_gn_bf16" else name]
        if bound == "hbm":
            gbs = wk["bytes"] / (ms * 1e-3) / 1e9
            out[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            tfl = wk["flops"] / (ms * 1e-3) / 1e12
            out[name] = {"ms": round(ms, 4), "TFLOP/s": round(tfl, 1),
                         "frac_mfma_bf16": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)}

    def step():
        vinf.groupnorm_stats(x, G, mean_out=mean, rstd_out=rstd, workspace=ws, stream=stream)
        vinf.temporal_conv3_gn(x, wt, mean, rstd, out=y, workspace=cws, stream=stream)
        vinf.dual_domain_attn(y, y, y, out=o, stream=stream)

    ms = timed(step, steps, stream)
    out["step"] = {"ms": round(ms, 4), "voxels_per_s": F * H * W / (ms * 1e-3),
                   "chain": "groupnorm_stats -> temporal_conv3_gn -> dual_domain_attn (Q = K = V)"}
    return out


def timed(fn, steps, stream, warm=2):
    """Average ms of fn() over `steps` calls (HIP events on the launch stream),
    after `warm` untimed calls."""
    import torch

    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def hbm_entry(ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes}


def next_rows(vinf, x, cv, G, stream, steps):
    """The clip-parallel forms and the attention ablations, each timed alone.

    Clip form: one of eight clips of a 2300-frame video (frames 864..1151,
    288 frames) at the same 64x40x320 bf16 locations, with its 8 + 7 context
    frames and the 16 gathered global rows, as one device of an 8-way clip
    split would run it.  Ablations: the local-only and global-only key sets at
    F=1024 on the chain's conv output (Q = K = V).  Projection: Q, K and V as
    three C x C maps of the conv output's tokens, and the attention over them,
    as two calls and as one fused call."""
    import numpy as np
    import torch

    import synth

    F, H, W, C = x.shape
    S, b = H * W, 2
    out = {}
    # attention of a clip, distinct Q/K/V (a device's projections are three tensors)
    F_total, f0, Fc = 2300, 864, 288
    pre, post = vinf.dda_clip_halo(F_total, f0, Fc)
    n_ext = pre + Fc + post
    q = cv[:Fc]
    k = x[:n_ext]
    v = torch.empty((n_ext, H, W, C), device=x.device, dtype=x.dtype)
    v.copy_(cv[F - n_ext:].flip(0))
    kg = torch.empty((16, H, W, C), device=x.device, dtype=x.dtype)
    vg = torch.empty_like(kg)
    kg.copy_(x[:16])
    vg.copy_(x[16:32])
    o = torch.empty_like(q)
    # The clip call is short and follows a pause (the buffers are filled above):
    # the clock takes some tens of launches to settle, hence the longer warm-up.
    ms = timed(lambda: vinf.dual_domain_attn_clip(q, k, v, F_total, f0, pre, post, kg, vg, out=o, stream=stream),
               steps, stream, warm=30)
    out["dda_bf16_clip"] = dict(hbm_entry(ms, S * C * b * (2 * Fc + 2 * n_ext + 32)),
                                shape=f"clip [{f0},{f0 + Fc}) of {F_total} frames, context {pre}+{post}, "
                                      f"{H}x{W}x{C}, distinct q/k/v, external global rows")
    del q, k, v, kg, vg, o
    # ablations on the chain's tensor (Q = K = V): the same bytes as the chain call less the global rows
    o = torch.empty_like(cv)
    for name, nl, ng, nbytes in (("dda_bf16_local_only", 16, 0, F * S * 4 * C * b),
                                 ("dda_bf16_global_only", 0, 16, F * S * 2 * C * b + S * 32 * C * b)):
        ms = timed(lambda: vinf.dual_domain_attn(cv, cv, cv, out=o, n_local=nl, n_global=ng, stream=stream), steps,
                   stream)
        out[name] = dict(hbm_entry(ms, nbytes), shape=f"F={F}, {H}x{W}x{C}, Q = K = V (n_local={nl}, n_global={ng})")
    del o
    # GroupNorm of one clip (288 frames): two sum sweeps and the apply
    xc = x[:Fc]
    yc = torch.empty_like(xc)
    ws = torch.empty(vinf.groupnorm_workspace_bytes(Fc, H, W, C, G, x.dtype), device=x.device, dtype=torch.uint8)
    s1 = torch.empty(G, device=x.device, dtype=torch.float64)
    s2 = torch.empty_like(s1)

    def gn_clip():
        vinf.groupnorm_clip_sums(xc, G, F_total, out=s1, workspace=ws, stream=stream)
        vinf.groupnorm_clip_sums(xc, G, F_total, s1, out=s2, workspace=ws, stream=stream)
        vinf.groupnorm_clip_apply(xc, G, F_total, s1, s2, out=yc, workspace=ws, stream=stream)

    ms = timed(gn_clip, steps, stream)
    out["groupnorm_clip"] = dict(hbm_entry(ms, Fc * S * 4 * C * b),
                                 shape=f"clip of {Fc} frames, {H}x{W}x{C}, groups={G} (sums, sums, apply)")
    # Q/K/V projection of the chain's conv output (weights of variance 1/C),
    # then the attention over the three projected tensors.
    wq_np = synth.make_qkv_weight(SEED_CONFIG, C, synth.BF16)
    wq = torch.from_numpy(wq_np.view(np.int16)).view(torch.bfloat16).to(x.device)
    qkv = tuple(torch.empty_like(cv) for _ in range(3))
    ms = timed(lambda: vinf.qkv_project(cv, wq, out=qkv, stream=stream), steps, stream)
    pflops, pbytes = 6 * C * C * F * S, F * S * 4 * C * b
    out["qkv_project_bf16"] = {"ms": round(ms, 4), "TFLOP/s": round(pflops / (ms * 1e-3) / 1e12, 1),
                               "frac_mfma_bf16": round(pflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                               **hbm_entry(ms, pbytes),
                               "shape": f"F={F}, {H}x{W}x{C}: q, k, v = three {C}x{C} maps of every token"}
    o = torch.empty_like(cv)
    ms = timed(lambda: vinf.projected_dual_domain_attn(cv, wq, out=o, qkv=qkv, stream=stream), steps, stream)
    out["projected_dda_bf16"] = {"ms": round(ms, 4), "voxels_per_s": F * S / (ms * 1e-3),
                                 "shape": f"F={F}, {H}x{W}x{C}: qkv_project, then dual_domain_attn on q, k, v"}
    ms = timed(lambda: vinf.projected_dual_domain_attn_fused(cv, wq, out=o, stream=stream), steps, stream)
    out["projected_dda_bf16_fused"] = {"ms": round(ms, 4), "voxels_per_s": F * S / (ms * 1e-3),
                                       "shape": f"F={F}, {H}x{W}x{C}: one launch, q, k, v projected inside the "
                                                f"attention's work items and never written"}
    del qkv, o
    # Reuse of attention outputs across a 30-step sampling schedule (range 3):
    # the attention cost per diffusion step, averaged over the schedule.
    n_steps, rng = 30, 3
    sched = vinf.attn_broadcast_schedule(n_steps, rng)
    o = torch.empty_like(cv)

    def thirty():
        for i in range(n_steps):
            vinf.dual_domain_attn_broadcast(cv, cv, cv, o, i, sched, stream=stream)

    ms = timed(thirty, max(1, steps // 10), stream)
    out["dda_bf16_broadcast"] = {"ms_per_step": round(ms / n_steps, 4), "computed_steps": int(sum(sched)),
                                 "steps": n_steps, "range": rng,
                                 "shape": f"F={F}, {H}x{W}x{C}, Q = K = V; every step in the first and last 15% "
                                          f"computes, the middle band one step in {rng}"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--cpu-side", type=int, default=32, help="locations per side of the CPU-baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy the input tensor once (a plain device copy of known size, for HBM counters)")
    ap.add_argument("--no-distinct", action="store_true",
                    help="skip the attention call on three distinct Q, K, V tensors")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the clip-form and ablation measurements")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the chain with the normalised tensor written out")
    ap.add_argument("--no-config3", action="store_true",
                    help="skip the per-call timings at F=1024, 32x20, C=640")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} requested)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import video_diffusion_temporal_amd as vinf

    F, H, W, C, G = (WORKLOAD[k] for k in ("F", "H", "W", "C", "G"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_np = synth.make_tensor(SEED_CONFIG, synth.X_GN, F, H, W, C, synth.BF16)
    w_np = synth.make_conv_weight(SEED_CONFIG, C, synth.BF16)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wt = torch.from_numpy(w_np.view(np.int16)).view(torch.bfloat16).to(dev)
    g = torch.empty_like(x)
    cv = torch.empty_like(x)
    o = torch.empty_like(x)
    mean = torch.empty(G, device=dev)
    rstd = torch.empty(G, device=dev)
    ws = torch.empty(vinf.groupnorm_workspace_bytes(F, H, W, C, G, x.dtype), device=dev, dtype=torch.uint8)
    cws = torch.empty(vinf.temporal_conv3_gn_workspace_bytes(C, x.dtype), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        g.copy_(x)  # 2 * F*H*W*C bytes of plain HBM traffic, before anything else
        torch.cuda.synchronize()

    # The step: GroupNorm statistics -> the conv of the GroupNorm output, the
    # normalisation applied to the conv's input tiles -> attention with Q = K = V.
    fused = [
        ("groupnorm_stats", lambda: vinf.groupnorm_stats(x, G, mean_out=mean, rstd_out=rstd, workspace=ws,
                                                         stream=stream)),
        ("conv3_bf16", lambda: vinf.temporal_conv3_gn(x, wt, mean, rstd, out=cv, workspace=cws, stream=stream)),
        ("dda_bf16", lambda: vinf.dual_domain_attn(cv, cv, cv, out=o, stream=stream)),
    ]
    # The same chain with the normalised tensor written and read back.
    unfused = [
        ("groupnorm", lambda: vinf.groupnorm_global(x, G, out=g, mean_out=mean, rstd_out=rstd, workspace=ws,
                                                    stream=stream)),
        ("conv3_bf16", lambda: vinf.temporal_conv3(g, wt, out=cv, stream=stream)),
        ("dda_bf16", lambda: vinf.dual_domain_attn(cv, cv, cv, out=o, stream=stream)),
    ]

    def run_chain(mods):
        """Warm up, then time args.steps steps with HIP events on the launch stream around every module."""
        for _ in range(args.warmup):
            for _, f in mods:
                f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(mods) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            for j, (_, f) in enumerate(mods):
                evs[i][j].record(stream)
                f()
            evs[i][-1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, (name, _) in enumerate(mods)}
        per["step"] = [e[0].elapsed_time(e[-1]) for e in evs]
        mod_ms = {name: sum(per[name]) / args.steps for name, _ in mods}
        return evs[0][0].elapsed_time(evs[-1][-1]) / args.steps, mod_ms, wall, {k: percentiles(v) for k, v in per.items()}

    work = algorithmic_work(F, H, W, C)

    def kernel_table(mod_ms):
        out = {}
        for k, ms in mod_ms.items():
            wk = work[k]
            gbs = wk["bytes"] / (ms * 1e-3) / 1e9
            tfl = wk["flops"] / (ms * 1e-3) / 1e12
            out[k] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "TFLOP/s": round(tfl, 2),
                      "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "frac_mfma_bf16": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4) if k == "conv3_bf16" else None}
        return out

    unfused_chain = None
    if not args.no_unfused:
        ms_u, mod_u, _, _ = run_chain(unfused)
        unfused_chain = {"ms_per_step": round(ms_u, 4), "voxels_per_s": F * H * W / (ms_u * 1e-3),
                         "kernels": kernel_table(mod_u),
                         "chain": "groupnorm (stats + apply, normalised tensor written) -> conv3 -> dual_domain_attn"}
    ms_step, mod_ms, wall, pct = run_chain(fused)
    vox = F * H * W
    kernels = kernel_table(mod_ms)
    # dominant single-kernel module (the GroupNorm statistics are four launches)
    dom = max(("conv3_bf16", "dda_bf16"), key=lambda k: mod_ms[k])
    wk = work[dom]
    if wk["bound"] == "hbm":
        achieved = wk["bytes"] / (mod_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_record(dom)}
    else:
        achieved = wk["flops"] / (mod_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic_record(dom)}
    roof["ms_per_launch"] = round(mod_ms[dom], 4)
    # The HBM bytes the counters saw per launch, over the same time and peak:
    # for the attention with Q = K = V one tensor is read once, not three times.
    if roof["traffic"]:
        roof["physical_gbs"] = round(roof["traffic"] / (mod_ms[dom] * 1e-3) / 1e9, 1)
        roof["physical_frac"] = round(roof["physical_gbs"] / HBM_PEAK_GBS, 4)

    # Attention on three distinct tensors (in the chain Q, K and V are one
    # tensor, so that call reads half the bytes a general call must).
    distinct = None
    if not args.no_distinct:
        kd = torch.empty_like(x)
        vd = torch.empty_like(x)
        kd.copy_(cv.flip(0))      # frames reversed: different data, same distribution
        vd.copy_(x)
        for _ in range(2):
            vinf.dual_domain_attn(cv, kd, vd, out=o, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            vinf.dual_domain_attn(cv, kd, vd, out=o, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        gbs = work["dda_bf16"]["bytes"] / (ms * 1e-3) / 1e9
        distinct = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del kd, vd

    nxt = None if args.no_next else next_rows(vinf, x, cv, G, stream, args.steps)
    c3 = None if args.no_config3 else config3_calls(vinf, args.steps, stream)
    for _, f in fused:  # o = the step's output again, for the parity check
        f()
    torch.cuda.synchronize()

    parity = None
    if not args.no_check:
        import oracle

        locs = np.array([0, 1337, H * W - 1], dtype=np.int64)
        ref, _, _ = oracle.chain(x_np, w_np, G, locs=locs, nthreads=min(os.cpu_count() or 1, 16))
        got = o.reshape(F, H * W, C)[:, torch.as_tensor(locs, device=dev)].float().cpu().numpy()
        err = np.abs(got.astype(np.float64) - ref)
        parity = {"locations": locs.tolist(), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
                  "ok": bool(err.max() <= 2e-2 and err.mean() <= 2e-3)}

    cpu = None if args.no_cpu_baseline else cpu_baseline(F, C, G, args.cpu_side)

    out = {
        "metric": "temporal-module voxels/sec (F*H'*W') at F=1024; % HBM peak, % MFMA peak",
        "value": vox / (ms_step * 1e-3),
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent, conv weights N(0,1/(3C)))",
        "config": {"workload": WORKLOAD["name"], "F": F, "H": H, "W": W, "C": C, "heads": C // 64, "groups": G,
                   "n_local": 16, "n_global": 16,
                   "chain": "groupnorm statistics -> conv3 of the groupnorm output (normalisation applied to the "
                            "conv's input tiles in LDS) -> dual_domain_attn"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "percentiles_ms": pct,
        "chain_unfused": unfused_chain,
        "config3": c3,
        "dda_bf16_distinct_qkv": distinct,
        "next_rows": nxt,
        "wall_s_timed": wall,
        "parity_sampled": parity,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
