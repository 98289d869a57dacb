#!/usr/bin/env python3
"""Benchmark one rank's optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--parts step,adamw,ns]

Prints ONE JSON line.  The headline workload ("step") is a GPT-2-small-shaped
full optimizer step at world 1: AdamW on the tied 50304 x 768 embedding
(weight decay 0.1) and 25 vectors of 768 (no decay) as two
zopt_adamw_shard_step calls, and Muon on 12 layers x {Wq, Wk, Wv, Wo 768^2;
fc 3072 x 768; proj 768 x 3072} as one zopt_muon_step_groups call over the
three same-shape groups; `value` is its time in ms per step.  Two sub-objects
report the other two parts of the metric on their own workloads:

  adamw_shard     the ZeRO-2 flat AdamW shard of rank 3 of 8 over a
                  2.0e9-parameter backbone (buckets of 1 << 25, 2.5e8 shard
                  elements): HBM GB/s at 28 algorithmic bytes per element;
                  With it, the clipped step on the same shard: the
                  gradient-norm pass (2 B per element), the clip statistics and
                  the AdamW step reading grad_scale from device memory;
  newton_schulz   rank 0's Muon share of a 32-layer d=4096 decoder (8 x
                  [14336, 4096], 4 x [4096, 14336], 8 x [4096, 4096],
                  8 x [1024, 4096]): bf16 TFLOP/s at 3 m^2 n + m^3
                  algorithmic flops per iteration, 5 iterations (and the same
                  for the 1B model's rank-0 share);
  tiny            the tiny configuration's AdamW and Muon step times.

Inputs are seeded and synthetic, generated on the GPU before timing, so the
timed region starts with everything resident in HBM.  Timing: W untimed
warm-up steps, then K steps bracketed by torch.cuda.synchronize() and HIP
events on the stream the library launches on.  `cpu_baseline` times the CPU
oracle (test infrastructure) on the host: the same headline step in full, and
the other workloads on stated samples.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "AdamW shard GB/s (%HBM peak); Muon NS TFLOP/s (%MFMA); optimizer step ms"
ROOT = os.path.dirname(os.path.abspath(__file__))

# HBM bytes per launch from two calibrated rocprofv3 counter passes (FETCH_SIZE,
# WRITE_SIZE; scaled by what they read for a zopt_round_bf16 pass of known size),
# recorded in profiles/.  Reported only while the kernel source is the one the
# counters were taken on.
MEASURED_TRAFFIC = {
    # the full buckets (bucket-grid launch) and the last bucket: 3.500 GB read, 3.500 GB written
    "adamw_shard": dict(source="sharded_optimizer_step_adamw_amd/csrc/adamw_shard.hip",
                        sha256="673b6ee27b692f43da0cb776f129120c95304617a7117f995f9273186f2e9bca",
                        bytes_per_launch=7.000e9,
                        profile="profiles/adamw_bucket_grid_kernel_zero2_2b_rank3.md"),
    # the Newton-Schulz of one 5-step Muon call: every NS launch of the call (the
    # symmetric products, the fix-ups of split X X^T, P X / Q X), FETCH_SIZE + WRITE_SIZE
    # summed over the call's dispatches and calibrated; the launch plan (which launches
    # exist, on which stream) is in zopt_api.hip.
    # GPT-2 small: 2.764 GB read, 1.591 GB written (32 launches on two streams)
    "ns_call_gpt2": dict(source="sharded_optimizer_step_adamw_amd/csrc/ns_gemm.hip",
                         sha256="b194c209b68ecdfc860e298b700b2dfd768eab25cdd8f9ccad2017d401ce9bf3",
                         also=[("sharded_optimizer_step_adamw_amd/csrc/zopt_api.hip",
                                "f9f3bae7e107017205a12a39b56884891e53c95f876d7cbd0364e70c42cf6db7")],
                         bytes_per_launch=4.355e9, profile="profiles/ns_gemm_gpt2_small_step.md"),
    # 8B rank-0 share: 88.22 GB read, 14.68 GB written (23 launches)
    "ns_call_llama8b": dict(source="sharded_optimizer_step_adamw_amd/csrc/ns_gemm.hip",
                            sha256="b194c209b68ecdfc860e298b700b2dfd768eab25cdd8f9ccad2017d401ce9bf3",
                            also=[("sharded_optimizer_step_adamw_amd/csrc/zopt_api.hip",
                                   "f9f3bae7e107017205a12a39b56884891e53c95f876d7cbd0364e70c42cf6db7")],
                            bytes_per_launch=102.9e9, profile="profiles/ns_gemm_llama8b_rank0.md"),
    # 1B rank-0 share: 4.655 GB read, 1.539 GB written (49 launches on two streams)
    "ns_call_llama1b": dict(source="sharded_optimizer_step_adamw_amd/csrc/ns_gemm.hip",
                            sha256="b194c209b68ecdfc860e298b700b2dfd768eab25cdd8f9ccad2017d401ce9bf3",
                            also=[("sharded_optimizer_step_adamw_amd/csrc/zopt_api.hip",
                                   "f9f3bae7e107017205a12a39b56884891e53c95f876d7cbd0364e70c42cf6db7")],
                            bytes_per_launch=6.194e9, profile="profiles/ns_gemm_llama1b_rank0.md"),
    "grad_sq_norm": dict(source="sharded_optimizer_step_adamw_amd/csrc/adamw_shard.hip",
                         sha256="673b6ee27b692f43da0cb776f129120c95304617a7117f995f9273186f2e9bca",
                         bytes_per_launch=0.5004e9,
                         profile="profiles/grad_sq_norm_kernel_zero2_2b_rank3.md"),
}


def measured_traffic(key):
    import hashlib
    t = MEASURED_TRAFFIC[key]
    if t["sha256"] is None:
        return None
    for src, sha in [(t["source"], t["sha256"])] + list(t.get("also", [])):
        with open(os.path.join(ROOT, src), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    return t["bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--parts", default="step,adamw,clip,ns,graph,tiny",
                    help="comma list of: step (headline), adamw, clip (the clipped step on the "
                         "adamw shard; needs adamw), ns (8B and 1B rank-0 Muon shares), graph "
                         "(eager vs captured Muon calls), tiny (the tiny configuration), copy (a "
                         "zopt_round_bf16 pass of known size: the calibration for HBM byte "
                         "counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain-form", action="store_true",
                    help="skip the plain-form Newton-Schulz A/B timings (for profiles)")
    return ap.parse_args()


def gram_segments(steps, per=3):
    """Segment lengths of the Gram form (the library's rule): ceil(steps / 3)
    segments as even as possible, longer ones first."""
    if steps <= 0:
        return []
    nseg = (steps + per - 1) // per
    base, extra = divmod(steps, nseg)
    return [base + (1 if i < extra else 0) for i in range(nseg)]


def ns_flops(m, n, steps, form=0, batch=1):
    """Algorithmic flops of `steps` Newton-Schulz steps on one m x n input
    (m <= n) of a group of `batch`, as the library computes them.  Plain
    iterations (form 1, n < 2 m, or batch m^2 (n - m) < 2^29): per step
    upper-triangle X X^T (m^2 n), upper-triangle A A (m^3), B X (2 m^2 n).
    Gram form otherwise (m <= 4096): per segment of L steps X X^T (m^2 n), L
    upper-triangle A_j A_j, 3 (L - 1) upper-triangle products of two
    symmetric m x m matrices (m^3 each), Q X (2 m^2 n)."""
    if form == 1 or n < 2 * m or m > 4096 or batch * m * m * (n - m) < 2 ** 29:
        return steps * (3 * m * m * n + m ** 3)
    return sum(3 * m * m * n + (4 * L - 3) * m ** 3 for L in gram_segments(steps))


def group_flops(groups, steps, form=0):
    return sum(g["count"] * ns_flops(min(g["rows"], g["cols"]), max(g["rows"], g["cols"]), steps,
                                     form, g["count"]) for g in groups)


PLAIN_FORM_AB = [True]


def timed_forms(z, timer, fn, K):
    """fn timed K times in the plain form (A/B against the default, on the
    same buffers); the default form restored after.  NaN when skipped."""
    if not PLAIN_FORM_AB[0]:
        return float("nan")
    z.set_ns_form(z.NS_FORM_PLAIN)
    try:
        fn(0)
        return timer.run(fn, K)
    finally:
        z.set_ns_form(z.NS_FORM_AUTO)


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, iters):
        torch = self.torch
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters  # ms per iteration


# ------------------------------------------------------------------ workloads

def make_adamw(torch, w, dev, n_grads=1):
    import workloads as wl
    n = w.n_total
    st = dict(master=wl.device_normal(w.wid, 0, (n,), w.master_std, dev),
              weight=torch.zeros(n, dtype=torch.bfloat16, device=dev),
              grads=[wl.device_grad_bf16(w.wid, 1, (n,), w.grad_std, dev,
                                         "normal_outliers" if w.outlier_frac else "normal",
                                         step=s) for s in range(n_grads)])
    return st


def adamw_zero2_state(torch, dev):
    import workloads as wl
    import sharded_optimizer_step_adamw_amd as z
    w = wl.ZERO2_ADAMW
    part = w.parts[0]
    sl = z.shard_len(part.n, part.bucket, part.world)
    st = dict(part=part, shard_len=sl,
              master=wl.device_normal(w.wid, 0, (sl,), w.master_std, dev),
              m=torch.zeros(sl, device=dev), v=torch.zeros(sl, device=dev),
              weight=torch.zeros(part.n, dtype=torch.bfloat16, device=dev),
              grads=[wl.device_grad_bf16(w.wid, 1, (part.n,), w.grad_std, dev, step=s)
                     for s in range(4)])
    return st


def muon_groups(torch, w, dev):
    import workloads as wl
    import sharded_optimizer_step_adamw_amd as z
    groups = []
    for gi, grp in enumerate(w.groups):
        shape = (grp.rows, grp.cols)
        groups.append(dict(
            rows=grp.rows, cols=grp.cols, count=grp.count,
            master=[wl.device_normal(w.wid, 100 * gi + i, shape, w.master_std, dev)
                    for i in range(grp.count)],
            momentum=[torch.zeros(shape, device=dev) for _ in range(grp.count)],
            grad=[wl.device_grad_bf16(w.wid, 5000 + 100 * gi + i, shape, w.grad_std, dev,
                                      w.grad_dist) for i in range(grp.count)],
            weight=[torch.empty(shape, dtype=torch.bfloat16, device=dev)
                    for _ in range(grp.count)]))
    ws_bytes = z.muon_groups_workspace_bytes([(g["count"], g["rows"], g["cols"]) for g in groups])
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    return groups, workspace


def muon_call(z, w, groups, workspace, ns_steps, health=None):
    """All groups of a workload in one zopt_muon_step_groups call (with a
    health tensor: zopt_muon_step_groups_guarded, guard 1000)."""
    z.muon_step_groups([(g["master"], g["momentum"], g["grad"], g["weight"]) for g in groups],
                       w.lr, w.momentum, w.nesterov, w.weight_decay, ns_steps, w.ns_coeffs,
                       w.ns_eps, w.adjust_lr, workspace=workspace,
                       ns_guard=None if health is None else 1000.0, ns_health=health)


def ns_health_check(torch, z, timer, w, groups, workspace, K, plain_ms):
    """The guarded call against the plain one: the health pass reads each
    matrix's bf16 result once (2 B per element of the padded-width X)."""
    nmat = sum(g["count"] for g in groups)
    health = torch.empty(2 + 3 * nmat, dtype=torch.float32, device=groups[0]["master"][0].device)
    timer.run(lambda _: muon_call(z, w, groups, workspace, w.ns_steps, health), 1)
    ms = timer.run(lambda _: muon_call(z, w, groups, workspace, w.ns_steps, health), K)
    h = health.cpu()
    tile = lambda m: 256 if m >= 1024 else 128 if m >= 256 else 64
    bytes_read = sum(2 * g["count"] * min(g["rows"], g["cols"]) *
                     (-(-max(g["rows"], g["cols"]) // tile(min(g["rows"], g["cols"])))
                      * tile(min(g["rows"], g["cols"]))) for g in groups)
    return dict(guarded_call_ms=round(ms, 4), overhead_ms=round(ms - plain_ms, 4),
                health_pass_bytes=bytes_read, rejected=int(h[0]),
                worst_ratio=round(float(h[1]), 4))


# ------------------------------------------------------------------ parts

def bench_step(torch, z, timer, dev, K, W):
    """The headline: one GPT-2-small optimizer step (2 AdamW calls + 1 Muon call
    over three groups)."""
    import workloads as wl
    wa, wm = wl.GPT2_ADAMW, wl.GPT2_MUON
    a = make_adamw(torch, wa, dev)
    n = wa.n_total
    a["m"], a["v"] = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
    groups, workspace = muon_groups(torch, wm, dev)
    counter = [0]

    def step(_):
        counter[0] += 1
        t = counter[0]
        for part in wa.parts:
            s = slice(part.offset, part.offset + part.n)
            z.adamw_shard_step(a["master"][s], a["m"][s], a["v"][s], a["grads"][0][s],
                               a["weight"][s], part.n, part.bucket, part.world, part.rank,
                               part.lr, part.beta1, part.beta2, part.eps, part.weight_decay, t)
        muon_call(z, wm, groups, workspace, wm.ns_steps)

    timer.run(step, W)
    ms = timer.run(step, K)

    # the dominant kernels: the Newton-Schulz of the Muon call (72 matrices,
    # 5 steps) on two streams -- the 48 x [768, 768] group in plain
    # iterations on one, the 768 x 3072 groups in Gram segments of 3 and 2
    # steps on the other; its time is the 5-step call less the call with no
    # steps (momentum, pre-scale and post-step only)
    t5 = timer.run(lambda _: muon_call(z, wm, groups, workspace, 5), K)
    t0 = timer.run(lambda _: muon_call(z, wm, groups, workspace, 0), K)
    ns_ms = t5 - t0
    ns_fl = group_flops(groups, 5)
    t5p = timed_forms(z, timer, lambda _: muon_call(z, wm, groups, workspace, 5), K)
    per_group = dict(muon_call_ms=round(t5, 4), zero_step_call_ms=round(t0, 4),
                     ns_ms=round(ns_ms, 4),
                     plain_form=None if t5p != t5p else dict(
                         muon_call_ms=round(t5p, 4), ns_ms=round(t5p - t0, 4),
                         algorithmic_flops=group_flops(groups, 5, form=1)),
                     groups=[dict(shape=[g["rows"], g["cols"]], count=g["count"]) for g in groups],
                     ns_health=ns_health_check(torch, z, timer, wm, groups, workspace, K, t5))
    adamw_bytes = 28 * n
    ta = timer.run(lambda i: [z.adamw_shard_step(
        a["master"][p.offset:p.offset + p.n], a["m"][p.offset:p.offset + p.n],
        a["v"][p.offset:p.offset + p.n], a["grads"][0][p.offset:p.offset + p.n],
        a["weight"][p.offset:p.offset + p.n], p.n, p.bucket, p.world, p.rank, p.lr, p.beta1,
        p.beta2, p.eps, p.weight_decay, 1000 + i) for p in wa.parts], K)
    del a, groups, workspace
    torch.cuda.empty_cache()
    return dict(ms=ms, ns_ms=ns_ms, ns_flops=ns_fl, muon=per_group,
                adamw_ms=ta, adamw_gbs=adamw_bytes / ta / 1e6)


def bench_adamw(torch, z, timer, dev, K, W, clip_leg=False):
    s = adamw_zero2_state(torch, dev)
    p, sl = s["part"], s["shard_len"]
    counter = [0]

    def step(i):
        counter[0] += 1
        z.adamw_shard_step(s["master"], s["m"], s["v"], s["grads"][counter[0] % 4], s["weight"],
                           p.n, p.bucket, p.world, p.rank, p.lr, p.beta1, p.beta2, p.eps,
                           p.weight_decay, counter[0])

    timer.run(step, W)
    ms = timer.run(step, K)
    clip = bench_clip(torch, z, timer, s, K, W) if clip_leg else None
    del s
    torch.cuda.empty_cache()
    gbs = 28 * sl / ms / 1e6
    roof = dict(kernel=("zopt_adamw_shard_step: adamw_bucket_grid_kernel over the 59 full "
                        "buckets + adamw_shard_kernel over the short last one (two launches "
                        "per step, timed together)"), bound="hbm",
                achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), traffic=measured_traffic("adamw_shard"),
                algorithmic_bytes_per_launch=28 * sl, avg_launch_ms=round(ms, 4),
                launches_per_step=2)
    out = dict(workload="zero2 flat AdamW shard: N=2.0e9, bucket 1<<25, world 8, rank 3",
               shard_len=sl, algorithmic_bytes_per_step=28 * sl, ms_per_step=round(ms, 4),
               gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4), steps=K,
               roofline=roof)
    if clip:
        out["clipped_step"] = clip
    return out


def bench_clip(torch, z, timer, s, K, W):
    """The clipped step on the same shard: zopt_grad_sq_norm (2 B read per
    element: the norm pass and its one-workgroup final sum), zopt_grad_clip_stats
    and zopt_adamw_shard_step_clipped reading grad_scale from device memory --
    no host round trip anywhere in the step."""
    p, sl = s["part"], s["shard_len"]
    dev = s["master"].device
    ws = torch.empty(z.grad_sq_norm_workspace_bytes(p.n, p.bucket, p.world, p.rank),
                     dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    stats = torch.empty(z.CLIP_STATS, dtype=torch.float32, device=dev)
    counter = [0]

    def norm(i):
        z.grad_sq_norm(s["grads"][i % 4], p.n, p.bucket, p.world, p.rank, out=sq, workspace=ws)

    def step(i):
        counter[0] += 1
        g = s["grads"][counter[0] % 4]
        z.grad_sq_norm(g, p.n, p.bucket, p.world, p.rank, out=sq, workspace=ws)
        z.grad_clip_stats(sq, 1.0, out=stats)
        z.adamw_shard_step_clipped(s["master"], s["m"], s["v"], g, s["weight"], p.n, p.bucket,
                                   p.world, p.rank, p.lr, p.beta1, p.beta2, p.eps,
                                   p.weight_decay, 10_000 + counter[0], stats,
                                   skip_nonfinite=True)

    timer.run(norm, W)
    norm_ms = timer.run(norm, K)
    timer.run(step, W)
    step_ms = timer.run(step, K)
    norm_gbs = 2 * sl / norm_ms / 1e6
    return dict(
        norm_ms=round(norm_ms, 4), clipped_step_ms=round(step_ms, 4),
        clipped_step_gbs=round(30 * sl / step_ms / 1e6, 1), algorithmic_bytes_per_step=30 * sl,
        clip_coef_last=round(float(stats[z.CLIP_COEF].item()), 6),
        roofline=dict(kernel="grad_sq_norm_kernel + its one-workgroup final sum (one call)",
                      bound="hbm", achieved=round(norm_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(norm_gbs / HBM_PEAK_GBS, 4),
                      traffic=measured_traffic("grad_sq_norm"),
                      algorithmic_bytes_per_launch=2 * sl, avg_launch_ms=round(norm_ms, 4)))


def bench_ns(torch, z, timer, dev, K, W, w=None):
    import workloads as wl
    w = w or wl.LLAMA8B_MUON
    groups, workspace = muon_groups(torch, w, dev)
    total_flops = group_flops(groups, w.ns_steps)
    plain_flops = group_flops(groups, w.ns_steps, form=1)
    timer.run(lambda _: muon_call(z, w, groups, workspace, w.ns_steps), max(1, W))
    t5 = timer.run(lambda _: muon_call(z, w, groups, workspace, w.ns_steps), K)
    t0 = timer.run(lambda _: muon_call(z, w, groups, workspace, 0), K)
    # the Newton-Schulz of the call: the 5-step call less the call with no
    # steps (momentum, pre-scale and post-step; with no steps the pre-scale
    # writes X0 = bf16(U s), and X0^T for matrices stored transposed, where a
    # call with steps writes bf16(U): the same bytes but for that transpose)
    ns_ms, call_ms = t5 - t0, t5
    t5p = timed_forms(z, timer, lambda _: muon_call(z, w, groups, workspace, w.ns_steps), K)
    plain = None if t5p != t5p else dict(
        muon_ms_per_step=round(t5p, 3), ns_ms_per_step=round(t5p - t0, 3),
        algorithmic_flops_per_step=group_flops(groups, w.ns_steps, form=1))
    rows = [dict(shape=[g["rows"], g["cols"]], count=g["count"]) for g in groups]
    health = ns_health_check(torch, z, timer, w, groups, workspace, K, t5)
    del groups, workspace
    torch.cuda.empty_cache()
    tf = total_flops / ns_ms / 1e9
    names = {"llama8b_rank0_muon": "llama8b rank-0 Muon share (W=8, 32 layers), 5 bf16 NS iterations",
             "llama1b_rank0_muon": "llama1b rank-0 Muon share (W=8, 16 layers), 5 bf16 NS iterations"}
    # the dominant kernels: the Newton-Schulz products of one 5-step call over
    # every matrix of the share (the unit), timed as the 5-step call less the
    # call with no steps
    if w.name == "llama8b_rank0_muon":
        kernel = ("Newton-Schulz of the 28 matrices, one stream, 23 merged steps: the 8 x [4096, "
                  "4096] group in plain iterations (ns_gemm_kernel<256,0,bf16> X X^T, "
                  "ns_gemm_kernel<256,1,bf16> P, ns_bx_kernel<256> P X), the three groups with "
                  "n >= 2m in Gram segments of 3 and 2 steps (X X^T, ns_gemm_kernel<256,1,fp16> "
                  "and ns_gemm_kernel<256,3,fp16> on the m x m chain, ns_bx_kernel<256> Q X)")
        traffic, tunit = measured_traffic("ns_call_llama8b"), "HBM bytes per 5-step call (all NS launches)"
    else:
        kernel = ("Newton-Schulz of the 12 matrices on two streams: the two 2048-row groups in "
                  "Gram segments (the 11264 x 2048 pair with X X^T split along K plus its "
                  "fix-up, and 2048 x 5632) on the caller's, the 2048 x 2048 group in plain "
                  "iterations and the 512 x 2048 group in Gram segments on the second")
        traffic, tunit = measured_traffic("ns_call_llama1b"), "HBM bytes per 5-step call (all NS launches)"
    roof = dict(kernel=kernel, bound="mfma", achieved=round(tf, 1), peak=BF16_PEAK_TFLOPS,
                unit="TFLOP/s", frac=round(tf / BF16_PEAK_TFLOPS, 4), traffic=traffic,
                traffic_unit=tunit, algorithmic_flops_per_unit=total_flops,
                avg_unit_ms=round(ns_ms, 4))
    return dict(workload=names.get(w.name, w.name),
                algorithmic_flops_per_step=total_flops, ns_ms_per_step=round(ns_ms, 3),
                muon_ms_per_step=round(call_ms, 3), ns_tflops=round(tf, 1),
                mfma_frac=round(tf / BF16_PEAK_TFLOPS, 4),
                # the plain iteration's flops (5 (3 m^2 n + m^3) per matrix) over the measured
                # time: the utilisation plain iterations would need to take this long
                frac_on_plain_iteration_flops=round(plain_flops / ns_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                muon_step_tflops=round(total_flops / call_ms / 1e9, 1), zero_step_call_ms=round(t0, 3),
                plain_form=plain, groups=rows, steps=K, ns_health=health, roofline=roof)


def bench_graph(torch, z, timer, dev, K, W):
    """A Muon call issued eagerly against the same call captured once and
    replayed (zopt_muon_graph_*), on the tiny workload (2 x [128, 512]) and
    the headline's 72 GPT-2-small matrices.  GPU time per call from HIP
    events over K back-to-back calls; host time per call is the wall time to
    enqueue 20 calls, measured three ways: through the Python binding (its
    tensor checks included), straight through the C ABI with prebuilt
    arguments, and a graph launch through the C ABI."""
    import ctypes
    import workloads as wl
    out = {}
    lib = z.lib()
    for w in (wl.TINY_MUON, wl.GPT2_MUON):
        groups, workspace = muon_groups(torch, w, dev)
        tup = [(g["master"], g["momentum"], g["grad"], g["weight"]) for g in groups]
        scalars = torch.tensor([w.lr, w.momentum, w.weight_decay], dtype=torch.float32,
                               device=dev)
        graph = z.MuonGraph(tup, scalars, w.nesterov, w.ns_steps, w.ns_coeffs, w.ns_eps,
                            w.adjust_lr, workspace=workspace)
        shapes, M, Mo, G, Wt, _, _ = z._muon_group_tables(tup)
        n, b, r, c = z._shape_arrays(shapes)
        size = ctypes.c_size_t(workspace.numel())
        stream = torch.cuda.current_stream(dev).cuda_stream
        cargs = (n, b, r, c, z._ptr_array(M), z._ptr_array(Mo), z._ptr_array(G),
                 z._ptr_array(Wt), w.lr, w.momentum, int(w.nesterov), w.weight_decay, w.ns_steps,
                 *(float(x) for x in w.ns_coeffs), w.ns_eps, w.adjust_lr, workspace.data_ptr(),
                 ctypes.byref(size), stream)
        handle = graph._handle

        def eager_binding(_):
            muon_call(z, w, groups, workspace, w.ns_steps)

        def eager_c(_):
            lib.zopt_muon_step_groups(*cargs)

        def replay(_):
            lib.zopt_muon_graph_launch(handle, stream)

        def host_us(fn, calls=20):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(calls):
                fn(i)
            t1 = time.perf_counter()
            torch.cuda.synchronize()
            return (t1 - t0) / calls * 1e6

        res = {}
        for name, fn in (("eager", eager_c), ("graph", replay)):
            timer.run(fn, W)
            res[name + "_gpu_ms"] = round(timer.run(fn, K), 4)
        for name, fn in (("eager_binding", eager_binding), ("eager_c_abi", eager_c),
                         ("graph_c_abi", replay)):
            host_us(fn)
            res[name + "_host_us"] = round(min(host_us(fn) for _ in range(3)), 1)
        graph.close()
        out[w.name] = res
        del groups, workspace, graph
        torch.cuda.empty_cache()
    return out


def bench_tiny(torch, z, timer, dev, K, W):
    """The tiny configuration: one AdamW call on rank 0's shard of a
    1,048,576-element vector (buckets of 262,144, world 4) and one Muon call on
    2 x [128, 512]; per-step time (both launch-bound: 7 MB of state)."""
    import workloads as wl
    wa, wm = wl.TINY_ADAMW, wl.TINY_MUON
    part = wa.parts[0]
    sl = z.shard_len(part.n, part.bucket, part.world)
    master = wl.device_normal(wa.wid, 0, (sl,), wa.master_std, dev)
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    grad = wl.device_grad_bf16(wa.wid, 1, (part.n,), wa.grad_std, dev)
    weight = torch.zeros(part.n, dtype=torch.bfloat16, device=dev)
    groups, workspace = muon_groups(torch, wm, dev)
    counter = [0]

    def adamw(_):
        counter[0] += 1
        z.adamw_shard_step(master, m, v, grad, weight, part.n, part.bucket, part.world, part.rank,
                           part.lr, part.beta1, part.beta2, part.eps, part.weight_decay, counter[0])

    def step(i):
        adamw(i)
        muon_call(z, wm, groups, workspace, wm.ns_steps)

    timer.run(step, W)
    step_ms = timer.run(step, K)
    adamw_ms = timer.run(adamw, K)
    muon_ms = timer.run(lambda _: muon_call(z, wm, groups, workspace, wm.ns_steps), K)
    del master, m, v, grad, weight, groups, workspace
    torch.cuda.empty_cache()
    return dict(workload="tiny: AdamW rank-0 shard of 1,048,576 (bucket 262,144, world 4) + Muon "
                         "2 x [128, 512], 5 NS iterations",
                step_ms=round(step_ms, 4), adamw_ms=round(adamw_ms, 4), muon_ms=round(muon_ms, 4),
                adamw_gbs=round(28 * sl / adamw_ms / 1e6, 1))


def bench_copy(torch, z, timer, dev, K, W):
    """zopt_round_bf16 over 2.5e8 fp32 values: 1.0e9 bytes read, 0.5e9 written
    per launch, the reference for scaling FETCH_SIZE / WRITE_SIZE counters."""
    n = 250_000_000
    src = torch.randn(n, device=dev)
    dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
    timer.run(lambda _: z.round_bf16(src, dst), W)
    ms = timer.run(lambda _: z.round_bf16(src, dst), K)
    del src, dst
    torch.cuda.empty_cache()
    return dict(elements=n, bytes_read=4 * n, bytes_written=2 * n, ms=round(ms, 4),
                gbs=round(6 * n / ms / 1e6, 1))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _cpu_threads():
    """The threads the all-cores legs use: the process's CPU share, capped by
    OMP_NUM_THREADS where it is set (the BLAS behind numpy follows it too)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else n


def _blas_limit(n):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:  # no control over BLAS threads: leave them as they are
        import contextlib
        return contextlib.nullcontext()


def _adamw_points_timed(oracle, arrays, hp, steps, threads, step0=1):
    """The oracle's element-wise AdamW (binary32, scalar C) over `steps`
    steps of the given elements, split into `threads` contiguous chunks run
    concurrently (ctypes releases the GIL during the call).  Seconds."""
    from concurrent.futures import ThreadPoolExecutor
    p, m, v, g = arrays
    n = p.size
    bounds = [(k * n // threads, (k + 1) * n // threads) for k in range(threads)]

    def run(b, t):
        lo, hi = b
        oracle.adamw_points(p[lo:hi], m[lo:hi], v[lo:hi], g[lo:hi], *hp, t)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for t in range(step0, step0 + steps):
            list(ex.map(run, bounds, [t] * threads))
    return time.perf_counter() - t0


def _gathered_grads(oracle, part, rng_grad):
    """binary32 gradients of rank part.rank's shard elements (the flat
    gradient gathered through the oracle's index map; padding 0)."""
    import numpy as np
    sl = oracle.shard_len(part.n, part.bucket, part.world)
    flat, real = oracle.shard_index_map(part.n, part.bucket, part.world, part.rank,
                                        np.arange(sl))
    g = np.zeros(sl, np.float32)
    g[real] = oracle.bf16_bits_to_f32(rng_grad[flat[real]])
    return g


def _muon_one_per_shape(oracle, wl, w, threads):
    """One matrix per distinct stored shape through the oracle's whole Muon
    step with no iteration (binary32 pre- and post-step in C, the float64
    pre-scale), plus the cost of one float64 Newton-Schulz iteration through
    numpy's BLAS on `threads` threads, timed once per distinct Newton-Schulz
    shape (min x max: both orientations of a shape iterate on the same
    product sizes) as ns(U, 1) - ns(U, 0).  Per matrix: t0 + 5 iterations;
    then times the group's matrix count.  Seconds, and the per-shape rows."""
    import numpy as np
    per_shape, total, iter_s = [], 0.0, {}
    with _blas_limit(threads):
        for gi, grp in enumerate(w.groups):
            shape = (grp.rows, grp.cols)
            r = wl.rng(w.wid, 700 + gi)
            p = r.standard_normal(shape, dtype=np.float32) * np.float32(w.master_std)
            if w.grad_dist == "student_t3":
                gx = r.standard_t(3, size=shape) * w.grad_std
            else:
                gx = r.standard_normal(shape, dtype=np.float32) * np.float32(w.grad_std)
            g = wl.to_bf16_bits(np.asarray(gx, np.float32))
            del gx
            mm = np.zeros(shape, np.float32)
            t = time.perf_counter()
            oracle.muon_step(p, mm, g, w.lr, w.momentum, w.nesterov, w.weight_decay, 0,
                             w.ns_coeffs, w.ns_eps, w.adjust_lr)
            t0 = time.perf_counter() - t
            key = (min(shape), max(shape))
            if key not in iter_s:
                u = oracle.muon_pre(np.zeros(shape, np.float32), g, w.momentum, w.nesterov)
                ts = []
                for steps in (0, 1):
                    t = time.perf_counter()
                    oracle.newton_schulz(u, steps, w.ns_coeffs, w.ns_eps)
                    ts.append(time.perf_counter() - t)
                iter_s[key] = max(ts[1] - ts[0], 0.0)
                del u
            one = t0 + w.ns_steps * iter_s[key]
            total += one * grp.count
            per_shape.append(dict(shape=list(shape), count=grp.count,
                                  s_step_no_iteration=round(t0, 3),
                                  s_per_iteration=round(iter_s[key], 3),
                                  s_per_matrix_extrapolated=round(one, 3)))
            del p, g, mm
    return total, per_shape


def cpu_baseline():
    """The CPU oracle (test infrastructure, untuned) on the host cores.

    `value` is the headline GPT-2-small step in full (not extrapolated) on all
    the threads the process may use: the two AdamW calls over 38,652,672
    elements split into one contiguous chunk per thread, and all 72 Muon
    matrices with float64 Newton-Schulz through numpy's BLAS.  `configs`
    times the other workloads the same way, each with its sample stated:
    the tiny one in full on 1 thread and on all; the ZeRO-2 shard on a
    seeded sample of 1,048,576 shard indices over 100 steps, extrapolated to
    the whole shard, plus the whole shard's step 1; the 1B and 8B Muon shares
    on one matrix per shape, extrapolated by iteration and matrix count."""
    import numpy as np
    import oracle
    import workloads as wl
    T = _cpu_threads()
    configs = {}

    # --- headline: the GPT-2-small step, whole
    wa, wm = wl.GPT2_ADAMW, wl.GPT2_MUON
    n = wa.n_total
    p0 = wl.host_normal(wa.wid, 0, n, wa.master_std)
    gb = wl.host_grad_bf16(wa.wid, 1, n, wa.grad_std, "normal_outliers")
    g32 = oracle.bf16_bits_to_f32(gb)
    adamw_s = {}
    for threads in (1, T):
        secs = 0.0
        for part in wa.parts:
            s = slice(part.offset, part.offset + part.n)
            arrays = (p0[s].copy(), np.zeros(part.n, np.float32), np.zeros(part.n, np.float32),
                      g32[s].copy())
            hp = (part.lr, part.beta1, part.beta2, part.eps, part.weight_decay)
            secs += _adamw_points_timed(oracle, arrays, hp, 1, threads)
        adamw_s[threads] = secs
    mats = []
    for gi, grp in enumerate(wm.groups):
        for i in range(grp.count):
            shape = (grp.rows, grp.cols)
            mats.append((wl.host_normal(wm.wid, 100 * gi + i, shape, wm.master_std),
                         np.zeros(shape, np.float32),
                         wl.host_grad_bf16(wm.wid, 5000 + 100 * gi + i, shape, wm.grad_std,
                                           "normal_outliers")))
    with _blas_limit(T):
        t0 = time.perf_counter()
        for master, mom, grad in mats:
            oracle.muon_step(master, mom, grad, wm.lr, wm.momentum, wm.nesterov,
                             wm.weight_decay, wm.ns_steps, wm.ns_coeffs, wm.ns_eps, wm.adjust_lr)
        muon_s = time.perf_counter() - t0
    head_ms = (adamw_s[T] + muon_s) * 1e3
    configs["gpt2_small_step"] = dict(
        ms_per_step=round(head_ms, 1), threads=T, extrapolated=False,
        adamw_ms_1_thread=round(adamw_s[1] * 1e3, 1), adamw_ms_all_threads=round(adamw_s[T] * 1e3, 1),
        muon_ms=round(muon_s * 1e3, 1),
        sample="whole step: AdamW over 38,652,672 elements, 72 Muon matrices, float64 NS")
    del p0, gb, g32, mats

    # --- tiny: whole, 10 steps, 1 thread and all
    ta, tm = wl.TINY_ADAMW, wl.TINY_MUON
    part = ta.parts[0]
    sl = oracle.shard_len(part.n, part.bucket, part.world)
    flat_g = wl.host_grad_bf16(ta.wid, 1, part.n, ta.grad_std)
    g = _gathered_grads(oracle, part, flat_g)
    p_t = wl.host_normal(ta.wid, 0, sl, ta.master_std)
    hp = (part.lr, part.beta1, part.beta2, part.eps, part.weight_decay)
    tiny = dict(sample="whole: AdamW rank-0 shard of 262,144 elements x 10 steps (one gradient "
                       "reused) + Muon 2 x [128, 512] x 10 steps, float64 NS",
                extrapolated=False, threads=T)
    mats = [(wl.host_normal(tm.wid, 10 + i, (128, 512), tm.master_std),
             wl.host_grad_bf16(tm.wid, 20 + i, (128, 512), tm.grad_std)) for i in range(2)]
    for threads, key in ((1, "ms_per_step_1_thread"), (T, "ms_per_step_all_threads")):
        arrays = (p_t.copy(), np.zeros(sl, np.float32), np.zeros(sl, np.float32), g)
        a_s = _adamw_points_timed(oracle, arrays, hp, ta.steps, threads)
        with _blas_limit(threads):
            ms = [(p.copy(), np.zeros((128, 512), np.float32), gg) for p, gg in mats]
            t0 = time.perf_counter()
            for _ in range(tm.steps):
                for master, mom, gg in ms:
                    oracle.muon_step(master, mom, gg, tm.lr, tm.momentum, tm.nesterov,
                                     tm.weight_decay, tm.ns_steps, tm.ns_coeffs, tm.ns_eps,
                                     tm.adjust_lr)
            m_s = time.perf_counter() - t0
        tiny[key] = round((a_s / ta.steps + m_s / tm.steps) * 1e3, 2)
    configs["tiny"] = tiny

    # --- ZeRO-2 shard: a seeded sample of shard indices over 100 steps,
    # extrapolated; and the whole shard's first step
    wz = wl.ZERO2_ADAMW
    part = wz.parts[0]
    sl = oracle.shard_len(part.n, part.bucket, part.world)
    k = 1_048_576
    r = wl.rng(wz.wid, 900)
    hp = (part.lr, part.beta1, part.beta2, part.eps, part.weight_decay)
    sample_p = r.standard_normal(k, dtype=np.float32) * np.float32(wz.master_std)
    sample_g = oracle.bf16_bits_to_f32(wl.to_bf16_bits(
        r.standard_normal(k, dtype=np.float32) * np.float32(wz.grad_std)))
    z2 = dict(sample=(f"a seeded sample of {k:,} shard elements over {wz.steps} steps (element-"
                      f"wise: exact for those elements), per-step time extrapolated linearly to "
                      f"the {sl:,}-element shard; plus the whole shard's step 1 (the sample's "
                      f"values repeated over it)"),
              extrapolated=True, threads=T)
    for threads, key in ((1, "ms_per_step_extrapolated_1_thread"),
                         (T, "ms_per_step_extrapolated_all_threads")):
        arrays = (sample_p.copy(), np.zeros(k, np.float32), np.zeros(k, np.float32), sample_g)
        secs = _adamw_points_timed(oracle, arrays, hp, wz.steps, threads)
        z2[key] = round(secs / wz.steps * (sl / k) * 1e3, 1)
    # the whole shard's step 1 (its values: the seeded sample repeated)
    full = (np.resize(sample_p, sl), np.zeros(sl, np.float32), np.zeros(sl, np.float32),
            np.resize(sample_g, sl))
    z2["whole_shard_step1_ms_all_threads"] = round(
        _adamw_points_timed(oracle, full, hp, 1, T) * 1e3, 1)
    del full
    configs["zero2_adamw_shard"] = z2

    # --- Muon shares: one matrix per shape
    for w, key in ((wl.LLAMA1B_MUON, "llama1b_rank0_muon"), (wl.LLAMA8B_MUON, "llama8b_rank0_muon")):
        total, per_shape = _muon_one_per_shape(oracle, wl, w, T)
        configs[key] = dict(
            ms_per_step_extrapolated=round(total * 1e3, 1), threads=T, extrapolated=True,
            sample=("one matrix per distinct stored shape through the whole Muon step with no "
                    "iteration (t0), and one float64 Newton-Schulz iteration (t_it) per distinct "
                    "Newton-Schulz shape; per matrix t0 + 5 t_it, times the group's matrix "
                    "count"),
            per_shape=per_shape)

    return dict(value=round(head_ms, 1), unit="ms per optimizer step", cores=T, kind="oracle",
                sample=("the whole headline step, not extrapolated: AdamW over 38,652,672 "
                        f"elements in scalar C split over {T} threads "
                        f"({adamw_s[T] * 1e3:.0f} ms; {adamw_s[1] * 1e3:.0f} ms on 1 thread), "
                        f"72 Muon matrices with float64 Newton-Schulz through numpy BLAS on {T} "
                        f"threads ({muon_s * 1e3:.0f} ms)"),
                cpu_model=_cpu_model(), host_cpus=os.cpu_count(), configs=configs)


def main():
    args = parse()
    PLAIN_FORM_AB[0] = not args.no_plain_form
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's optimizer step on one GPU; runs on more than "
              "one GPU are not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    import sharded_optimizer_step_adamw_amd as z
    z.lib()  # fails loudly if libzopt.so is not built
    dev = torch.device("cuda:0")
    timer = Timer(torch)
    parts = set(args.parts.split(","))
    K, W = args.steps, args.warmup
    out = dict(metric=METRIC)
    res_step = bench_step(torch, z, timer, dev, K, W) if "step" in parts else None
    res_adamw = (bench_adamw(torch, z, timer, dev, max(K, 100), W, clip_leg="clip" in parts)
                 if "adamw" in parts else None)
    res_ns = bench_ns(torch, z, timer, dev, max(2, K // 5), W) if "ns" in parts else None
    if "ns" in parts:
        import workloads as wl
        res_ns1b = bench_ns(torch, z, timer, dev, K, W, wl.LLAMA1B_MUON)
    else:
        res_ns1b = None
    res_tiny = bench_tiny(torch, z, timer, dev, K, W) if "tiny" in parts else None
    res_copy = bench_copy(torch, z, timer, dev, K, W) if "copy" in parts else None
    res_graph = bench_graph(torch, z, timer, dev, K, W) if "graph" in parts else None
    if res_step:
        tf = res_step["ns_flops"] / res_step["ns_ms"] / 1e9
        out.update(value=round(res_step["ms"], 4), unit="ms per optimizer step")
        roof = dict(
            kernel=("Newton-Schulz of the Muon call (72 matrices, 5 steps) on two streams: the "
                    "48 x [768, 768] group in plain iterations (ns_gemm_kernel<256> X X^T and P, "
                    "ns_bx_kernel<256> P X) on one, the 3072 x 768 and 768 x 3072 groups in Gram "
                    "segments of 3 and 2 steps (X X^T, fp16 m x m chain on ns_gemm_kernel<256>, "
                    "ns_bx_kernel<256> Q X) on the other"),
            bound="mfma", achieved=round(tf, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
            frac=round(tf / BF16_PEAK_TFLOPS, 4), traffic=measured_traffic("ns_call_gpt2"),
            traffic_unit="HBM bytes per 5-step call (all NS launches)",
            algorithmic_flops_per_unit=res_step["ns_flops"],
            avg_unit_ms=round(res_step["ns_ms"], 4),
            unit_time=("HIP-event time of the 5-step Muon call less that of the call with no "
                       "steps; with two streams this credits to the iterations the overlap of one "
                       "stream's pre-passes and post-steps with the other's iterations, so it is "
                       "shorter than the traced span of the NS launches"))
    else:
        roof = None
    out.update(n_gpus=1, steps=K, warmup=W,
               ms_per_step=out.get("value"), higher_is_better=False, scaling="weak",
               vs_baseline=None, dtype="fp32+bf16", data="synthetic",
               config=dict(workload=("gpt2-small optimizer step, world 1: AdamW on 50304x768 "
                                     "embedding + 25x768 vectors (2 calls), Muon on 12 layers "
                                     "x {4x768x768, 3072x768, 768x3072} (1 call, 3 groups), "
                                     "5 bf16 Newton-Schulz iterations"),
                           adamw_elements=38_652_672, muon_matrices=72),
               roofline=roof)
    if res_step:
        out["step_detail"] = dict(adamw_ms=round(res_step["adamw_ms"], 4),
                                  adamw_gbs=round(res_step["adamw_gbs"], 1),
                                  muon=res_step["muon"])
    if res_adamw:
        out["adamw_shard"] = res_adamw
    if res_ns:
        out["newton_schulz"] = res_ns
    if res_ns1b:
        out["newton_schulz_1b"] = res_ns1b
    if res_tiny:
        out["tiny"] = res_tiny
    if res_copy:
        out["round_bf16_calibration"] = res_copy
    if res_graph:
        out["muon_graph"] = res_graph
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline()
    props = torch.cuda.get_device_properties(0)
    out["device"] = f"{torch.cuda.get_device_name(0)} ({getattr(props, 'gcnArchName', '?')}, " \
                    f"{props.multi_processor_count} CUs)"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
