"""Pins for the oracle's AdamW over a flat bucketed shard.

What AdamW computes: decoupled weight decay (a (1 - lr*wd) multiply), then the
two moments, then the bias-corrected addcdiv, with the bias corrections as
per-step scalars on the post-increment step [dmuon PR #16, commit "foreach
AdamW"; BluScript trainer source, optimizer-precision note].  eps is added
after the bias correction of the root (the textbook decoupled AdamW).

Pins, none of which re-types the oracle's formula:
  * the step-1 closed form  p1 = p0 (1 - lr wd) - lr g / (|g| + eps),
    m1 = (1 - b1) g, v1 = (1 - b2) g^2  (float64, within a few ulps);
  * a constant gradient: every step applies that same closed form;
  * a zero gradient: the moments stay 0 and p is only decayed;
  * torch.optim.AdamW on CPU (a library routine) over 10 steps;
  * sharded == unsharded: the union of all ranks' shard steps equals the
    world = 1 step bit for bit [DEG zero.py docstring: element-wise AdamW over
    a flat tensor is the same arithmetic as over the separate tensors];
  * bf16 gradients step exactly as their fp32 values, and grad_scale on load
    steps exactly as a gradient scaled beforehand [DeepSpeed PR #9021,
    commits "bf16 gradients of fp32 params" and "grad_scale"].
"""
import numpy as np
import pytest
import torch

import oracle

LR, B1, B2, EPS, WD = (float(np.float32(x)) for x in (1e-3, 0.9, 0.95, 1e-8, 0.1))


def ulp(x):
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)


def bf16_grads(rng, n, std=1e-3):
    g = (rng.standard_normal(n) * std).astype(np.float32)
    return oracle.rne_bf16(g)


def test_scalars_are_rounded_once_from_double():
    sc = oracle.adamw_scalars(LR, B1, B2, WD, 3)
    assert sc[0] == np.float32(LR / (1 - B1 ** 3))
    assert sc[1] == np.float32(np.sqrt(1 - B2 ** 3))
    assert sc[2] == np.float32(1 - LR * WD)
    assert sc[3] == np.float32(1 - B1) and sc[4] == np.float32(1 - B2)


@pytest.mark.parametrize("kind", ["random", "zero", "tiny", "huge", "near_eps"])
def test_step1_closed_form(kind):
    rng = np.random.default_rng(11)
    n = 4096
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = {
        "random": (rng.standard_normal(n) * 1e-3),
        "zero": np.zeros(n),
        "tiny": rng.standard_normal(n) * 1e-30,
        "huge": rng.standard_normal(n) * 1e15,
        "near_eps": rng.standard_normal(n) * 1e-8,
    }[kind].astype(np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.adamw_points(p, m, v, g.copy(), LR, B1, B2, EPS, WD, 1)
    g64, p64 = g.astype(np.float64), p0.astype(np.float64)
    want_p = p64 * (1 - LR * WD) - LR * g64 / (np.abs(g64) + EPS)
    want_m = (1 - B1) * g64
    want_v = (1 - B2) * g64 * g64
    assert np.all(np.abs(p - want_p) <= 3 * ulp(p0) + 4 * ulp(LR))
    assert np.all(np.abs(m - want_m) <= 2 * ulp(want_m))
    if kind != "tiny":  # (1-b2) g^2 underflows for |g| ~ 1e-30
        assert np.all(np.abs(v - want_v) <= 3 * ulp(want_v))


def test_overflowing_second_moment_stops_the_update():
    """Beyond |g| ~ 8e19, (1 - b2) g^2 overflows binary32 to +inf; sqrt(inf)
    is inf, m / inf is 0, and only the decay remains (IEEE propagation, no
    special case)."""
    p = np.array([0.5, -0.25], np.float32)
    m, v = np.zeros(2, np.float32), np.zeros(2, np.float32)
    oracle.adamw_points(p, m, v, np.array([3e20, -3e20], np.float32), LR, B1, B2, EPS,
                        WD, 1)
    assert np.all(np.isinf(v))
    assert np.array_equal(p, np.array([0.5, -0.25], np.float32) * np.float32(1 - LR * WD))


def test_constant_gradient_repeats_the_closed_form():
    """With a constant g, m/bc1 = g and sqrt(v/bc2) = |g| at every step, so
    each step is p <- p (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(12)
    n = 4096
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    want = p.astype(np.float64)
    g64 = g.astype(np.float64)
    for t in range(1, 11):
        oracle.adamw_points(p, m, v, g.copy(), LR, B1, B2, EPS, WD, t)
        want = want * (1 - LR * WD) - LR * g64 / (np.abs(g64) + EPS)
        assert np.all(np.abs(p - want) <= t * (4 * ulp(want) + 8 * ulp(LR))), t


def test_zero_gradient_only_decays():
    rng = np.random.default_rng(13)
    n = 1000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    ref = p.copy()
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    decay = np.float32(1 - LR * WD)
    for t in range(1, 8):
        oracle.adamw_points(p, m, v, np.zeros(n, np.float32), LR, B1, B2, EPS, WD, t)
        ref = ref * decay
        assert np.array_equal(p, ref) and not m.any() and not v.any()
    # and with no decay nothing moves at all
    q = ref.copy()
    oracle.adamw_points(q, m, v, np.zeros(n, np.float32), LR, B1, B2, EPS, 0.0, 9)
    assert np.array_equal(q, ref)


def test_matches_torch_adamw_over_ten_steps():
    rng = np.random.default_rng(14)
    n = 50000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([param], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=WD,
                            foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g_max = np.zeros(n)  # running max |g|: the scale of every moment term
    for t in range(1, 11):
        gf = oracle.bf16_bits_to_f32(bf16_grads(rng, n))
        g_max = np.maximum(g_max, np.abs(gf))
        param.grad = torch.from_numpy(gf.copy())
        opt.step()
        oracle.adamw_points(p, m, v, gf.copy(), LR, B1, B2, EPS, WD, t)
        tp = param.detach().numpy().astype(np.float64)
        st = opt.state[param]
        tm = st["exp_avg"].numpy().astype(np.float64)
        tv = st["exp_avg_sq"].numpy().astype(np.float64)
        # torch forms m with lerp and divides by the root's scalar with a
        # reciprocal multiply: the two agree to a few ulps of the terms per
        # step, while any formula difference (bias correction, eps placement,
        # decay order, beta swap) is orders of magnitude larger
        assert np.all(np.abs(p - tp) <= t * (4 * ulp(tp) + 16 * ulp(LR))), t
        assert np.all(np.abs(m - tm) <= t * 4 * ulp(g_max)), t
        assert np.all(np.abs(v - tv) <= t * 4 * ulp(g_max * g_max)), t
        assert np.max(np.abs(m - tm)) < 1e-6 * np.max(np.abs(tm))


LAYOUTS = [(4096, 1024, 4), (4103, 1000, 4), (5000, 333, 8), (777, 64, 2),
           (1 << 14, 1 << 12, 8), (3, 8, 4), (1000, 1000, 1)]


@pytest.mark.parametrize("n,bucket,world", LAYOUTS)
def test_sharded_equals_unsharded(n, bucket, world):
    rng = np.random.default_rng(n + bucket + world)
    p_full = (rng.standard_normal(n) * 0.02).astype(np.float32)
    # unsharded reference: world = 1 over the whole flat vector
    ref_p, ref_m, ref_v = p_full.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    ref_w = np.zeros(n, np.uint16)
    sl = oracle.shard_len(n, bucket, world)
    shards = []
    for r in range(world):
        flat, real = oracle.shard_index_map(n, bucket, world, r, np.arange(sl))
        sp = np.zeros(sl, np.float32)
        sp[real] = p_full[flat[real]]
        shards.append((flat, real, sp, np.zeros(sl, np.float32), np.zeros(sl, np.float32)))
    w = np.full(n, 0xABCD, np.uint16)
    for t in range(1, 4):
        g = bf16_grads(rng, n)
        oracle.adamw_shard_step(ref_p, ref_m, ref_v, g, ref_w, n, n, 1, 0,
                                LR, B1, B2, EPS, WD, t)
        for r, (flat, real, sp, sm, sv) in enumerate(shards):
            oracle.adamw_shard_step(sp, sm, sv, g, w, n, bucket, world, r,
                                    LR, B1, B2, EPS, WD, t)
    got = np.zeros(n, np.float32)
    for flat, real, sp, sm, sv in shards:
        got[flat[real]] = sp[real]
        assert np.array_equal(sm[real], ref_m[flat[real]])
        assert np.array_equal(sv[real], ref_v[flat[real]])
        # padding saw zero gradients from zero state: it stays zero
        assert not sp[~real].any() and not sm[~real].any() and not sv[~real].any()
    assert np.array_equal(got, ref_p)
    assert np.array_equal(w, ref_w)


def test_non_owned_weights_untouched():
    n, bucket, world, rank = 4103, 1000, 4, 2
    rng = np.random.default_rng(3)
    sl = oracle.shard_len(n, bucket, world)
    flat, real = oracle.shard_index_map(n, bucket, world, rank, np.arange(sl))
    p = (rng.standard_normal(sl) * 0.02).astype(np.float32)
    m, v = np.zeros(sl, np.float32), np.zeros(sl, np.float32)
    w = np.full(n, 0x5A5A, np.uint16)
    oracle.adamw_shard_step(p, m, v, bf16_grads(rng, n), w, n, bucket, world, rank,
                            LR, B1, B2, EPS, WD, 1)
    owned = np.zeros(n, bool)
    owned[flat[real]] = True
    assert np.all(w[~owned] == 0x5A5A)
    assert np.array_equal(w[flat[real]], oracle.rne_bf16(p[real]))


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.37, 3.0e3])
def test_bf16_and_grad_scale_step_as_prescaled_fp32(scale):
    n = 1003  # a scalar tail for any vector width
    rng = np.random.default_rng(5)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    a = [p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    b = [p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    for t in range(1, 4):
        g = bf16_grads(rng, n)
        wa = np.zeros(n, np.uint16)
        oracle.adamw_shard_step(*a, g, wa, n, n, 1, 0, LR, B1, B2, EPS, WD, t,
                                grad_scale=scale)
        pre = oracle.bf16_bits_to_f32(g) * np.float32(scale)
        wb = oracle.adamw_points(*b, pre.astype(np.float32), LR, B1, B2, EPS, WD, t)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        assert np.array_equal(wa, wb)
