"""GPU parity of the clipping calls against the oracle: zopt_grad_sq_norm,
zopt_grad_clip_stats and zopt_adamw_shard_step_clipped.

The bars:
  * the sum of squares within 1e-10 relative of the oracle's.  The GPU adds
    exact squares in double along per-thread runs of at most a few hundred
    terms and two workgroup trees (error below 1e3 * 2^-53 of the sum); the
    oracle adds them in long double in index order (below n * 2^-64, 1.4e-11
    at n = 2.5e8);
  * the clip statistics bit for bit as the oracle derives them from the
    GPU's own sum (teacher-forced: the same binary32 operations), and the
    total norm within one ulp, the coefficient within two, the flags equal,
    from the oracle's own sum;
  * the clipped AdamW step bit for bit as the oracle's AdamW with grad_scale
    set to the statistics' value, and as zopt_adamw_shard_step given that
    value; with skip_nonfinite a found_inf leaves every output untouched.
Layouts span padding, odd buckets, several ranks, unaligned bases (the
element-wise path) and the 2.0e9-element ZeRO-2 rank-3 shard.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
SQ_RTOL = 1e-10


def f32(x):
    return float(np.float32(x))


def u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_bf16(bits: np.ndarray, off: int = 0) -> torch.Tensor:
    b = np.concatenate([np.zeros(off, np.uint16), bits])
    return torch.from_numpy(b.view(np.int16).copy()).to(DEV).view(torch.bfloat16)[off:]


def owned_mask(n, bucket, world, rank):
    sl = oracle.shard_len(n, bucket, world)
    flat, real = oracle.shard_index_map(n, bucket, world, rank, np.arange(sl))
    owned = np.zeros(n, bool)
    owned[flat[real]] = True
    return owned


def grads(rng, n, std=1e-3, outliers=True):
    g = rng.standard_normal(n) * std
    if outliers:
        g[rng.random(n) < 0.01] *= 100.0
    return wl.to_bf16_bits(g.astype(np.float32))


def check_stats_teacher_forced(sq_dev, stats_dev, max_norm, inv_scale):
    want = oracle.clip_stats(sq_dev.cpu().numpy(), max_norm, inv_scale)
    got = stats_dev.cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def ulps(a, b):
    a, b = np.float32(a), np.float32(b)
    return abs(int(a.view(np.int32)) - int(b.view(np.int32)))


@pytest.mark.parametrize("n,bucket,world,rank,off", [
    (1_048_576, 262_144, 4, 0, 0),     # the tiny AdamW workload
    (1_048_576, 262_144, 4, 3, 0),
    (4103, 1000, 4, 2, 0),             # padded last bucket
    (5000, 333, 8, 7, 0),              # adjusted bucket 328
    ((1 << 14) + 3, 1 << 12, 8, 0, 0),
    (3, 8, 4, 3, 0),                   # a shard of padding only
    (1, 1, 1, 0, 0),
    (100_003, 4096, 1, 0, 0),          # ragged tail
    (1 << 22, 1 << 19, 8, 5, 0),       # vector path, several tiles per workgroup
    (40_000_000, 1 << 25, 1, 0, 0),    # more tiles than workgroups, last bucket ragged
    (1 << 16, 1 << 13, 4, 1, 3),       # unaligned gradient base: element-wise path
])
def test_sq_norm_and_stats_match_oracle(n, bucket, world, rank, off):
    rng = np.random.default_rng(n + rank + off)
    g = grads(rng, n)
    owned = owned_mask(n, bucket, world, rank)
    g_poison = np.where(owned, g, np.uint16(0x7FC0)).astype(np.uint16)  # stray reads show as NaN
    gg = to_dev_bf16(g_poison, off)
    sq = z.grad_sq_norm(gg, n, bucket, world, rank)
    want = oracle.grad_sq_norm(g_poison, n, bucket, world, rank)
    got = float(sq.item())
    assert np.isfinite(got)
    assert abs(got - want) <= SQ_RTOL * want, (got, want)
    for max_norm, inv_scale in ((1.0, 1.0), (1e-4, 1.0), (1e9, 1.0), (0.05, 0.25),
                                (float("inf"), 1.0)):
        st = z.grad_clip_stats(sq, max_norm, inv_scale)
        check_stats_teacher_forced(sq, st, max_norm, inv_scale)
        own = oracle.clip_stats([want], max_norm, inv_scale)
        s = st.cpu().numpy()
        assert ulps(s[0], own[0]) <= 1 and ulps(s[1], own[1]) <= 2
        assert s[2] == own[2] and s[3] == own[3]


def test_sq_norm_is_run_to_run_identical():
    n = 10_000_019
    g = grads(np.random.default_rng(1), n)
    gg = to_dev_bf16(g)
    a = [z.grad_sq_norm(gg, n, 1 << 22, 1, 0).item() for _ in range(3)]
    assert a[0] == a[1] == a[2]


def test_stats_from_several_partials():
    rng = np.random.default_rng(4)
    parts = rng.random(37) * 10.0 ** rng.integers(-6, 6, 37)
    sq = torch.from_numpy(parts).to(DEV)
    for max_norm in (1.0, 100.0, 1e6):
        st = z.grad_clip_stats(sq, max_norm)
        check_stats_teacher_forced(sq, st, max_norm, 1.0)


@pytest.mark.parametrize("kind", ["inf", "-inf", "nan", "overflow", "zero"])
def test_special_gradients(kind):
    n = 50_000
    g = grads(np.random.default_rng(2), n)
    if kind == "inf":
        g[777] = 0x7F80
    elif kind == "-inf":
        g[n - 1] = 0xFF80
    elif kind == "nan":
        g[5] = 0x7FC0
    elif kind == "overflow":
        g[100:104] = 0x7F00          # 2^127: the norm overflows binary32, not double
    else:
        g[:] = 0
    gg = to_dev_bf16(g)
    sq = z.grad_sq_norm(gg, n, 8192, 1, 0)
    want = oracle.grad_sq_norm(g, n, 8192, 1, 0)
    got = sq.item()
    if np.isfinite(want):
        assert abs(got - want) <= SQ_RTOL * want
    else:
        assert np.isnan(got) == np.isnan(want) and np.isinf(got) == np.isinf(want)
    st = z.grad_clip_stats(sq, 1.0)
    check_stats_teacher_forced(sq, st, 1.0, 1.0)
    s = st.cpu().numpy()
    assert s[z.CLIP_FOUND_INF] == (0.0 if kind == "zero" else 1.0)
    assert s[z.CLIP_CLIPPED] == 0.0


def clipped_vs_oracle(n, bucket, world, rank, steps, seed, max_norm, off=0, weight=True,
                      skip=False, hp=HP):
    """Norm -> stats -> clipped AdamW on the GPU for `steps` steps; the oracle
    steps with grad_scale = the statistics' value; the host-scale GPU entry
    point steps a second copy with the same value.  All bitwise."""
    rng = np.random.default_rng(seed)
    sl = oracle.shard_len(n, bucket, world)
    owned = owned_mask(n, bucket, world, rank)
    p = (rng.standard_normal(sl) * 0.02).astype(np.float32)
    m, v = np.zeros(sl, np.float32), np.zeros(sl, np.float32)
    w = np.full(n, 0x5A5A, np.uint16)
    gp = torch.from_numpy(p.copy()).to(DEV)
    gm, gv = torch.zeros_like(gp), torch.zeros_like(gp)
    hp2 = (gp.clone(), gm.clone(), gv.clone())
    gw = to_dev_bf16(w) if weight else None
    gw2 = to_dev_bf16(w) if weight else None
    hps = {k: f32(x) for k, x in hp.items()}
    for t in range(1, steps + 1):
        g = grads(rng, n)
        g = np.where(owned, g, np.uint16(0x7FC0)).astype(np.uint16)
        gg = to_dev_bf16(g, off)
        sq = z.grad_sq_norm(gg, n, bucket, world, rank)
        st = z.grad_clip_stats(sq, max_norm)
        z.adamw_shard_step_clipped(gp, gm, gv, gg, gw, n, bucket, world, rank, step=t,
                                   clip_stats=st, skip_nonfinite=skip, **hps)
        scale = float(st[z.CLIP_GRAD_SCALE].item())
        z.adamw_shard_step(*hp2, gg, gw2, n, bucket, world, rank, step=t, grad_scale=scale, **hps)
        oracle.adamw_shard_step(p, m, v, np.where(owned, g, 0).astype(np.uint16),
                                w if weight else None, n, bucket, world, rank, hps["lr"],
                                hps["beta1"], hps["beta2"], hps["eps"], hps["weight_decay"], t,
                                scale)
    torch.cuda.synchronize()
    for got, got2, want in ((gp, hp2[0], p), (gm, hp2[1], m), (gv, hp2[2], v)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
        np.testing.assert_array_equal(got2.cpu().numpy().view(np.uint32), want.view(np.uint32))
    if weight:
        np.testing.assert_array_equal(u16(gw), w)
        np.testing.assert_array_equal(u16(gw2), w)
        assert np.all(w[~owned] == 0x5A5A)
    return st


@pytest.mark.parametrize("n,bucket,world,rank,max_norm,off", [
    (1_048_576, 262_144, 4, 0, 0.05, 0),   # clipped (the share's norm is about 5)
    (1_048_576, 262_144, 4, 2, 100.0, 0),  # not clipped: grad_scale 1
    (4103, 1000, 4, 2, 0.01, 0),
    (5000, 333, 8, 7, 0.001, 0),
    (1 << 16, 1 << 13, 4, 1, 0.02, 5),     # unaligned gradient base
])
def test_clipped_adamw_bitwise(n, bucket, world, rank, max_norm, off):
    st = clipped_vs_oracle(n, bucket, world, rank, 3, seed=n + rank, max_norm=max_norm, off=off)
    s = st.cpu().numpy()
    assert s[z.CLIP_CLIPPED] == (1.0 if max_norm < 0.5 else 0.0)


def test_clipped_adamw_no_weight_and_skip_flag_on_finite():
    clipped_vs_oracle(70_001, 8192, 2, 1, 2, seed=3, max_norm=0.01, weight=False, skip=True)


@pytest.mark.parametrize("skip", [True, False])
def test_found_inf_skip_leaves_outputs(skip):
    n, bucket, world, rank = 20_000, 4096, 2, 1
    rng = np.random.default_rng(8)
    sl = oracle.shard_len(n, bucket, world)
    owned = owned_mask(n, bucket, world, rank)
    g = grads(rng, n)
    first = int(np.flatnonzero(owned)[10])
    g[first] = 0x7F80                       # +inf in this rank's share
    gg = to_dev_bf16(g)
    p = (rng.standard_normal(sl) * 0.02).astype(np.float32)
    gp = torch.from_numpy(p.copy()).to(DEV)
    gm, gv = torch.full_like(gp, 1e-4), torch.full_like(gp, 1e-6)
    gw = to_dev_bf16(np.full(n, 0x5A5A, np.uint16))
    sq = z.grad_sq_norm(gg, n, bucket, world, rank)
    st = z.grad_clip_stats(sq, 1.0)
    assert st[z.CLIP_FOUND_INF].item() == 1.0
    z.adamw_shard_step_clipped(gp, gm, gv, gg, gw, n, bucket, world, rank, step=1,
                               clip_stats=st, skip_nonfinite=skip, **HP)
    torch.cuda.synchronize()
    if skip:
        np.testing.assert_array_equal(gp.cpu().numpy().view(np.uint32), p.view(np.uint32))
        assert bool((gm == 1e-4).all()) and bool((gv == 1e-6).all())
        assert np.all(u16(gw) == 0x5A5A)
    else:
        # grad_scale 0 (an infinite norm): inf * 0 is NaN at that element, the
        # rest step with a zero gradient -- exactly the oracle's step at scale 0
        m, v = np.full(sl, 1e-4, np.float32), np.full(sl, 1e-6, np.float32)
        w = np.full(n, 0x5A5A, np.uint16)
        oracle.adamw_shard_step(p, m, v, np.where(owned, g, 0).astype(np.uint16), w, n, bucket,
                                world, rank, *(f32(HP[k]) for k in
                                               ("lr", "beta1", "beta2", "eps", "weight_decay")),
                                1, 0.0)
        for got, want in ((gp, p), (gm, m), (gv, v)):
            got = got.cpu().numpy()
            nan = np.isnan(want)
            assert nan.sum() == 1 and np.array_equal(np.isnan(got), nan)
            np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
        np.testing.assert_array_equal(u16(gw), w)


def test_zero2_full_size_norm_and_clipped_step():
    """N = 2.0e9, bucket 1 << 25, world 8, rank 3, in the launch configuration
    the benchmark times: the norm of the whole 2.5e8-element share against
    the oracle's, the statistics teacher-forced, and one clipped step on a
    seeded sample of 1,048,576 shard elements stepped by the oracle."""
    w8 = wl.ZERO2_ADAMW
    part = w8.parts[0]
    n, sl = part.n, z.shard_len(part.n, part.bucket, part.world)
    gg = wl.device_grad_bf16(w8.wid, 1, (n,), w8.grad_std, DEV, step=1)
    sq = z.grad_sq_norm(gg, n, part.bucket, part.world, part.rank)
    g_host = u16(gg)
    want = oracle.grad_sq_norm(g_host, n, part.bucket, part.world, part.rank)
    del g_host
    got = sq.item()
    assert abs(got - want) <= SQ_RTOL * want, (got, want)
    st = z.grad_clip_stats(sq, 1.0)
    check_stats_teacher_forced(sq, st, 1.0, 1.0)
    assert st[z.CLIP_CLIPPED].item() == 1.0          # the norm is ~15.8
    rng = np.random.default_rng(77)
    j = np.unique(rng.integers(0, sl, 1 << 20)).astype(np.int64)
    flat, real = oracle.shard_index_map(n, part.bucket, part.world, part.rank, j)
    assert real.all()
    gp = wl.device_normal(w8.wid, 0, (sl,), w8.master_std, DEV)
    gm, gv = torch.zeros_like(gp), torch.zeros_like(gp)
    gw = torch.zeros((n,), dtype=torch.bfloat16, device=DEV)
    jt, ft = torch.from_numpy(j).to(DEV), torch.from_numpy(flat).to(DEV)
    p = gp[jt].cpu().numpy()
    m, v = np.zeros_like(p), np.zeros_like(p)
    hps = [f32(x) for x in (part.lr, part.beta1, part.beta2, part.eps, part.weight_decay)]
    z.adamw_shard_step_clipped(gp, gm, gv, gg, gw, n, part.bucket, part.world, part.rank,
                               *hps, 1, st)
    scale = np.float32(st[z.CLIP_GRAD_SCALE].item())
    gs = (oracle.bf16_bits_to_f32(u16(gg[ft])) * scale).astype(np.float32)
    w = oracle.adamw_points(p, m, v, gs, *hps, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gp[jt].cpu().numpy().view(np.uint32), p.view(np.uint32))
    np.testing.assert_array_equal(gm[jt].cpu().numpy().view(np.uint32), m.view(np.uint32))
    np.testing.assert_array_equal(gv[jt].cpu().numpy().view(np.uint32), v.view(np.uint32))
    np.testing.assert_array_equal(u16(gw[ft]), w)
