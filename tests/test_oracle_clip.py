"""Pins for the oracle's gradient norm, clip statistics and Newton-Schulz health.

What they compute: the squared L2 norm of the summed gradient a rank holds
[DEG zero.py: ZeroMaster.grad_sq_norm], the clip coefficient
min(1, clip / (norm + 1e-6)) [BluScript trainer source, cross-group global
clipping block], found_inf judged on the norm so an infinite norm reports
found_inf and not clipped [dmuon PR #16, commit "device-tensor stats"], and
the Newton-Schulz health figures: ||O||_F / sqrt(min(rows, cols)) (1 when
healthy) and the guard that refuses an update with an element above 1000
[BluScript trainer source, per-step report, nsrej / nsratio].

Pins, none of which re-types the oracle's arithmetic:
  * the ranks' partial sums add up to the norm of the whole flat vector, and
    positions a rank does not own (other ranks' pieces, padding) may hold NaN
    without changing its sum (a partition of the flat vector);
  * math.fsum of the exact squares (brute force) on small vectors;
  * torch.nn.utils.clip_grad_norm_ on CPU (a library routine): total norm
    and the factor it scales the gradients by;
  * closed forms: 3-4-5, constant vectors, all-ones matrices, semi-orthogonal
    matrices from a QR factorisation (ratio 1) and their multiples;
  * special cases: infinite and NaN gradients, a norm overflowing binary32,
    loss-scale invariance (gradients scaled by 2^k with inv_scale 2^-k give
    the same statistics bit for bit), the guard's edge at exactly 1000.
"""
import math

import numpy as np
import pytest
import torch

import oracle

F32 = np.float32


def bf16(x):
    return oracle.rne_bf16(np.asarray(x, dtype=np.float32))


def exact_sq(bits):
    return math.fsum(float(v) ** 2 for v in oracle.bf16_bits_to_f32(bits).astype(np.float64))


# ----------------------------------------------------------------- norm

@pytest.mark.parametrize("n,bucket,world", [(1000, 64, 4), (37, 7, 3), (4096, 1024, 8),
                                            (5, 100, 8), (777, 777, 1)])
def test_partials_partition_the_flat_vector(n, bucket, world):
    rng = np.random.default_rng(n + world)
    g = bf16(rng.standard_normal(n) * 1e-3)
    whole = exact_sq(g)
    parts = [oracle.grad_sq_norm(g, n, bucket, world, r) for r in range(world)]
    assert math.isclose(math.fsum(parts), whole, rel_tol=1e-15)
    assert math.isclose(oracle.grad_sq_norm(g, n, bucket, 1, 0), whole, rel_tol=1e-15)
    sl = oracle.shard_len(n, bucket, world)
    for r in range(world):
        flat, real = oracle.shard_index_map(n, bucket, world, r, np.arange(sl))
        mine = flat[real]
        poisoned = np.full(n, 0x7FC0, dtype=np.uint16)
        poisoned[mine] = g[mine]
        assert oracle.grad_sq_norm(poisoned, n, bucket, world, r) == parts[r]
        assert math.isclose(parts[r], exact_sq(g[mine]), rel_tol=1e-15)


def test_constant_gradient_closed_form():
    n = 3000
    c = 2.0 ** -10
    g = bf16(np.full(n, c))
    assert oracle.grad_sq_norm(g, n, 512, 1, 0) == n * c * c
    assert oracle.clip_stats([n * c * c], 1.0)[0] == F32(math.sqrt(n) * c)


def test_brute_force_small():
    rng = np.random.default_rng(5)
    for n in (1, 2, 17, 300):
        g = bf16(rng.standard_normal(n) * 10.0 ** rng.integers(-8, 8, n))
        assert math.isclose(oracle.grad_sq_norm(g, n, 64, 1, 0), exact_sq(g), rel_tol=1e-15)


def test_extreme_bf16_values_square_exactly():
    # the largest finite bf16 squared (~1.16e77) and the smallest subnormal
    # squared (2^-266) are both exact in double
    big, tiny = np.uint16(0x7F7F), np.uint16(0x0001)
    g = np.array([big, tiny, big], dtype=np.uint16)
    vb = float(oracle.bf16_bits_to_f32(np.array([big]))[0])
    assert oracle.grad_sq_norm(g, 3, 4, 1, 0) == 2 * vb * vb
    g = np.array([tiny], dtype=np.uint16)
    assert oracle.grad_sq_norm(g, 1, 1, 1, 0) == 2.0 ** -266


# ----------------------------------------------------------------- stats

def test_three_four_five():
    st = oracle.clip_stats([25.0], 1.0)
    total_norm, coef, clipped, found_inf, scale = st
    assert total_norm == 5.0
    assert abs(coef - 1.0 / (5.0 + 1e-6)) <= np.spacing(F32(0.2))
    assert clipped == 1.0 and found_inf == 0.0 and scale == coef
    st = oracle.clip_stats([25.0], 10.0)
    assert st[1] == 1.0 and st[2] == 0.0 and st[4] == 1.0


@pytest.mark.parametrize("max_norm,scale", [(1.0, 1.0), (0.05, 1.0), (100.0, 1.0), (0.5, 3.0)])
def test_matches_torch_clip_grad_norm(max_norm, scale):
    rng = np.random.default_rng(17)
    shapes = [(64, 33), (1000,), (7, 7, 3)]
    gs = [bf16(rng.standard_normal(s) * 0.01 * scale) for s in shapes]
    f32 = [oracle.bf16_bits_to_f32(g.ravel()).reshape(g.shape) for g in gs]
    params = [torch.nn.Parameter(torch.zeros(s, dtype=torch.float64)) for s in shapes]
    for p, g in zip(params, f32):
        p.grad = torch.from_numpy(g.astype(np.float64)).clone()
    tn = float(torch.nn.utils.clip_grad_norm_(params, max_norm))
    factor = float(params[0].grad.reshape(-1)[np.argmax(np.abs(f32[0]))] /
                   float(f32[0].reshape(-1)[np.argmax(np.abs(f32[0]))]))
    flat = np.concatenate([g.ravel() for g in gs])
    st = oracle.clip_stats([oracle.grad_sq_norm(flat, flat.size, 4096, 1, 0)], max_norm)
    assert abs(st[0] - tn) <= 2 * np.spacing(F32(tn))
    assert abs(st[1] - factor) <= 4 * np.spacing(F32(factor))
    assert st[2] == (1.0 if tn > max_norm else 0.0)


def test_partial_sums_add_in_order():
    parts = [2.0 ** -3, 2.0 ** -5, 1.0, 0.25]     # dyadic: every order is exact
    assert np.array_equal(oracle.clip_stats(parts, 0.5), oracle.clip_stats([sum(parts)], 0.5))


def test_loss_scale_invariance():
    rng = np.random.default_rng(23)
    g = rng.standard_normal(4096).astype(np.float32) * 1e-3
    base = bf16(g)
    for k in (1, 7, 15):
        scaled = bf16(oracle.bf16_bits_to_f32(base) * F32(2.0 ** k))   # exact power-of-two scaling
        a = oracle.clip_stats([oracle.grad_sq_norm(base, 4096, 4096, 1, 0)], 0.01)
        b = oracle.clip_stats([oracle.grad_sq_norm(scaled, 4096, 4096, 1, 0)], 0.01, 2.0 ** -k)
        assert np.array_equal(a[:4], b[:4])
        assert b[4] == F32(F32(2.0 ** -k) * a[1])


@pytest.mark.parametrize("bad", [np.inf, -np.inf])
def test_infinite_gradient_found_inf_not_clipped(bad):
    g = bf16([1.0, bad, 2.0])
    sq = oracle.grad_sq_norm(g, 3, 8, 1, 0)
    total_norm, coef, clipped, found_inf, scale = oracle.clip_stats([sq], 1.0)
    assert np.isinf(total_norm) and found_inf == 1.0 and clipped == 0.0
    assert coef == 0.0 and scale == 0.0


def test_nan_gradient_found_inf():
    g = np.array([0x3F80, 0x7FC0], dtype=np.uint16)
    st = oracle.clip_stats([oracle.grad_sq_norm(g, 2, 8, 1, 0)], 1.0)
    assert np.isnan(st[0]) and np.isnan(st[1]) and st[2] == 0.0 and st[3] == 1.0


def test_norm_overflowing_binary32_is_found_inf():
    # four elements of 2^127: the norm 2^128 is finite in double, not in binary32
    g = bf16(np.full(4, 2.0 ** 127))
    sq = oracle.grad_sq_norm(g, 4, 4, 1, 0)
    assert sq == 4 * 2.0 ** 254
    st = oracle.clip_stats([sq], 1.0)
    assert np.isinf(st[0]) and st[3] == 1.0 and st[2] == 0.0


def test_zero_gradient():
    st = oracle.clip_stats([0.0], 1.0)
    assert st[0] == 0.0 and st[1] == 1.0 and st[2] == 0.0 and st[3] == 0.0 and st[4] == 1.0


# ----------------------------------------------------------------- NS health

@pytest.mark.parametrize("rows,cols", [(8, 16), (16, 8), (64, 64), (33, 100), (1, 7)])
def test_health_ratio_of_semi_orthogonal_is_one(rows, cols):
    rng = np.random.default_rng(rows * cols)
    m, n = min(rows, cols), max(rows, cols)
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))      # n x m, orthonormal columns
    o = (q.T if rows <= cols else q).astype(np.float32)
    assert o.shape == (rows, cols)
    ratio, amax, rej = oracle.ns_health(o)
    assert abs(ratio - 1.0) < 1e-6 and rej == 0.0
    assert amax == np.abs(o).max()
    r3, _, _ = oracle.ns_health(3.0 * o)
    assert abs(r3 - 3.0) < 3e-6


def test_health_all_ones_closed_form():
    o = np.ones((2, 8), dtype=np.float32)
    assert oracle.ns_health(o)[0] == F32(math.sqrt(8.0))


def test_guard_edge_and_non_finite():
    o = np.zeros((4, 6), dtype=np.float32)
    o[1, 2] = 1000.0
    assert oracle.ns_health(o)[2] == 0.0
    o[1, 2] = np.nextafter(F32(1000.0), F32(np.inf))
    assert oracle.ns_health(o)[2] == 1.0
    o[1, 2] = -1001.0
    assert oracle.ns_health(o)[2] == 1.0
    o[1, 2] = np.nan
    h = oracle.ns_health(o)
    assert h[2] == 1.0 and np.isnan(h[1])
    o[1, 2] = np.inf
    assert oracle.ns_health(o)[2] == 1.0
    o[1, 2] = 5.0
    assert oracle.ns_health(o, guard=4.0)[2] == 1.0 and oracle.ns_health(o, guard=5.0)[2] == 0.0


def test_call_health_counts_and_worst_passed_ratio():
    rng = np.random.default_rng(3)
    q, _ = np.linalg.qr(rng.standard_normal((12, 4)))
    ok1 = q.T.astype(np.float32)                      # ratio 1
    ok3 = (3.0 * q.T).astype(np.float32)              # ratio 3
    bad = np.full((4, 12), 10.0, dtype=np.float32)
    bad[0, 0] = 2000.0                                # rejected, ratio far above 3
    rejected, worst, rows = oracle.ns_call_health([ok1, bad, ok3])
    assert rejected == 1 and abs(worst - 3.0) < 3e-6
    assert list(rows[:, 2]) == [0.0, 1.0, 0.0]
    rejected, worst, _ = oracle.ns_call_health([bad])
    assert rejected == 1 and worst == 0.0


def test_guarded_muon_step_leaves_master_when_rejected():
    rng = np.random.default_rng(9)
    p = (rng.standard_normal((8, 16)) * 0.02).astype(np.float32)
    m = np.zeros((8, 16), np.float32)
    g = bf16(rng.standard_normal((8, 16)) * 1e-3)
    o = np.full((8, 16), 1e4, dtype=np.float32)
    p0 = p.copy()
    w, _ = oracle.muon_step(p, m, g, 1e-3, 0.95, True, 0.1, o_override=o, guard=1000.0)
    assert w is None and np.array_equal(p, p0) and np.any(m != 0)
    w, _ = oracle.muon_step(p, m, g, 1e-3, 0.95, True, 0.1, o_override=o / 1e4, guard=1000.0)
    assert w is not None and not np.array_equal(p, p0)
