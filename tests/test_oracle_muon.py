"""Pins for the oracle's Muon: momentum pre-step, Newton-Schulz, post-step.

Muon's step on a whole matrix [BluScript trainer source, ShardedMuon comment
block and Muon config block]: a momentum EMA with Nesterov look-ahead
(momentum 0.95), Newton-Schulz orthogonalisation X <- aX + (bXX' + c(XX')^2)X
(5 iterations) of the Frobenius-pre-scaled update, then a decayed, scaled
update of the fp32 master (weight decay pinned to AdamW's, the update RMS
lifted to 0.2 under the match-AdamW convention).

Pins:
  * Newton-Schulz acts on the singular values as the scalar polynomial
    phi(s) = a s + b s^3 + c s^5 iterated: checked for U diag(s) V^T inputs
    (numpy QR orthogonal factors; repeated, tiny, zero singular values), for
    diagonal inputs, and against a pure-Python triple-loop run on 8 x 16;
  * invariances: positive scaling, transposition, negation, zero input;
  * momentum: step-1 closed form and a constant gradient's closed form
    M_t = (1 - mu^t) g (the EMA form; the SGD form would give another value);
  * post-step: float64 closed form, the printed 4.5x / 21.2x convention
    ratios, and entry RMS 0.2 of the scaled update of an orthogonal matrix.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
A, B, C = oracle.NS_COEFFS


def orthogonal(rng, k):
    q, r = np.linalg.qr(rng.standard_normal((k, k)))
    return q * np.sign(np.diag(r))


def closed_form(u, vt, sigma, steps=5):
    s_hat = sigma / (np.linalg.norm(sigma) + oracle.NS_EPS)
    return (u[:, :len(sigma)] * oracle.ns_scalar_map(s_hat, steps)) @ vt[:len(sigma)]


def test_scalar_map_values():
    # phi(1) = a + b + c; phi(0) = 0; the map is odd
    assert abs(oracle.ns_scalar_map(1.0, 1) - (A + B + C)) < 1e-15
    assert abs(A + B + C - 0.701) < 1e-12
    assert oracle.ns_scalar_map(0.0, 5) == 0.0
    x = np.linspace(0.01, 1, 50)
    assert np.max(np.abs(oracle.ns_scalar_map(-x) + oracle.ns_scalar_map(x))) < 1e-14


@pytest.mark.parametrize("m,n", [(8, 16), (16, 8), (12, 12), (5, 40), (64, 96)])
@pytest.mark.parametrize("spectrum", ["spread", "repeated", "tiny_and_zero", "equal"])
def test_ns_is_scalar_polynomial_on_singular_values(m, n, spectrum):
    rng = np.random.default_rng(m * 1000 + n)
    k = min(m, n)
    sigma = {
        "spread": np.geomspace(1.0, 1e-3, k),
        "repeated": np.repeat([2.0, 0.5], [k // 2, k - k // 2]),
        "tiny_and_zero": np.concatenate([[1.0, 0.3], np.full(k - 4, 1e-6), [0.0, 0.0]])
        if k >= 4 else np.array([1.0, 0.0][:k]),
        "equal": np.ones(k),
    }[spectrum]
    u, v = orthogonal(rng, m), orthogonal(rng, n)
    g = (u[:, :k] * sigma) @ v.T[:k]
    got = oracle.newton_schulz(g)
    want = closed_form(u, v.T, sigma)
    assert got.shape == (m, n)
    assert np.max(np.abs(got - want)) < 1e-12


def test_ns_diagonal_input():
    sigma = np.array([3.0, 1.0, 0.25, 0.0, 1e-4])
    g = np.zeros((5, 9))
    g[np.arange(5), np.arange(5)] = sigma
    got = oracle.newton_schulz(g)
    want = np.zeros((5, 9))
    want[np.arange(5), np.arange(5)] = oracle.ns_scalar_map(
        sigma / (np.linalg.norm(sigma) + oracle.NS_EPS))
    assert np.max(np.abs(got - want)) < 1e-14


def naive_ns(g, steps=5):
    """Pure-Python loops: transpose so rows <= cols, pre-scale, iterate."""
    rows = [list(map(float, r)) for r in g]
    tr = len(rows) > len(rows[0])
    if tr:
        rows = [list(c) for c in zip(*rows)]
    m, n = len(rows), len(rows[0])
    norm = math.sqrt(sum(x * x for r in rows for x in r)) + 1e-7
    x = [[e / norm for e in r] for r in rows]
    for _ in range(steps):
        a_ = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)]
              for i in range(m)]
        aa = [[sum(a_[i][t] * a_[t][j] for t in range(m)) for j in range(m)]
              for i in range(m)]
        b_ = [[B * a_[i][j] + C * aa[i][j] for j in range(m)] for i in range(m)]
        x = [[A * x[i][j] + sum(b_[i][t] * x[t][j] for t in range(m))
              for j in range(n)] for i in range(m)]
    if tr:
        x = [list(c) for c in zip(*x)]
    return np.array(x)


@pytest.mark.parametrize("shape", [(8, 16), (16, 8)])
def test_ns_brute_force_small(shape):
    rng = np.random.default_rng(21)
    g = rng.standard_normal(shape)
    assert np.max(np.abs(oracle.newton_schulz(g) - naive_ns(g))) < 1e-12


def test_ns_invariances():
    rng = np.random.default_rng(22)
    g = rng.standard_normal((24, 40))
    o = oracle.newton_schulz(g)
    # scaling is exact once eps scales with it; with a fixed eps it moves the
    # result only by about eps / ||g||
    assert np.allclose(oracle.newton_schulz(37.5 * g, eps=37.5e-7), o, rtol=0, atol=1e-12)
    assert np.allclose(oracle.newton_schulz(37.5 * g), o, rtol=0, atol=1e-6)
    assert np.allclose(oracle.newton_schulz(g.T), o.T, rtol=0, atol=1e-12)
    assert np.allclose(oracle.newton_schulz(-g), -o, rtol=0, atol=0)
    assert not oracle.newton_schulz(np.zeros((6, 10))).any()
    # five quintic steps leave the singular values near 1 (not exactly 1)
    s = np.linalg.svd(o, compute_uv=False)
    assert np.all((s > 0.5) & (s < 1.3))


def test_ns_steps_zero_is_the_prescale():
    rng = np.random.default_rng(23)
    g = rng.standard_normal((7, 3))
    want = g / (np.linalg.norm(g) + 1e-7)
    assert np.allclose(oracle.newton_schulz(g, steps=0), want, rtol=0, atol=1e-15)


# ------------------------------------------------------------- momentum

def bf16(rng, shape, std=1e-3):
    return oracle.rne_bf16((rng.standard_normal(shape) * std).astype(np.float32))


def test_momentum_step1_closed_form():
    rng = np.random.default_rng(31)
    gb = bf16(rng, (64, 32))
    g = oracle.bf16_bits_to_f32(gb).astype(np.float64)
    for mu in (0.95, 0.9, 0.0):
        mu = float(np.float32(mu))   # the oracle takes mu as binary32
        mom = np.zeros((64, 32), np.float32)
        u = oracle.muon_pre(mom, gb, mu, nesterov=True)
        assert np.all(np.abs(mom - (1 - mu) * g) <= 2 * np.spacing(np.abs(mom)))
        want_u = (1 - mu) * g + mu * (1 - mu) * g
        assert np.all(np.abs(u - want_u) <= 4 * np.spacing(np.abs(u).astype(np.float32)))
    # at step 1 the pre-scaled update does not depend on mu or on nesterov
    # (exactly so without the eps of the pre-scale, which is 1e-7 absolute)
    outs = []
    for mu, nest in ((0.95, True), (0.5, True), (0.95, False)):
        mom = np.zeros((64, 32), np.float32)
        outs.append(oracle.frobenius_prescale(oracle.muon_pre(mom, gb, mu, nest), eps=0.0))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-6 * np.max(np.abs(outs[0]))


def test_constant_gradient_momentum_is_an_ema():
    rng = np.random.default_rng(32)
    gb = bf16(rng, (16, 16))
    g = oracle.bf16_bits_to_f32(gb).astype(np.float64)
    mu = float(np.float32(0.95))
    mom = np.zeros((16, 16), np.float32)
    for t in range(1, 11):
        u = oracle.muon_pre(mom, gb, mu, nesterov=True)
        want_m = (1 - mu ** t) * g
        want_u = (1 - mu) * g + mu * want_m
        tol = t * 4 * np.spacing(np.abs(want_m).astype(np.float32))
        assert np.all(np.abs(mom - want_m) <= tol), t
        assert np.all(np.abs(u - want_u) <= 2 * tol), t
        u_plain = oracle.muon_pre(mom.copy(), gb, mu, nesterov=False)
        assert np.all(np.abs(u_plain - (1 - mu ** (t + 1)) * g) <= 2 * tol)


# ------------------------------------------------------------- post-step

def test_adjust_conventions_match_printed_ratios():
    fig = json.load(open(GOLDEN))["muon_adjust_lr_ratio"]
    for name, (rows, cols) in fig["shapes_rows_cols"].items():
        ratio = oracle.muon_scale(rows, cols, 1) / oracle.muon_scale(rows, cols, 0)
        assert round(ratio, fig["printed_decimals"]) == fig["printed_ratio"][name]
        assert abs(ratio - 0.2 * math.sqrt(cols)) < 1e-12


@pytest.mark.parametrize("rows,cols", [(64, 64), (32, 128), (128, 32)])
def test_match_convention_gives_entry_rms_02(rows, cols):
    target = json.load(open(GOLDEN))["match_rms_target"]["entry_rms"]
    rng = np.random.default_rng(rows + cols)
    k = min(rows, cols)
    o = orthogonal(rng, rows)[:, :k] @ orthogonal(rng, cols)[:k]   # all s = 1
    scaled = oracle.muon_scale(rows, cols, 1) * o
    assert abs(np.sqrt(np.mean(scaled ** 2)) - target) < 1e-12


def test_post_step_closed_form():
    rng = np.random.default_rng(41)
    rows, cols = 48, 80
    p0 = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    o = (rng.standard_normal((rows, cols)) * 0.1).astype(np.float32)
    lr, wd = float(np.float32(8e-4)), float(np.float32(0.1))
    for adjust in (0, 1):
        p = p0.copy()
        w = oracle.muon_post(p, o, lr, wd, adjust)
        scale = 0.2 * math.sqrt(max(rows, cols)) if adjust else math.sqrt(max(1, rows / cols))
        want = p0.astype(np.float64) * (1 - lr * wd) - lr * scale * o.astype(np.float64)
        tol = 2 * np.spacing(np.abs(p0)) + 2 * np.spacing(np.float32(lr * scale) * np.abs(o))
        assert np.all(np.abs(p - want) <= tol)
        assert np.array_equal(w, oracle.rne_bf16(p))
    # no step and no decay: nothing moves
    p = p0.copy()
    w = oracle.muon_post(p, o, 0.0, 0.0, 1)
    assert np.array_equal(p, p0) and np.array_equal(w, oracle.rne_bf16(p0))
