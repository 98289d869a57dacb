"""CPU checks of the bf16 rounding model used by the GPU Newton-Schulz tests."""
import numpy as np

import oracle
from ns_bf16_model import newton_schulz_bf16_model


def test_without_rounding_it_is_the_float64_iteration():
    rng = np.random.default_rng(1)
    for shape in ((8, 16), (16, 8), (30, 30)):
        g = rng.standard_normal(shape)
        assert np.max(np.abs(newton_schulz_bf16_model(g, round_bf16=False)
                             - oracle.newton_schulz(g))) < 1e-12


def test_bf16_rounding_error_is_of_the_expected_size():
    rng = np.random.default_rng(2)
    g = rng.standard_normal((64, 256))
    ref = oracle.newton_schulz(g)
    err = np.linalg.norm(newton_schulz_bf16_model(g) - ref) / np.linalg.norm(ref)
    assert 1e-3 < err < 2e-2


def _fp32_products_of_bf16(x):
    """X X^T of bf16(x) with binary32 accumulation, as a matrix core forms it
    (the products of two bf16 values are exact in binary32)."""
    xb = oracle.bf16_bits_to_f32(oracle.rne_bf16(np.asarray(x, np.float32)))
    with np.errstate(over="ignore", invalid="ignore"):
        return xb @ xb.T  # float32 operands: float32 accumulation


def test_folded_prescale_range():
    """The range over which the first iteration may apply s to fp32 products
    of bf16(U) instead of reading bf16(U s): at both ends of [2^-60, 2^100]
    those products are finite and, times s^2, equal X0 X0^T to binary32
    rounding; past the upper end they overflow binary32, which is why the
    pre-step writes X0 = bf16(U s) there."""
    from ns_bf16_model import FOLD_MAX, FOLD_MIN
    rng = np.random.default_rng(5)
    g = rng.standard_normal((64, 256))
    g /= np.linalg.norm(g)
    for total in (FOLD_MIN, FOLD_MAX):
        u = g * np.sqrt(total)
        s = 1.0 / (np.sqrt(total) + oracle.NS_EPS)
        p = _fp32_products_of_bf16(u).astype(np.float64) * (s * s)
        ub = oracle.bf16_bits_to_f32(oracle.rne_bf16(u.astype(np.float32))).astype(np.float64)
        ref = (ub * s) @ (ub * s).T
        assert np.all(np.isfinite(p))
        assert np.max(np.abs(p - ref)) <= 1e-5 * np.max(np.abs(ref))
    # ||U||_F^2 = 2^140: the diagonal of U U^T (about 2^140 / 64 per row) is
    # past binary32's 2^128
    assert np.isinf(_fp32_products_of_bf16(g * 2.0 ** 70)).any()


def test_model_outside_the_folded_range_matches_float64():
    """Huge and tiny gradients, and Inf: the pre-scaled bf16 input keeps the
    bf16 iteration within the tolerance of float64 (the oracle scales in
    float64); an infinite entry gives NaN where the oracle does."""
    rng = np.random.default_rng(6)
    g = rng.standard_normal((48, 160))
    for scale in (1e-30, 1e17, 1e30):
        u = (g * scale).astype(np.float32)
        ref = oracle.newton_schulz(u)
        err = np.linalg.norm(newton_schulz_bf16_model(u) - ref) / np.linalg.norm(ref)
        assert err < 2e-2, (scale, err)
    u = g.astype(np.float32)
    u[3, 7] = np.inf
    with np.errstate(invalid="ignore"):
        assert np.isnan(oracle.newton_schulz(u)).all()
        assert np.isnan(newton_schulz_bf16_model(u)).all()


def test_gram_segments():
    from ns_bf16_model import gram_segments
    assert gram_segments(0) == []
    assert gram_segments(1) == [1]
    assert gram_segments(5) == [3, 2]
    assert gram_segments(4) == [2, 2]
    assert gram_segments(7) == [3, 2, 2]
    assert gram_segments(10) == [3, 3, 2, 2]
    assert all(sum(gram_segments(s)) == s and max(gram_segments(s)) <= 3 for s in range(1, 101))


def test_gram_form_without_rounding_is_the_float64_iteration():
    """The Gram identities (A_{j+1} = P_j^2 A_j, X_L = P_{L-1} ... P_0 X_0)
    reproduce the plain iteration exactly in float64, for every segment
    split, both orientations and several coefficient sets."""
    from ns_bf16_model import newton_schulz_gram_model
    rng = np.random.default_rng(3)
    for shape in ((12, 40), (40, 12), (20, 20)):
        g = rng.standard_normal(shape)
        for steps in (1, 2, 3, 4, 5, 7):
            for coeffs in (oracle.NS_COEFFS, (1.5, -0.5, 0.0), (2.0, -1.5, 0.5)):
                ref = oracle.newton_schulz(g, steps, coeffs)
                got = newton_schulz_gram_model(g, steps, coeffs, chain=None)
                assert np.max(np.abs(got - ref)) < 1e-10, (shape, steps, coeffs)


def _closed_form_input(m, n, sigma, seed):
    rng = np.random.default_rng(seed)
    k = min(m, n)
    qu, _ = np.linalg.qr(rng.standard_normal((m, m)))
    qv, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return (qu[:, :k] * sigma) @ qv.T[:k]


def test_fp16_chain_is_as_accurate_as_plain_bf16():
    """The reason the Gram chain is held in fp16: with it, the Gram form's
    error against float64 is no larger than the plain bf16 iteration's
    (here within 10%) on a Gaussian input and on two singular-value
    spectra, while a bf16 chain is up to ~2.5x larger on the two-cluster
    spectrum."""
    from ns_bf16_model import newton_schulz_gram_model
    rng = np.random.default_rng(4)
    cases = [rng.standard_normal((96, 320)),
             _closed_form_input(64, 192, np.repeat([1.0, 0.3], [32, 32]), 7),
             _closed_form_input(64, 192, np.geomspace(1.0, 0.1, 64), 8)]
    worst_bf16_ratio = 0.0
    for g in cases:
        ref = oracle.newton_schulz(g)
        err = lambda o: np.linalg.norm(o - ref) / np.linalg.norm(ref)  # noqa: E731
        plain = err(newton_schulz_bf16_model(g))
        f16 = err(newton_schulz_gram_model(g, chain="f16"))
        bf16 = err(newton_schulz_gram_model(g, chain="bf16"))
        assert f16 <= 1.1 * plain, (plain, f16)
        worst_bf16_ratio = max(worst_bf16_ratio, bf16 / plain)
    assert worst_bf16_ratio > 1.5
