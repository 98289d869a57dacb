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
