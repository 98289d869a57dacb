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
