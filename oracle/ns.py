"""Newton-Schulz orthogonalisation in float64 -- part of the CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.

What it computes [BluScript trainer source, ShardedMuon comment block: the
update is NewtonSchulz of the momentum, the iterated matrix polynomial
X <- aX + (bXX' + c(XX')^2)X, in which every output entry depends on the
whole matrix; Muon config block: five iterations]:

  1. Transpose the input if it has more rows than columns, so the Gram matrix
     X X^T is the smaller square (m = min(rows, cols), n = max(rows, cols)).
  2. Scale by the Frobenius norm: X0 = U / (||U||_F + eps), eps = 1e-7.
  3. Repeat `steps` times:  A = X X^T;  B = b A + c A A;  X = a X + B X.
  4. Transpose back.

The pages print no coefficients; (a, b, c) = (3.4445, -4.7750, 2.0315) is the
quintic used everywhere here, the same for every iteration.  The matrix
products are numpy's float64 matmul; nothing else is blocked, fused or
reordered.
"""
from __future__ import annotations

import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7
NS_STEPS = 5


def frobenius_prescale(u: np.ndarray, eps: float = NS_EPS) -> np.ndarray:
    """U / (||U||_F + eps) in float64, in U's own orientation."""
    x = np.asarray(u, dtype=np.float64)
    return x / (np.sqrt(np.sum(x * x)) + eps)


def newton_schulz(u: np.ndarray, steps: int = NS_STEPS, coeffs=NS_COEFFS,
                  eps: float = NS_EPS) -> np.ndarray:
    """The orthogonalised update of one [rows, cols] matrix, float64, same shape."""
    a, b, c = (float(t) for t in coeffs)
    x = np.asarray(u, dtype=np.float64)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    x = frobenius_prescale(x, eps)
    for _ in range(steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    if transposed:
        x = x.T
    return np.ascontiguousarray(x)


def ns_scalar_map(sigma, steps: int = NS_STEPS, coeffs=NS_COEFFS):
    """The polynomial the iteration applies to each singular value of the
    pre-scaled input: phi(s) = a s + b s^3 + c s^5, applied `steps` times."""
    a, b, c = (float(t) for t in coeffs)
    s = np.asarray(sigma, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s
