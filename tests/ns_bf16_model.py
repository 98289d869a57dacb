"""A model of Newton-Schulz rounding in bf16 -- test-side diagnostic.

Not the reference (that is oracle.newton_schulz, float64).  This model runs
the same iteration with every stored matrix rounded to bf16 (the oracle's
pinned round-to-nearest-even), products accumulated in float64 and rounded
to fp32, and the diagonals of A = X X^T and B = b A + c A A carried in fp32
beside their bf16 off-diagonal parts.  Like the kernels, it keeps the first
iteration's input as bf16(U) and applies the pre-scale s = 1/(||U||_F + eps)
to that iteration's products in fp32 (s^2 to X X^T, s to B X).  It bounds the error a bf16
Newton-Schulz has against float64 on a given input, so a test can tell
rounding that is intrinsic to bf16 from a fault in the kernels.  With
`round_bf16=False` it is the float64 iteration itself (checked in the CPU
tests).
"""
import numpy as np

import oracle


def _bf(x, on):
    if not on:
        return x
    return oracle.bf16_bits_to_f32(oracle.rne_bf16(np.asarray(x, np.float32))).astype(np.float64)


def _f32(x, on):
    return np.asarray(x, np.float32).astype(np.float64) if on else x


def newton_schulz_bf16_model(u, steps=5, coeffs=oracle.NS_COEFFS, eps=oracle.NS_EPS,
                             round_bf16=True):
    a, b, c = coeffs
    x = np.asarray(u, np.float64)
    tr = x.shape[0] > x.shape[1]
    if tr:
        x = x.T
    s = _f32(1.0 / _f32(np.sqrt(_f32(np.sum(x * x), round_bf16)) + eps, round_bf16), round_bf16)
    if steps == 0:
        x = _bf(x * s, round_bf16)
        return np.ascontiguousarray(x.T if tr else x)
    x = _bf(x, round_bf16)
    for k in range(steps):
        g = _f32(x @ x.T, round_bf16)
        if k == 0:
            g = _f32(g * (s * s), round_bf16)
        da = np.diag(g).copy()
        aoff = _bf(g - np.diag(da), round_bf16)
        aa = _f32(aoff @ aoff, round_bf16) + da[:, None] * aoff + aoff * da[None, :] + np.diag(da * da)
        bm = _f32(b * (aoff + np.diag(da)) + c * aa, round_bf16)
        db = np.diag(bm).copy()
        boff = _bf(bm - np.diag(db), round_bf16)
        xn = _f32((a + db)[:, None] * x + _f32(boff @ x, round_bf16), round_bf16)
        if k == 0:
            xn = _f32(xn * s, round_bf16)
        x = _bf(xn, round_bf16)
    return np.ascontiguousarray(x.T if tr else x)
