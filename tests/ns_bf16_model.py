"""A model of Newton-Schulz rounding in bf16 -- test-side diagnostic.

Not the reference (that is oracle.newton_schulz, float64).  This model runs
the same iteration with every stored matrix rounded to bf16 (the oracle's
pinned round-to-nearest-even), products accumulated in float64 and rounded
to fp32, and the diagonals of A = X X^T and B = b A + c A A carried in fp32
beside their bf16 off-diagonal parts.  Like the kernels, it forms
s = 1/(||U||_F + eps) in float64 and, when ||U||_F^2 lies in
[FOLD_MIN, FOLD_MAX], keeps the first iteration's input as bf16(U) and applies
s to that iteration's products in fp32 (s^2 to X X^T, s to B X); outside that
range the input is bf16(U s).  It estimates the error a bf16 Newton-Schulz
has against float64 on a given input -- a printed diagnostic beside the GPU
tests, never their pass criterion, which is the float64 oracle.  With
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


# the range of ||U||_F^2 over which the first iteration applies s to its
# fp32 products of bf16(U)
FOLD_MIN, FOLD_MAX = 2.0 ** -60, 2.0 ** 100


def newton_schulz_bf16_model(u, steps=5, coeffs=oracle.NS_COEFFS, eps=oracle.NS_EPS,
                             round_bf16=True):
    a, b, c = coeffs
    x = np.asarray(u, np.float64)
    tr = x.shape[0] > x.shape[1]
    if tr:
        x = x.T
    total = float(np.sum(x * x))
    s = 1.0 / (np.sqrt(total) + eps)
    folded = round_bf16 and FOLD_MIN <= total <= FOLD_MAX
    if steps == 0 or not folded:
        x = _bf(_f32(x * s, round_bf16), round_bf16)
        if steps == 0:
            return np.ascontiguousarray(x.T if tr else x)
        s = 1.0
    else:
        x = _bf(x, round_bf16)
    s2 = _f32(s * s, round_bf16)
    s = _f32(s, round_bf16)
    for k in range(steps):
        g = _f32(x @ x.T, round_bf16)
        if k == 0:
            g = _f32(g * s2, round_bf16)
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


def gram_segments(steps, per=3):
    """Segment lengths of `steps` Newton-Schulz steps on the Gram matrix:
    ceil(steps / per) segments as even as possible, longer ones first."""
    if steps <= 0:
        return []
    nseg = (steps + per - 1) // per
    base, extra = divmod(steps, nseg)
    return [base + (1 if i < extra else 0) for i in range(nseg)]


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def newton_schulz_gram_model(u, steps=5, coeffs=oracle.NS_COEFFS, eps=oracle.NS_EPS,
                             chain="f16"):
    """The same steps in segments on the m x m Gram matrix, as the kernels
    run them for matrices whose long side is at least twice the short one.
    Per segment of L steps from X: A = X X^T, then for j < L: P_j = a I +
    b A_j + c A_j^2, Q_j = P_j Q_{j-1} (Q_0 = P_0), A_{j+1} = (P_j P_j) A_j;
    X' = Q_{L-1} X.  Each m x m matrix is stored with its off-diagonal part
    rounded to `chain` ("f16" or "bf16"; "bf16" for every matrix of a segment
    of one step) and its diagonal in fp32, the upper triangle mirrored;
    Q_{L-1} is rounded to bf16 for the product with the bf16 X, which is
    rounded to bf16 after it.  The pre-scale is applied as in
    newton_schulz_bf16_model (X0 = bf16(U s) here, outside the kernels' fold
    range as well).  chain=None: no rounding anywhere, the float64 Gram
    identities themselves (checked against the oracle in the CPU tests)."""
    a, b, c = coeffs
    on = chain is not None
    x = np.asarray(u, np.float64)
    tr = x.shape[0] > x.shape[1]
    if tr:
        x = x.T
    s = 1.0 / (np.sqrt(float(np.sum(x * x))) + eps)
    x = _bf(_f32(x * s, on), on)

    def store(mat, rnd):
        mat = np.triu(mat) + np.triu(mat, 1).T
        if not on:
            return mat
        d = np.diag(mat).copy()
        return rnd(mat - np.diag(d)) + np.diag(_f32(d, True))

    bf = lambda v: _bf(v, True)  # noqa: E731
    for L in gram_segments(steps):
        rnd = _f16 if (chain == "f16" and L > 1) else bf
        A = store(_f32(x @ x.T, on), rnd)
        Q = None
        for j in range(L):
            P = store(a * np.eye(len(A)) + b * A + c * _f32(A @ A, on), rnd)
            Q = P if Q is None else store(_f32(P @ Q, on), rnd)
            if j + 1 < L:
                A = store(_f32(store(_f32(P @ P, on), rnd) @ A, on), rnd)
        x = _bf(_f32(store(Q, bf) @ x, on), on)
    return np.ascontiguousarray(x.T if tr else x)
