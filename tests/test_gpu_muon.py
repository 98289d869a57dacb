"""GPU parity of zopt_muon_step against the oracle, stage by stage.

  momentum   the fp32 momentum equals the oracle's bit for bit;
  NS         the bf16 orthogonalised update O (read from the workspace) is
             within 2e-2 relative Frobenius error of the oracle's float64
             Newton-Schulz of the same U;
  post-step  teacher-forced: the oracle's post-step on the GPU's own O gives
             the same fp32 master and bf16 weight bit for bit.

Shapes cover ragged sizes (tile padding), both orientations (rows > cols is
transposed), every workload's shapes, and the scalar-polynomial closed form
of Newton-Schulz on U diag(s) V^T inputs.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NS_TOL = 2e-2


def f32(x):
    return float(np.float32(x))


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def make_inputs(batch, rows, cols, seed, dist="normal", master_std=0.02, grad_std=1e-3,
                momentum_nonzero=False):
    rng = np.random.default_rng(seed)
    P = [(rng.standard_normal((rows, cols)) * master_std).astype(np.float32) for _ in range(batch)]
    if dist == "student_t3":
        G = [wl.to_bf16_bits((rng.standard_t(3, (rows, cols)) * grad_std).astype(np.float32))
             for _ in range(batch)]
    else:
        G = [wl.to_bf16_bits((rng.standard_normal((rows, cols)) * grad_std).astype(np.float32))
             for _ in range(batch)]
    M = [((rng.standard_normal((rows, cols)) * grad_std).astype(np.float32) if momentum_nonzero
          else np.zeros((rows, cols), np.float32)) for _ in range(batch)]
    return P, M, G


def dev_f32(a):
    return torch.from_numpy(a.copy()).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def check_step(batch, rows, cols, seed, ns_steps=5, nesterov=True, adjust=1, lr=8e-4, mu=0.95,
               wd=0.1, dist="normal", momentum_nonzero=True, weights=True, check_ns=True,
               P=None, M=None, G=None, coeffs=oracle.NS_COEFFS):
    if P is None:
        P, M, G = make_inputs(batch, rows, cols, seed, dist, momentum_nonzero=momentum_nonzero)
    gP = [dev_f32(p) for p in P]
    gM = [dev_f32(m) for m in M]
    gG = [dev_bf16(g) for g in G]
    gW = [torch.full((rows, cols), 3.0, dtype=torch.bfloat16, device=DEV) for _ in range(batch)]
    lr32, mu32, wd32 = f32(lr), f32(mu), f32(wd)
    ws = z.muon_step(gP, gM, gG, gW if weights else None, lr32, mu32, nesterov, wd32, ns_steps,
                     ns_coeffs=tuple(f32(x) for x in coeffs), adjust_lr=adjust)
    torch.cuda.synchronize()
    worst = 0.0
    for i in range(batch):
        m = M[i].copy()
        u = oracle.muon_pre(m, G[i], mu32, nesterov)
        np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
        o_gpu = u16(z.muon_output_view(ws, batch, rows, cols, ns_steps, i))
        o_gpu32 = oracle.bf16_bits_to_f32(o_gpu)
        if check_ns:
            o_ref = oracle.newton_schulz(u, ns_steps, tuple(f32(x) for x in coeffs))
            err = rel_fro(o_gpu32.astype(np.float64), o_ref)
            worst = max(worst, err)
            assert err <= NS_TOL, (i, err)
        p = P[i].copy()
        w = oracle.muon_post(p, o_gpu32, lr32, wd32, adjust)
        np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), p.view(np.uint32))
        if weights:
            np.testing.assert_array_equal(u16(gW[i]), w)
    return worst, ws


@pytest.mark.parametrize("rows,cols", [(64, 1 << 21), (1 << 21, 64)])
def test_longest_side_at_the_limit(rows, cols):
    """The longest side the library accepts, 2^21, on a 64-row matrix in both
    orientations (Gram form on 64 x 64 tiles, X X^T split along K over 2^21):
    the kernels' 32-bit panel and stage offsets reach their largest values
    here.  Momentum and post-step bit for bit, Newton-Schulz within the bar."""
    worst, _ = check_step(1, rows, cols, seed=2 ** 21 + rows)
    print(f"{rows} x {cols}: NS rel err {worst:.3e}", flush=True)


def test_tiny_workload_ten_steps():
    """2 x [128, 512], 10 Muon steps carrying momentum and master across steps."""
    w = wl.TINY_MUON
    rows, cols = w.groups[0].rows, w.groups[0].cols
    P = [wl.host_normal(w.wid, 10 + i, (rows, cols), w.master_std) for i in range(2)]
    M = [np.zeros((rows, cols), np.float32) for _ in range(2)]
    gP, gM = [dev_f32(p) for p in P], [dev_f32(m) for m in M]
    lr, mu, wd = f32(w.lr), f32(w.momentum), f32(w.weight_decay)
    for t in range(1, 11):
        G = [wl.host_grad_bf16(w.wid, 20 + i, (rows, cols), w.grad_std, step=t) for i in range(2)]
        ws = z.muon_step(gP, gM, [dev_bf16(g) for g in G], None, lr, mu, True, wd, 5)
        torch.cuda.synchronize()
        for i in range(2):
            u = oracle.muon_pre(M[i], G[i], mu, True)
            o = oracle.bf16_bits_to_f32(u16(z.muon_output_view(ws, 2, rows, cols, 5, i)))
            assert rel_fro(o.astype(np.float64), oracle.newton_schulz(u)) <= NS_TOL
            oracle.muon_post(P[i], o, lr, wd, 1, want_weight=False)
            np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), M[i].view(np.uint32))
            np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), P[i].view(np.uint32))


@pytest.mark.parametrize("batch,rows,cols", [
    (1, 100, 300), (2, 300, 100), (3, 1, 17), (2, 17, 1), (1, 65, 130), (2, 130, 65),
    (1, 64, 64), (4, 257, 511), (1, 9, 1000), (2, 640, 200),
    (1, 1100, 1300), (2, 1300, 1100), (1, 1024, 1024), (1, 1030, 2100),
    (1, 1, 1), (64, 1, 1), (64, 33, 70),
])
def test_ragged_shapes(batch, rows, cols):
    check_step(batch, rows, cols, seed=rows * 7 + cols)


@pytest.mark.parametrize("ns_steps", [0, 1, 2, 7])
def test_ns_step_counts(ns_steps):
    check_step(2, 96, 200, seed=3, ns_steps=ns_steps)
    check_step(1, 200, 96, seed=4, ns_steps=ns_steps)


@pytest.mark.parametrize("coeffs,steps", [
    ((1.5, -0.5, 0.0), 8),              # cubic Newton-Schulz: c = 0, A A term read in the epilogue
    ((1.5, -0.5, 1e-6), 6),             # b / c beyond the in-loop form's range
    ((2.0, -1.5, 0.5), 5),              # another quintic with p(1) = 1
    ((3.4445, -4.7750, 2.0315), 3),
])
def test_ns_coefficient_sets(coeffs, steps):
    check_step(2, 200, 330, seed=11, ns_steps=steps, coeffs=coeffs)
    check_step(1, 330, 200, seed=12, ns_steps=steps, coeffs=coeffs)
    check_step(1, 1100, 1300, seed=13, ns_steps=steps, coeffs=coeffs)


@pytest.fixture
def ns_form():
    yield z.set_ns_form
    z.set_ns_form(z.NS_FORM_AUTO)


# Groups whose long side is at least twice the short one and whose work
# batch m^2 (n - m) reaches 2^29: Newton-Schulz runs in segments on the Gram
# matrix by default.  Both orientations, ragged sizes, 64-, 128- and 256-tile
# symmetric products.
GRAM_SHAPES = [(48, 120, 1000), (64, 1000, 100), (8, 300, 1100), (4, 1500, 400), (1, 1100, 2300)]


@pytest.mark.parametrize("ns_steps", [1, 2, 3, 4, 5, 7])
def test_gram_form_matches_oracle_and_plain_form(ns_form, ns_steps):
    """Each form -- the default (fp16 chain), plain iterations and the Gram
    form with a bf16 chain -- within NS_TOL of the float64 oracle, momentum and
    post-step bit for bit (check_step); the default and the plain results
    within NS_TOL of each other."""
    forms = (z.NS_FORM_AUTO, z.NS_FORM_PLAIN, z.NS_FORM_GRAM_BF16)
    for (b, r, c) in GRAM_SHAPES:
        outs = {}
        for form in forms:
            ns_form(form)
            worst, ws = check_step(b, r, c, seed=r + c + ns_steps, ns_steps=ns_steps)
            outs[form] = oracle.bf16_bits_to_f32(
                u16(z.muon_output_view(ws, b, r, c, ns_steps, 0))).astype(np.float64)
            print(f"{b}x[{r}, {c}] ns_steps={ns_steps} form {form}: worst NS rel err {worst:.3e}",
                  flush=True)
        assert rel_fro(outs[z.NS_FORM_AUTO], outs[z.NS_FORM_PLAIN]) <= NS_TOL


def test_short_side_past_fp16_range_runs_plain_bf16(ns_form):
    """m = 4160 > 4096: the group runs plain iterations with every matrix in
    bf16 (fp16 would hold A's off-diagonal entries in its subnormal range),
    also when its shape would otherwise take the Gram form, and its result
    equals the plain form's bit for bit."""
    P, M, G = make_inputs(1, 4160, 8320, 41, momentum_nonzero=True)
    worst, ws = check_step(1, 4160, 8320, 41, P=P, M=M, G=G)
    o = u16(z.muon_output_view(ws, 1, 4160, 8320, 5, 0)).copy()
    print(f"[4160, 8320]: NS rel err {worst:.3e}", flush=True)
    ns_form(z.NS_FORM_PLAIN)
    _, ws1 = check_step(1, 4160, 8320, 41, P=P, M=M, G=G, check_ns=False)
    np.testing.assert_array_equal(u16(z.muon_output_view(ws1, 1, 4160, 8320, 5, 0)), o)


@pytest.mark.parametrize("coeffs,steps", [
    ((1.5, -0.5, 0.0), 8),
    ((2.0, -1.5, 0.5), 5),
    ((3.4445, -4.7750, 2.0315), 3),
])
def test_gram_form_coefficient_sets(coeffs, steps):
    check_step(40, 160, 800, seed=21, ns_steps=steps, coeffs=coeffs)
    check_step(4, 1300, 520, seed=22, ns_steps=steps, coeffs=coeffs)


def test_gram_form_large_coefficients_take_a_bf16_chain():
    """Coefficients whose m x m chain could leave fp16's range (p(0)^3 = 21^3
    > 2^13 in a segment of three steps) run the Gram form with its chain in
    bf16.  Each input has 16 equal singular values, 1/4 after the pre-scale,
    where p(1/16) = 1 and the map's slope is 0, so every step keeps X and
    rounding does not grow; 64 matrices of 16 x 32800 reach the Gram form's
    work threshold."""
    batch, rows, cols = 64, 16, 32800
    rng = np.random.default_rng(31)
    G, P, M = [], [], []
    for _ in range(batch):
        q, _ = np.linalg.qr(rng.standard_normal((cols, rows)))
        G.append(wl.to_bf16_bits((q.T * 1e-3).astype(np.float32)))
        P.append((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
        M.append(np.zeros((rows, cols), np.float32))
    worst, _ = check_step(batch, rows, cols, 32, ns_steps=3, coeffs=(21.0, -632.0, 4992.0), P=P,
                          M=M, G=G)
    print(f"coefficients (21, -632, 4992), 3 steps: worst NS rel err {worst:.3e}", flush=True)


@pytest.mark.parametrize("nesterov,adjust", [(False, 1), (True, 0), (False, 0)])
def test_momentum_and_scale_variants(nesterov, adjust):
    check_step(2, 192, 320, seed=5, nesterov=nesterov, adjust=adjust)
    check_step(2, 320, 192, seed=6, nesterov=nesterov, adjust=adjust)


def test_no_weight_buffer_and_zero_gradient():
    rows, cols = 128, 256
    P, M, G = make_inputs(1, rows, cols, 8, momentum_nonzero=False)
    G = [np.zeros_like(G[0])]
    check_step(1, rows, cols, 8, P=P, M=M, G=G, weights=False, check_ns=False)
    # zero update: the output is exactly zero (0 / (0 + eps) = 0)
    gP, gM, gG = [dev_f32(P[0])], [dev_f32(M[0])], [dev_bf16(G[0])]
    ws = z.muon_step(gP, gM, gG, None, f32(8e-4), f32(0.95), True, f32(0.1), 5)
    assert not z.muon_output_view(ws, 1, rows, cols, 5, 0).float().any()


def ns_on_spectrum(m, n, sigma, seed):
    """GPU Newton-Schulz of G = U diag(sigma) V^T (mu = 0, so the update is
    G itself); returns (GPU result, the G it saw, the U diag V^T factors)."""
    rng = np.random.default_rng(seed)
    k = min(m, n)
    qu, _ = np.linalg.qr(rng.standard_normal((m, m)))
    qv, _ = np.linalg.qr(rng.standard_normal((n, n)))
    g = ((qu[:, :k] * sigma) @ qv.T[:k]) * 1e-3
    gb = wl.to_bf16_bits(g.astype(np.float32))
    gf = oracle.bf16_bits_to_f32(gb).astype(np.float64)
    gP = [torch.zeros((m, n), dtype=torch.float32, device=DEV)]
    gM = [torch.zeros((m, n), dtype=torch.float32, device=DEV)]
    ws = z.muon_step(gP, gM, [dev_bf16(gb)], None, 0.0, 0.0, True, 0.0, 5)
    o = oracle.bf16_bits_to_f32(u16(z.muon_output_view(ws, 1, m, n, 5, 0))).astype(np.float64)
    return o, gf, qu[:, :k], qv.T[:k]


@pytest.mark.parametrize("m,n", [(64, 192), (256, 512), (384, 128)])
@pytest.mark.parametrize("spectrum", ["decade", "two_clusters"])
def test_ns_closed_form_on_singular_values(m, n, spectrum):
    """For G = U diag(s) V^T the float64 oracle acts as phi^5 on s (pinned on
    the CPU); the GPU's bf16 result must lie within the tolerance of both."""
    k = min(m, n)
    sigma = (np.geomspace(1.0, 0.1, k) if spectrum == "decade"
             else np.repeat([1.0, 0.3], [k // 2, k - k // 2]))
    o, gf, u, vt = ns_on_spectrum(m, n, sigma, seed=m + n)
    assert rel_fro(o, oracle.newton_schulz(gf)) <= NS_TOL
    closed = (u * oracle.ns_scalar_map(sigma / np.linalg.norm(sigma))) @ vt
    assert rel_fro(o, closed) <= NS_TOL


# Singular values spanning two decades are the one input class measured
# outside 2e-2: the smallest directions grow by ~3.44 per iteration and so
# does the bf16 rounding noise in them, so any bf16 Newton-Schulz ends
# ~2.5-3e-2 from float64 there.  The bar for it is stated here, against the
# float64 oracle.
NS_TOL_TWO_DECADE = 3e-2


@pytest.mark.parametrize("m,n", [(64, 192), (384, 128)])
def test_ns_two_decade_spectrum_is_bf16_limited(m, n):
    """Singular values 1 .. 1e-2 (geometric): within NS_TOL_TWO_DECADE of the
    float64 oracle.  The bf16 rounding model's error on the same input is
    printed beside it as a diagnostic only."""
    from ns_bf16_model import newton_schulz_bf16_model
    sigma = np.geomspace(1.0, 1e-2, min(m, n))
    o, gf, _, _ = ns_on_spectrum(m, n, sigma, seed=m + n)
    ref = oracle.newton_schulz(gf)
    model_err = rel_fro(newton_schulz_bf16_model(gf), ref)
    gpu_err = rel_fro(o, ref)
    print(f"two-decade spectrum {m}x{n}: GPU {gpu_err:.3e} (bf16 model {model_err:.3e})")
    assert gpu_err <= NS_TOL_TWO_DECADE


def extreme_grads(rows, cols, kind, seed):
    """bf16 gradients of a magnitude far from the usual: a Gaussian times
    `kind` (a float), or 'bf16max': N(0, 1e-3) with 1% of the entries set to
    +-0x7F7F, the largest finite bf16."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((rows, cols))
    if kind == "bf16max":
        g = (g * 1e-3).astype(np.float32)
        mask = rng.random((rows, cols)) < 0.01
        bits = wl.to_bf16_bits(g)
        bits[mask] = np.where(rng.random(int(mask.sum())) < 0.5, 0x7F7F, 0xFF7F)
        return bits
    return wl.to_bf16_bits((g * kind).astype(np.float32))


@pytest.mark.parametrize("rows,cols,kinds,ns_steps", [
    (768, 3072, (1e17, 1e30, "bf16max", 1e12, 1e-30, 1e-10), 5),
    (3072, 768, (1e17, "bf16max"), 5),
    (768, 3072, (1e17, 1e30, "bf16max", 1e-30), 0),
    (4096, 4096, (1e17, "bf16max"), 5),
    (4096, 4096, (1e30,), 0),
])
def test_extreme_gradient_magnitudes(rows, cols, kinds, ns_steps):
    """Huge and tiny finite gradients (||U||_F^2 from ~2^-190 to ~2^270,
    inside and outside the range where the first iteration applies the
    pre-scale to products of bf16(U)), each in one group beside a matrix of
    ordinary gradients: the update is NaN-free and within 2e-2 of float64,
    the momentum and the teacher-forced post-step bit for bit."""
    k = len(kinds) + 1
    P, M, G = make_inputs(k, rows, cols, seed=rows + cols + ns_steps, momentum_nonzero=False)
    for i, kind in enumerate(kinds):
        G[i + 1] = extreme_grads(rows, cols, kind, seed=17 + i)
    gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
    gW = [torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    lr, mu, wd = f32(8e-4), f32(0.95), f32(0.1)
    ws = z.muon_step(gP, gM, gG, gW, lr, mu, True, wd, ns_steps)
    torch.cuda.synchronize()
    for i in range(k):
        kind = "normal" if i == 0 else kinds[i - 1]
        m = M[i].copy()
        u = oracle.muon_pre(m, G[i], mu, True)
        np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
        o = oracle.bf16_bits_to_f32(u16(z.muon_output_view(ws, k, rows, cols, ns_steps, i)))
        assert not np.isnan(o).any(), kind
        err = rel_fro(o.astype(np.float64), oracle.newton_schulz(u, ns_steps))
        print(f"{rows}x{cols} ns_steps={ns_steps} grads {kind}: NS rel err {err:.3e}", flush=True)
        assert err <= NS_TOL, (kind, err)
        p = P[i].copy()
        w = oracle.muon_post(p, o, lr, wd, 1)
        np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), p.view(np.uint32))
        np.testing.assert_array_equal(u16(gW[i]), w)


@pytest.mark.parametrize("rows,cols,ns_steps", [(200, 520, 5), (520, 200, 5), (200, 520, 0)])
def test_infinite_gradient_gives_nan_update_like_the_oracle(rows, cols, ns_steps):
    """An infinite gradient entry: ||U||_F is infinite, so the oracle's
    pre-scaled matrix holds NaN at that entry and 0 elsewhere, and Newton-
    Schulz spreads the NaN over the whole update -- the GPU's update is NaN
    wherever the oracle's is, the matrix beside it in the group is unaffected,
    momentum and the teacher-forced post-step are bit for bit (NaN where the
    oracle's is NaN)."""
    P, M, G = make_inputs(2, rows, cols, seed=23, momentum_nonzero=True)
    G[1] = G[1].copy()
    G[1][rows // 3, cols // 5] = 0x7F80  # +Inf
    gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
    lr, mu, wd = f32(8e-4), f32(0.95), f32(0.1)
    ws = z.muon_step(gP, gM, gG, None, lr, mu, True, wd, ns_steps)
    torch.cuda.synchronize()
    for i in range(2):
        m = M[i].copy()
        u = oracle.muon_pre(m, G[i], mu, True)
        np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
        o = oracle.bf16_bits_to_f32(u16(z.muon_output_view(ws, 2, rows, cols, ns_steps, i)))
        with np.errstate(invalid="ignore"):
            ref = oracle.newton_schulz(u, ns_steps)
        np.testing.assert_array_equal(np.isnan(o), np.isnan(ref))
        if i == 0:
            assert rel_fro(o.astype(np.float64), ref) <= NS_TOL
        p = P[i].copy()
        oracle.muon_post(p, o, lr, wd, 1, want_weight=False)
        got = gP[i].cpu().numpy()
        nan = np.isnan(p)
        assert np.array_equal(np.isnan(got), nan)  # NaN payloads may differ
        np.testing.assert_array_equal(got[~nan].view(np.uint32), p[~nan].view(np.uint32))


def test_deterministic_run_to_run():
    P, M, G = make_inputs(3, 200, 520, seed=9, momentum_nonzero=True)
    outs = []
    for _ in range(2):
        gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
        gW = [torch.empty((200, 520), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
        ws = z.muon_step(gP, gM, gG, gW, f32(8e-4), f32(0.95), True, f32(0.1), 5)
        outs.append([u16(z.muon_output_view(ws, 3, 200, 520, 5, i)) for i in range(3)] +
                    [u16(w) for w in gW] + [p.cpu().numpy() for p in gP])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_gpt2_small_shapes():
    """Every GPT-2-small Muon group (48 x 768^2, 12 x 3072x768, 12 x 768x3072),
    1% outlier gradients; NS checked on a few matrices of each group."""
    w = wl.GPT2_MUON
    for gi, grp in enumerate(w.groups):
        k = grp.count
        P = [wl.host_normal(w.wid, 100 * gi + i, (grp.rows, grp.cols), w.master_std)
             for i in range(k)]
        G = [wl.host_grad_bf16(w.wid, 5000 + 100 * gi + i, (grp.rows, grp.cols), w.grad_std,
                               "normal_outliers") for i in range(k)]
        M = [np.zeros((grp.rows, grp.cols), np.float32) for _ in range(k)]
        gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
        ws = z.muon_step(gP, gM, gG, None, f32(w.lr), f32(w.momentum), True,
                         f32(w.weight_decay), 5)
        torch.cuda.synchronize()
        for i in sorted({0, k // 2, k - 1}):
            u = oracle.muon_pre(M[i], G[i], f32(w.momentum), True)
            np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), M[i].view(np.uint32))
            o = oracle.bf16_bits_to_f32(u16(z.muon_output_view(ws, k, grp.rows, grp.cols, 5, i)))
            assert rel_fro(o.astype(np.float64), oracle.newton_schulz(u)) <= NS_TOL
            oracle.muon_post(P[i], o, f32(w.lr), f32(w.weight_decay), 1, want_weight=False)
            np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), P[i].view(np.uint32))


NS_BLOCK = 128
NS_TOL_BLOCK = 5e-2


def blockwise_rel_fro(o, ref, blk=NS_BLOCK):
    """The largest relative Frobenius error over the blk x blk blocks of the
    update (ragged edge blocks included).  A wrong 16 x 16 MFMA block inside a
    128 x 128 block is 1/8 of its norm: ~0.12 there, while on the whole of a
    4096 x 14336 matrix it would add well under the 2e-2 bar."""
    worst = 0.0
    for r in range(0, o.shape[0], blk):
        for c in range(0, o.shape[1], blk):
            worst = max(worst, rel_fro(o[r:r + blk, c:c + blk], ref[r:r + blk, c:c + blk]))
    return worst


@pytest.mark.parametrize("workload", ["llama1b_rank0_muon", "llama8b_rank0_muon"])
def test_full_size_groups_one_matrix_each(workload):
    """The full 1B and 8B rank-0 shares in the launch configuration the
    benchmark times (one zopt_muon_step_groups call over all groups);
    momentum and post-step are checked on every matrix, NS against fp64 on the
    first and the last matrix of every group: within 2e-2 on the whole matrix
    and within NS_TOL_BLOCK on every 128 x 128 block."""
    w = wl.MUON_WORKLOADS[workload]
    calls, inputs = [], []
    for gi, grp in enumerate(w.groups):
        k = grp.count
        shape = (grp.rows, grp.cols)
        gP = [wl.device_normal(w.wid, 100 * gi + i, shape, w.master_std, DEV) for i in range(k)]
        gG = [wl.device_grad_bf16(w.wid, 5000 + 100 * gi + i, shape, w.grad_std, DEV, w.grad_dist)
              for i in range(k)]
        gM = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in range(k)]
        calls.append((gP, gM, gG, None))
        inputs.append(([p.cpu().numpy() for p in gP], [u16(g) for g in gG]))
    shapes = [(g.count, g.rows, g.cols) for g in w.groups]
    ws = z.muon_step_groups(calls, f32(w.lr), f32(w.momentum), True, f32(w.weight_decay), 5)
    torch.cuda.synchronize()
    for gi, grp in enumerate(w.groups):
        shape = (grp.rows, grp.cols)
        gP, gM = calls[gi][0], calls[gi][1]
        P0, G = inputs[gi]
        for i in range(grp.count):
            m = np.zeros(shape, np.float32)
            u = oracle.muon_pre(m, G[i], f32(w.momentum), True)
            np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
            o = oracle.bf16_bits_to_f32(u16(z.muon_groups_output_view(ws, shapes, 5, gi, i)))
            if i in (0, grp.count - 1):
                ref = oracle.newton_schulz(u)
                o64 = o.astype(np.float64)
                err, berr = rel_fro(o64, ref), blockwise_rel_fro(o64, ref)
                print(f"{workload} group {shape} x{grp.count} matrix {i}: NS rel err {err:.3e}, "
                      f"worst {NS_BLOCK}-block {berr:.3e}", flush=True)
                assert err <= NS_TOL
                assert berr <= NS_TOL_BLOCK
            p = P0[i]
            oracle.muon_post(p, o, f32(w.lr), f32(w.weight_decay), 1, want_weight=False)
            np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), p.view(np.uint32))


def grouped_vs_separate(specs, seed, ns_steps=5, ns_check=lambda b, r, c, i: True):
    """One zopt_muon_step_groups call over `specs` [(batch, rows, cols)]:
    every matrix is checked against the oracle (momentum and post-step bit for
    bit, NS within tolerance where ns_check says so) and against separate
    zopt_muon_step calls on the same inputs, which must agree bit for bit."""
    lr, mu, wd = f32(8e-4), f32(0.95), f32(0.1)
    host = [make_inputs(b, r, c, seed + 31 * k, momentum_nonzero=True)
            for k, (b, r, c) in enumerate(specs)]

    def upload():
        out = []
        for (b, r, c), (P, M, G) in zip(specs, host):
            out.append(([dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G],
                        [torch.full((r, c), 3.0, dtype=torch.bfloat16, device=DEV)
                         for _ in range(b)]))
        return out

    grouped = upload()
    ws = z.muon_step_groups(grouped, lr, mu, True, wd, ns_steps)
    separate = upload()
    wss = [z.muon_step(*g, lr, mu, True, wd, ns_steps) for g in separate]
    torch.cuda.synchronize()
    worst = 0.0
    for k, ((b, r, c), (P, M, G)) in enumerate(zip(specs, host)):
        gP, gM, _, gW = grouped[k]
        sP, sM, _, sW = separate[k]
        for i in range(b):
            o_bits = u16(z.muon_groups_output_view(ws, specs, ns_steps, k, i))
            assert np.array_equal(o_bits, u16(z.muon_output_view(wss[k], b, r, c, ns_steps, i))), \
                ("grouped != separate", k, i)
            for x, y in ((gP[i], sP[i]), (gM[i], sM[i])):
                assert np.array_equal(x.cpu().numpy().view(np.uint32),
                                      y.cpu().numpy().view(np.uint32)), ("grouped != separate", k, i)
            assert np.array_equal(u16(gW[i]), u16(sW[i]))
            m = M[i].copy()
            u = oracle.muon_pre(m, G[i], mu, True)
            np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
            o = oracle.bf16_bits_to_f32(o_bits)
            if ns_check(b, r, c, i):
                err = rel_fro(o.astype(np.float64), oracle.newton_schulz(u, ns_steps))
                worst = max(worst, err)
                assert err <= NS_TOL, (k, i, err)
            p = P[i].copy()
            wref = oracle.muon_post(p, o, lr, wd, 1)
            np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), p.view(np.uint32))
            np.testing.assert_array_equal(u16(gW[i]), wref)
    return worst


@pytest.mark.parametrize("ns_steps", [4, 10])
def test_gram_and_plain_groups_in_one_call(ns_steps):
    """Gram-form groups (64-, 128- and 256-tile, one stored transposed) beside
    plain ones in one call, their programs merged into one launch sequence --
    at 10 steps four segments and 34 Gram steps: each matrix against the
    oracle and bit for bit against separate calls.  (Many more steps leave
    the 2e-2 bar on some Gaussian inputs in either form: at 20 steps the
    plain bf16 iteration ends 4.0e-2 from float64 on one of 48 such
    120 x 1000 matrices, the Gram form 3.3e-2.)"""
    specs = [(48, 120, 1000), (2, 200, 200), (4, 1500, 400), (3, 300, 330), (1, 1100, 2300)]
    worst = grouped_vs_separate(specs, seed=51, ns_steps=ns_steps)
    print(f"{ns_steps} steps: worst NS rel err {worst:.3e}", flush=True)


def test_groups_mixed_tiles_match_oracle_and_separate_calls():
    """Eight groups over all three tile sizes, both orientations and ragged
    sizes, in one call."""
    specs = [(3, 200, 520), (2, 1100, 1300), (2, 1300, 1100), (2, 300, 700), (4, 96, 64),
             (1, 1030, 2100), (2, 520, 200), (3, 768, 3072)]
    grouped_vs_separate(specs, seed=77, ns_check=lambda b, r, c, i: i == 0 or r * c < 300_000)


def test_groups_more_than_fit_one_launch():
    """Eleven groups of the same tile size: the products take two launches."""
    specs = [(1 + k % 3, 64 + 9 * k, 100 + 13 * k) for k in range(11)]
    grouped_vs_separate(specs, seed=91)


def test_sixteen_groups_mixed_on_two_streams():
    """The most groups a call takes, 16: plain and Gram-form groups on all
    three tile sizes, both orientations, vectors (1 x 17, 17 x 1) and a
    1024-row group of 16 matrices whose 256-tile products, with the 768 x
    3072 Gram groups', stay under two rounds -- so the call runs on two
    streams, divided by class.  Every matrix equals its separate one-group
    call bit for bit; the first matrix of the smaller groups the oracle."""
    specs = [(16, 1024, 1024), (2, 768, 3072), (1, 3072, 768), (4, 300, 2000), (2, 2000, 300),
             (3, 200, 520), (2, 520, 200), (1, 64, 64), (5, 96, 64), (1, 1, 17), (2, 17, 1),
             (1, 257, 511), (1, 640, 200), (2, 130, 65), (1, 1030, 2100), (3, 512, 2048)]
    grouped_vs_separate(specs, seed=1616, ns_check=lambda b, r, c, i: i == 0 and r * c <= 2_100_000)


def test_two_stream_calls_from_two_host_threads():
    """Two host threads, each on a stream of its own, issue three two-stream
    grouped calls apiece (GPT-2-small-like groups: 24 x [768, 768] on 256
    tiles beside two Gram-form 768 x 3072 groups) on their own buffers: the
    library's one second stream and its fork and join events serve both,
    one call's enqueue at a time.  Every output equals the same calls made
    one after another on one stream, bit for bit."""
    import threading
    specs = [(24, 768, 768), (2, 768, 3072), (2, 3072, 768)]
    lr, mu, wd = f32(8e-4), f32(0.95), f32(0.1)

    def state(seed):
        host = [make_inputs(b, r, c, seed + 31 * k, momentum_nonzero=True)
                for k, (b, r, c) in enumerate(specs)]
        return [([dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G],
                 [torch.empty((r, c), dtype=torch.bfloat16, device=DEV) for _ in range(b)])
                for (b, r, c), (P, M, G) in zip(specs, host)]

    def outputs(groups):
        # per group: master and momentum bits (fp32), weight bits (bf16)
        return [(np.concatenate([t.cpu().numpy().view(np.uint32).ravel() for t in g[0] + g[1]]),
                 np.concatenate([u16(t).ravel() for t in g[3]]))
                for g in groups]

    seeds = (700, 900)
    ref = []
    for sd in seeds:
        groups = state(sd)
        for _ in range(3):
            z.muon_step_groups(groups, lr, mu, True, wd, 5)
        torch.cuda.synchronize()
        ref.append(outputs(groups))

    runs = [state(sd) for sd in seeds]
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            st = torch.cuda.Stream(device=DEV)
            ws = torch.empty(z.muon_groups_workspace_bytes(specs), dtype=torch.uint8, device=DEV)
            with torch.cuda.stream(st):
                for _ in range(3):
                    z.muon_step_groups(runs[k], lr, mu, True, wd, 5, workspace=ws, stream=st)
            st.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        got = outputs(runs[k])
        for gi in range(len(specs)):
            for part in range(2):
                assert np.array_equal(got[gi][part], ref[k][gi][part]), ("thread", k, "group", gi)


@pytest.mark.parametrize("ns_steps", [0, 1, 4])
def test_groups_step_counts(ns_steps):
    grouped_vs_separate([(2, 130, 260), (1, 700, 300), (1, 1024, 1100)], seed=13,
                        ns_steps=ns_steps)


def test_gpt2_small_one_call():
    """The headline's Muon call: all 72 GPT-2-small matrices in one grouped
    call (48 x 768^2, 12 x 3072x768, 12 x 768x3072), 1% outlier gradients;
    momentum and post-step on every matrix, NS on three matrices per group."""
    w = wl.GPT2_MUON
    calls, host = [], []
    for gi, grp in enumerate(w.groups):
        k = grp.count
        P = [wl.host_normal(w.wid, 100 * gi + i, (grp.rows, grp.cols), w.master_std)
             for i in range(k)]
        G = [wl.host_grad_bf16(w.wid, 5000 + 100 * gi + i, (grp.rows, grp.cols), w.grad_std,
                               "normal_outliers") for i in range(k)]
        calls.append(([dev_f32(p) for p in P],
                      [torch.zeros((grp.rows, grp.cols), device=DEV) for _ in range(k)],
                      [dev_bf16(g) for g in G],
                      [torch.empty((grp.rows, grp.cols), dtype=torch.bfloat16, device=DEV)
                       for _ in range(k)]))
        host.append((P, G))
    shapes = [(g.count, g.rows, g.cols) for g in w.groups]
    ws = z.muon_step_groups(calls, f32(w.lr), f32(w.momentum), True, f32(w.weight_decay), 5)
    torch.cuda.synchronize()
    for gi, grp in enumerate(w.groups):
        P, G = host[gi]
        gP, gM, _, gW = calls[gi]
        for i in range(grp.count):
            m = np.zeros((grp.rows, grp.cols), np.float32)
            u = oracle.muon_pre(m, G[i], f32(w.momentum), True)
            np.testing.assert_array_equal(gM[i].cpu().numpy().view(np.uint32), m.view(np.uint32))
            o = oracle.bf16_bits_to_f32(u16(z.muon_groups_output_view(ws, shapes, 5, gi, i)))
            if i in (0, grp.count // 2, grp.count - 1):
                assert rel_fro(o.astype(np.float64), oracle.newton_schulz(u)) <= NS_TOL
            wref = oracle.muon_post(P[i], o, f32(w.lr), f32(w.weight_decay), 1)
            np.testing.assert_array_equal(gP[i].cpu().numpy().view(np.uint32), P[i].view(np.uint32))
            np.testing.assert_array_equal(u16(gW[i]), wref)


@pytest.mark.parametrize("batch,rows,cols,ns_steps", [
    (2, 200, 520, 5), (2, 520, 200, 5), (1, 300, 1030, 5), (1, 1030, 300, 5),
    (1, 1100, 1300, 5), (2, 130, 65, 0), (1, 65, 130, 1),
])
def test_workspace_needs_no_initialisation(batch, rows, cols, ns_steps):
    """The workspace's prior contents do not matter: one filled with 0xFF
    bytes (NaN in every bf16 and fp32 slot, the Newton-Schulz padding
    included) gives bit for bit the outputs of a zero-filled one, on ragged
    shapes of both orientations and all three tile sizes, with and without
    iterations."""
    P, M, G = make_inputs(batch, rows, cols, seed=rows + 3 * cols, momentum_nonzero=True)
    outs = []
    for fill in (0x00, 0xFF):
        gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
        gW = [torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV) for _ in range(batch)]
        ws = torch.full((z.muon_workspace_bytes(batch, rows, cols),), fill, dtype=torch.uint8,
                        device=DEV)
        z.muon_step(gP, gM, gG, gW, f32(8e-4), f32(0.95), True, f32(0.1), ns_steps, workspace=ws)
        torch.cuda.synchronize()
        outs.append([u16(z.muon_output_view(ws, batch, rows, cols, ns_steps, i))
                     for i in range(batch)] + [u16(w) for w in gW] +
                    [t.cpu().numpy().view(np.uint32) for t in gP + gM])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    for o in outs[1][:batch]:
        assert not np.isnan(oracle.bf16_bits_to_f32(o)).any()


def test_grouped_workspace_needs_no_initialisation():
    """The same for a grouped call over both pass-1 forms (a flat stream with
    padding, a transposed matrix on 128 x 128 tiles) and a 64-tile group."""
    specs = [(2, 300, 1030), (1, 1030, 300), (2, 1536, 768), (3, 100, 300)]
    inputs = [make_inputs(b, r, c, seed=11 + r + c, momentum_nonzero=True) for b, r, c in specs]
    need = z.muon_groups_workspace_bytes(specs)
    outs = []
    for fill in (0x00, 0xFF):
        groups, flat = [], []
        for (b, r, c), (P, M, G) in zip(specs, inputs):
            gP, gM, gG = [dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G]
            gW = [torch.empty((r, c), dtype=torch.bfloat16, device=DEV) for _ in range(b)]
            groups.append((gP, gM, gG, gW))
            flat += gP + gM
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        z.muon_step_groups(groups, f32(8e-4), f32(0.95), True, f32(0.1), 5, workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().view(np.uint32) for t in flat] +
                    [u16(w) for g in groups for w in g[3]])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    for w in outs[1][-sum(b for b, _, _ in specs):]:
        assert not np.isnan(oracle.bf16_bits_to_f32(w)).any()


@pytest.mark.parametrize("ns_steps", [1, 5])
@pytest.mark.parametrize("form", ["auto", "plain"])
def test_two_stream_groups(ns_steps, form, ns_form):
    """A call whose Newton-Schulz iterations run on two streams: three groups
    on 256 tiles whose X X^T launch holds 136 + 72 + 72 = 280 workgroups,
    under two rounds of the GPU's 256, so the groups are divided between
    the caller's stream and the second one: by default the two plain groups
    on one and the 2048 x 5632 group, on the Gram matrix, on the other (a
    call that mixes the forms is divided by class); in plain iterations
    throughout the groups one by one (the 4096^2 group on one stream, the
    others on the other).  Every matrix equals the separate calls' (one
    group each: one stream) bit for bit; the 2048-row matrices against the
    oracle."""
    ns_form(z.NS_FORM_AUTO if form == "auto" else z.NS_FORM_PLAIN)
    specs = [(1, 4096, 4096), (2, 2048, 2048), (2, 2048, 5632)]
    grouped_vs_separate(specs, seed=123, ns_steps=ns_steps,
                        ns_check=lambda b, r, c, i: r == 2048 and i == 0)


def test_gpt2_small_groups_equal_separate_calls():
    """The headline's three GPT-2-small groups in one call -- on two streams,
    the two 768 x 3072 Gram-form groups on the caller's with their momentum
    passes before the fork, the 48 x [768, 768] plain group on the second --
    equal three separate one-group calls (one stream each) bit for bit, and
    the first matrix of each group the oracle."""
    specs = [(48, 768, 768), (12, 3072, 768), (12, 768, 3072)]
    grouped_vs_separate(specs, seed=2024, ns_check=lambda b, r, c, i: i == 0)


def test_llama1b_groups_equal_separate_calls():
    """The 1B rank-0 share's four groups in one call -- on two streams, three
    classes (2048-row Gram groups on 256 tiles, one with X X^T split along K;
    the 512-row Gram group on 128 tiles; the square plain group), the Gram
    class on the caller's stream -- equal four separate one-group calls bit
    for bit; momentum and post-step of every matrix against the oracle (its
    Newton-Schulz is checked against float64 in the full-size test)."""
    specs = [(2, 11264, 2048), (2, 2048, 5632), (4, 2048, 2048), (4, 512, 2048)]
    grouped_vs_separate(specs, seed=4096, ns_check=lambda b, r, c, i: False)


def test_groups_of_768_to_1023_rows_on_256_tiles():
    """Groups whose short side is 768 or 897..1023 take 256 x 256 tiles when
    those pad it no further than 128 x 128 would: beside a 4096^2 group the
    3 x [768, 2000] and 2 x [960, 1500] groups run their symmetric products on
    256 tiles (174 X X^T workgroups in all, so on two streams), alone on 128
    tiles (too few 256-tiles of their own).  Every matrix equals the separate
    calls' bit for bit; the 768- and 960-row matrices against the oracle."""
    specs = [(3, 768, 2000), (2, 960, 1500), (1, 4096, 4096)]
    grouped_vs_separate(specs, seed=555, ns_check=lambda b, r, c, i: r < 4096)


@pytest.mark.parametrize("ns_steps", [1, 5])
def test_split_reduction_groups(ns_steps):
    """X X^T split along K (a group whose reduction is at least 8192 long and
    whose upper-triangle tiles of 256 are too few to fill the GPU): ragged
    shapes of both orientations, on 256 tiles beside a 4096^2 group in the
    grouped call and on 128 tiles in the separate ones -- each split matrix
    against the oracle, every matrix against the separate calls bit for bit;
    one iteration puts the pre-scale in the fix-up."""
    specs = [(1, 1100, 8300), (2, 8200, 1030), (1, 4096, 4096)]
    grouped_vs_separate(specs, seed=77, ns_steps=ns_steps, ns_check=lambda b, r, c, i: r != c)


def test_binding_rejects_bad_tensors():
    """The binding checks every tensor of a grouped call before anything is
    enqueued: a wrong dtype, a non-contiguous view, a wrong shape or a host
    tensor anywhere in a group is an error naming the group, list and index,
    and the good call on the same buffers still runs."""
    def good():
        return [([torch.zeros(64, 96, device=DEV) for _ in range(3)],
                 [torch.zeros(64, 96, device=DEV) for _ in range(3)],
                 [torch.zeros(64, 96, dtype=torch.bfloat16, device=DEV) for _ in range(3)],
                 [torch.zeros(64, 96, dtype=torch.bfloat16, device=DEV) for _ in range(3)]),
                ([torch.zeros(32, 32, device=DEV)], [torch.zeros(32, 32, device=DEV)],
                 [torch.zeros(32, 32, dtype=torch.bfloat16, device=DEV)],
                 [torch.zeros(32, 32, dtype=torch.bfloat16, device=DEV)])]
    cases = [
        ((0, 2, 2), torch.zeros(64, 96, device=DEV), TypeError, "group 0 grad[2]: dtype"),
        ((0, 0, 1), torch.zeros(96, 64, device=DEV).t(), ValueError, "group 0 master[1]: must be contiguous"),
        ((1, 3, 0), torch.zeros(32, 33, dtype=torch.bfloat16, device=DEV), ValueError,
         "group 1 weight[0]: shape (32, 33)"),
        ((0, 1, 0), torch.zeros(64, 96), ValueError, "group 0 momentum[0]: must be a GPU tensor"),
    ]
    for (gi, li, i), bad, exc, msg in cases:
        groups = good()
        groups[gi][li][i] = bad
        with pytest.raises(exc, match=re.escape(msg)):
            z.muon_step_groups(groups, 1e-3, 0.95, True, 0.1, 5)
    z.muon_step_groups(good(), 1e-3, 0.95, True, 0.1, 5)
    torch.cuda.synchronize()
