"""GPU parity of zopt_muon_step_groups_guarded: the Newton-Schulz health
figures and the divergence guard, against the oracle.

The bars, per matrix, on the GPU's own bf16 result O (read from the
workspace) given to the oracle's ns_health:
  * absmax and the rejected flag equal the oracle's (both exact: a maximum
    and a comparison);
  * the ratio within 2 ulps (the squares are exact in double on both sides;
    only the summation order differs, far below a binary32 ulp);
  * the totals: the rejected count equal, the worst passing ratio within 2
    ulps of the oracle's ns_call_health;
  * updates: a matrix that passes gets bit for bit what the unguarded call
    gives it; a rejected matrix keeps its master and weight, and its momentum
    has taken its step like every other.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LR, MU, WD = (float(np.float32(x)) for x in (8e-4, 0.95, 0.1))
SENTINEL = 3.0


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t):
    return t.cpu().numpy().view(np.uint32)


def ulps(a, b):
    a, b = np.float32(a), np.float32(b)
    return abs(int(a.view(np.int32)) - int(b.view(np.int32)))


def host_inputs(specs, seed, nan_at=None):
    out = []
    for k, (b, r, c) in enumerate(specs):
        rng = np.random.default_rng(seed + 31 * k)
        P = [(rng.standard_normal((r, c)) * 0.02).astype(np.float32) for _ in range(b)]
        G = []
        for i in range(b):
            g = rng.standard_normal((r, c)) * 1e-3
            g[rng.random((r, c)) < 0.01] *= 100.0
            bits = wl.to_bf16_bits(g.astype(np.float32))
            if nan_at == (k, i):
                bits[r // 2, c // 3] = 0x7FC0
            G.append(bits)
        M = [(rng.standard_normal((r, c)) * 1e-3).astype(np.float32) for _ in range(b)]
        out.append((P, M, G))
    return out


def upload(specs, host):
    groups = []
    for (b, r, c), (P, M, G) in zip(specs, host):
        groups.append(([torch.from_numpy(p.copy()).to(DEV) for p in P],
                       [torch.from_numpy(m.copy()).to(DEV) for m in M],
                       [torch.from_numpy(g.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
                        for g in G],
                       [torch.full((r, c), SENTINEL, dtype=torch.bfloat16, device=DEV)
                        for _ in range(b)]))
    return groups


def run(specs, seed, ns_steps, guard, nan_at=None, guard_from=None):
    """Unguarded and guarded calls on the same inputs; returns everything the
    checks need.  guard_from(list of per-matrix absmax) picks the guard from
    the unguarded call's results when given."""
    host = host_inputs(specs, seed, nan_at)
    plain = upload(specs, host)
    ws = z.muon_step_groups(plain, LR, MU, True, WD, ns_steps)
    torch.cuda.synchronize()
    os_ = [oracle.bf16_bits_to_f32(u16(z.muon_groups_output_view(ws, specs, ns_steps, k, i)))
           for k, (b, r, c) in enumerate(specs) for i in range(b)]
    if guard_from is not None:
        guard = guard_from([oracle.ns_health(o)[1] for o in os_])
    nmat = sum(b for b, _, _ in specs)
    health = torch.full((2 + 3 * nmat,), -7.0, dtype=torch.float32, device=DEV)
    guarded = upload(specs, host)
    ws2 = z.muon_step_groups(guarded, LR, MU, True, WD, ns_steps, ns_guard=guard,
                             ns_health=health)
    torch.cuda.synchronize()
    os2 = [oracle.bf16_bits_to_f32(u16(z.muon_groups_output_view(ws2, specs, ns_steps, k, i)))
           for k, (b, r, c) in enumerate(specs) for i in range(b)]
    return host, plain, guarded, os_, os2, health.cpu().numpy(), guard


def check(specs, host, plain, guarded, os_, os2, health, guard):
    nmat = len(os_)
    rej_want, worst_want, rows = oracle.ns_call_health(os2, guard)
    j = 0
    for k, (b, r, c) in enumerate(specs):
        P, M, G = host[k]
        for i in range(b):
            # the guard does not change Newton-Schulz itself
            assert np.array_equal(os_[j].view(np.uint32), os2[j].view(np.uint32))
            got = health[2 + 3 * j: 5 + 3 * j]
            want = rows[j]
            assert ulps(got[0], want[0]) <= 2, (k, i, got, want)
            if np.isnan(want[1]):
                assert np.isnan(got[1])
            else:
                assert got[1] == want[1], (k, i, got, want)
            assert got[2] == want[2]
            gp, gm, gw = guarded[0 + k][0][i], guarded[k][1][i], guarded[k][3][i]
            pp, pm, pw = plain[k][0][i], plain[k][1][i], plain[k][3][i]
            m = M[i].copy()
            oracle.muon_pre(m, G[i], MU, True)
            gmv = gm.cpu().numpy()
            nan = np.isnan(m)
            assert np.array_equal(np.isnan(gmv), nan)     # NaN payloads may differ
            assert np.array_equal(gmv[~nan].view(np.uint32), m[~nan].view(np.uint32))
            if want[2]:
                assert np.array_equal(bits32(gp), P[i].view(np.uint32)), ("rejected moved", k, i)
                assert bool((gw == SENTINEL).all())
            else:
                assert np.array_equal(bits32(gp), bits32(pp)), ("passed differs", k, i)
                assert np.array_equal(u16(gw), u16(pw))
            j += 1
    assert j == nmat
    assert health[0] == rej_want
    assert ulps(health[1], worst_want) <= 2, (health[1], worst_want)
    return rej_want


SPECS = [(3, 200, 520), (2, 1100, 1300), (2, 520, 200), (4, 96, 64), (1, 768, 3072)]


def test_healthy_step_nothing_rejected():
    """Five groups over all tile sizes and both orientations, 5 iterations,
    the pages' guard of 1000: ratios near 1, nothing rejected, every update
    as the unguarded call's."""
    out = run(SPECS, seed=5, ns_steps=5, guard=1000.0)
    assert check(SPECS, *out) == 0
    health = out[5]
    ratios = health[2::3][: sum(b for b, _, _ in SPECS)]
    assert np.all(np.abs(ratios - 1.0) < 0.35), ratios


@pytest.mark.parametrize("ns_steps", [0, 2, 5])
def test_guard_rejects_exactly_the_matrices_above_it(ns_steps):
    """The guard set at the median of the matrices' absmax: those above are
    rejected and left untouched, the rest updated as without the guard."""
    out = run(SPECS, seed=11 + ns_steps, ns_steps=ns_steps, guard=None,
              guard_from=lambda amax: float(np.median(amax)))
    rej = check(SPECS, *out)
    assert 0 < rej < 12


def test_guard_edge_is_inclusive():
    """A guard equal to a matrix's absmax lets it pass; the next float below
    rejects it."""
    specs = [(2, 130, 260), (1, 300, 300)]
    out = run(specs, seed=3, ns_steps=5, guard=None, guard_from=lambda amax: float(amax[1]))
    check(specs, *out)
    assert out[5][2 + 3 * 1 + 2] == 0.0
    out = run(specs, seed=3, ns_steps=5, guard=None,
              guard_from=lambda amax: float(np.nextafter(np.float32(amax[1]), np.float32(0))))
    check(specs, *out)
    assert out[5][2 + 3 * 1 + 2] == 1.0


def test_nan_matrix_is_rejected_alone():
    """A NaN gradient in one matrix makes its whole result NaN: that matrix
    alone is rejected (guard +inf: report only for the rest)."""
    out = run(SPECS, seed=21, ns_steps=5, guard=float("inf"), nan_at=(1, 1))
    assert check(SPECS, *out) == 1
    health = out[5]
    j = 3 + 1   # group 1, matrix 1
    assert np.isnan(health[2 + 3 * j + 1]) and health[2 + 3 * j + 2] == 1.0


def test_gpt2_small_guarded_call():
    """The headline's 72 matrices in one guarded call: nothing rejected, every
    update bit for bit as the unguarded call's, ratios against the oracle."""
    specs = [(g.count, g.rows, g.cols) for g in wl.GPT2_MUON.groups]
    out = run(specs, seed=8, ns_steps=5, guard=1000.0)
    assert check(specs, *out) == 0
