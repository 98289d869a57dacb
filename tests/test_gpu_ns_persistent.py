"""The persistent X' = a X + B X launches.  With the resident workgroups
capped (zopt_set_ns_workgroup_limit) every workgroup walks many tiles: walks
that cross from one group to the next inside a launch (different shapes,
strides and reduction lengths), the stage pipeline running on from one tile
into the next, X'^T written on the last iteration for matrices stored
transposed, and launches holding a reduction shorter than the pipeline
(K = 64), where each tile starts its own.  Every tile is computed the same
way whichever workgroup takes it, so results must equal the uncapped call's
bit for bit, and stay within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
from test_gpu_muon import (DEV, NS_TOL, dev_bf16, dev_f32, f32, make_inputs, rel_fro, u16,
                           grouped_vs_separate)

pytestmark = pytest.mark.gpu


@pytest.fixture
def limit():
    yield z.set_ns_workgroup_limit
    z.set_ns_workgroup_limit(0)


SPECS = [(3, 200, 520), (2, 1100, 1300), (2, 1300, 1100), (2, 300, 700), (4, 96, 64),
         (1, 1030, 2100), (2, 520, 200), (3, 768, 768), (2, 1024, 512)]


def run(specs, host, ns_steps):
    lr, mu, wd = f32(8e-4), f32(0.95), f32(0.1)
    calls = []
    for (b, r, c), (P, M, G) in zip(specs, host):
        calls.append(([dev_f32(p) for p in P], [dev_f32(m) for m in M], [dev_bf16(g) for g in G],
                      [torch.full((r, c), 3.0, dtype=torch.bfloat16, device=DEV)
                       for _ in range(b)]))
    ws = z.muon_step_groups(calls, lr, mu, True, wd, ns_steps)
    torch.cuda.synchronize()
    out = []
    for k, (b, r, c) in enumerate(specs):
        gP, gM, _, gW = calls[k]
        for i in range(b):
            out.append((u16(z.muon_groups_output_view(ws, specs, ns_steps, k, i)),
                        gP[i].cpu().numpy().view(np.uint32), gM[i].cpu().numpy().view(np.uint32),
                        u16(gW[i])))
    return out


@pytest.mark.parametrize("ns_steps", [1, 2, 5])
def test_capped_walks_equal_uncapped(limit, ns_steps):
    host = [make_inputs(b, r, c, 500 + 7 * k, momentum_nonzero=True)
            for k, (b, r, c) in enumerate(SPECS)]
    ref = run(SPECS, host, ns_steps)
    for cap in (8, 24, 40):
        print(f"workgroup limit {cap}, ns_steps {ns_steps}", flush=True)
        limit(cap)
        got = run(SPECS, host, ns_steps)
        limit(0)
        for n, (a, b) in enumerate(zip(ref, got)):
            for x, y, what in zip(a, b, ("ns output", "master", "momentum", "weight")):
                assert np.array_equal(x, y), (cap, n, what)


def test_capped_walks_match_oracle(limit):
    """The mixed-tile grouped call under a cap of 8 workgroups, against the
    oracle and against separate calls."""
    limit(8)
    grouped_vs_separate(SPECS, seed=4242, ns_check=lambda b, r, c, i: i == 0 or r * c < 300_000)
