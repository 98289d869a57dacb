"""GPU parity of the captured Muon call (zopt_muon_graph_*) against eager
calls and the oracle.

The bar: every replay gives bit for bit what zopt_muon_step_groups (or its
guarded form) gives for the same inputs and the same lr / momentum / weight
decay -- which the graph reads from device memory when it runs -- on
several replays in a row with the scalars changed between them and the
program's own eager work and synchronisations in between.  One replay is
also checked against the oracle stage by stage (momentum bitwise, post-step
teacher-forced on the GPU's own Newton-Schulz result).
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SCHEDULE = [(8e-4, 0.95, 0.1), (6e-4, 0.9, 0.05), (1e-5, 0.0, 0.0), (2e-3, 0.99, 0.2)]


def f32(x):
    return float(np.float32(x))


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


def host_inputs(specs, seed):
    out = []
    for k, (b, r, c) in enumerate(specs):
        rng = np.random.default_rng(seed + 17 * k)
        P = [(rng.standard_normal((r, c)) * 0.02).astype(np.float32) for _ in range(b)]
        M = [(rng.standard_normal((r, c)) * 1e-3).astype(np.float32) for _ in range(b)]
        out.append((P, M, rng))
    return out


def upload(specs, host):
    groups = []
    for (b, r, c), (P, M, _) in zip(specs, host):
        groups.append(([torch.from_numpy(p.copy()).to(DEV) for p in P],
                       [torch.from_numpy(m.copy()).to(DEV) for m in M],
                       [torch.empty((r, c), dtype=torch.bfloat16, device=DEV) for _ in range(b)],
                       [torch.full((r, c), 3.0, dtype=torch.bfloat16, device=DEV)
                        for _ in range(b)]))
    return groups


def new_grads(specs, rng, step):
    """Fresh bf16 gradients per step (the same bits fed to both paths)."""
    return [[wl.to_bf16_bits((rng.standard_normal((r, c)) * 1e-3 * (1 + step)).astype(np.float32))
             for _ in range(b)] for (b, r, c) in specs]


def set_grads(groups, grads):
    for (_, _, G, _), gs in zip(groups, grads):
        for t, g in zip(G, gs):
            t.copy_(torch.from_numpy(g.view(np.int16).copy()).to(DEV).view(torch.bfloat16))


def compare(a, b, where):
    for ga, gb in zip(a, b):
        for ta, tb in zip(ga[0] + ga[1], gb[0] + gb[1]):
            assert np.array_equal(bits(ta), bits(tb)), where
        for ta, tb in zip(ga[3], gb[3]):
            assert np.array_equal(u16(ta), u16(tb)), where


def replay_vs_eager(specs, seed, ns_steps=5, guard=None, steps=4, oracle_check=False):
    host = host_inputs(specs, seed)
    eager, graphed = upload(specs, host), upload(specs, host)
    nmat = sum(b for b, _, _ in specs)
    scalars = torch.empty(3, dtype=torch.float32, device=DEV)
    h_graph = h_eager = None
    if guard is not None:
        h_graph = torch.zeros(2 + 3 * nmat, dtype=torch.float32, device=DEV)
        h_eager = torch.zeros_like(h_graph)
    graph = z.MuonGraph(graphed, scalars, ns_steps=ns_steps, ns_guard=guard, ns_health=h_graph)
    rng = np.random.default_rng(seed + 1)
    try:
        for t in range(steps):
            lr, mu, wd = (f32(x) for x in SCHEDULE[t % len(SCHEDULE)])
            grads = new_grads(specs, rng, t)
            set_grads(eager, grads)
            set_grads(graphed, grads)
            before = [[p.clone() for p in g[0]] for g in graphed] if oracle_check and t == 1 else None
            mom_before = ([[m.clone() for m in g[1]] for g in graphed]
                          if oracle_check and t == 1 else None)
            scalars.copy_(torch.tensor([lr, mu, wd], dtype=torch.float32))
            graph.launch()
            ws = z.muon_step_groups(eager, lr, mu, True, wd, ns_steps, ns_guard=guard,
                                    ns_health=h_eager)
            torch.cuda.synchronize()
            compare(graphed, eager, ("step", t))
            if guard is not None:
                assert np.array_equal(bits(h_graph), bits(h_eager)), ("health", t)
            if before is not None:
                for k, (b, r, c) in enumerate(specs):
                    for i in range(b):
                        m = mom_before[k][i].cpu().numpy()
                        oracle.muon_pre(m, grads[k][i], mu, True)
                        assert np.array_equal(bits(graphed[k][1][i]), m.view(np.uint32))
                        o = oracle.bf16_bits_to_f32(u16(z.muon_groups_output_view(
                            graph.workspace, specs, ns_steps, k, i)))
                        p = before[k][i].cpu().numpy()
                        w = oracle.muon_post(p, o, lr, wd, 1)
                        assert np.array_equal(bits(graphed[k][0][i]), p.view(np.uint32))
                        assert np.array_equal(u16(graphed[k][3][i]), w)
            del ws
    finally:
        graph.close()


def test_tiny_workload_replays():
    """The tiny Muon workload (2 x [128, 512]), four replays with the
    schedule changing every step, one replay checked against the oracle."""
    replay_vs_eager([(2, 128, 512)], seed=1, oracle_check=True)


def test_mixed_groups_replays():
    """Five groups over all tile sizes and both orientations."""
    replay_vs_eager([(3, 200, 520), (2, 1100, 1300), (2, 520, 200), (4, 96, 64),
                     (1, 768, 3072)], seed=2, steps=3, oracle_check=True)


@pytest.mark.parametrize("ns_steps", [0, 1])
def test_step_counts(ns_steps):
    replay_vs_eager([(2, 130, 260), (1, 700, 300)], seed=3, ns_steps=ns_steps, steps=2)


def test_guarded_replays():
    """With the health pass and the guard inside the graph: the health
    figures and the updates equal the eager guarded call's."""
    replay_vs_eager([(3, 200, 520), (2, 520, 200), (1, 1030, 2100)], seed=4, guard=1000.0,
                    steps=3)


def test_two_stream_call_replays():
    """A call whose Newton-Schulz iterations are divided over two streams
    (three 256-tile groups with 280 X X^T workgroups in all): the captured
    fork and join replay to the eager call's results, with and without the
    health pass."""
    specs = [(1, 4096, 4096), (2, 2048, 2048), (2, 2048, 5632)]
    replay_vs_eager(specs, seed=6, steps=3)
    replay_vs_eager(specs, seed=7, steps=2, guard=1000.0)


def test_gpt2_small_replays():
    """The headline's 72 matrices in one captured call, three replays."""
    specs = [(g.count, g.rows, g.cols) for g in wl.GPT2_MUON.groups]
    replay_vs_eager(specs, seed=5, steps=3)
