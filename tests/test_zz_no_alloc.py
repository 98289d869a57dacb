"""zopt_grad_sq_norm_noalloc, the allocation-free form of zopt_grad_sq_norm,
through the C ABI: its sum equals the workspace form's bit for bit (the same
kernels, the same fixed order) on two calls in a row, the second on a
smaller shard -- so partials a longer call left in the library's scratch
cannot leak into a shorter one -- and lies within 1e-10 of the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_adamw_amd as z
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def grads(rng, n):
    g = rng.standard_normal(n) * 1e-3
    g[rng.random(n) < 0.01] *= 100.0
    return wl.to_bf16_bits(g.astype(np.float32))


def with_workspace(g, n, bucket, world, rank, stream):
    sl = z.shard_len(n, bucket, world)
    size = ctypes.c_size_t(0)
    L = z.lib()
    assert L.zopt_grad_sq_norm(None, n, bucket, world, rank, sl, None, None,
                               ctypes.byref(size), None) == z.ZOPT_OK
    ws = torch.empty(size.value, dtype=torch.uint8, device=DEV)
    out = torch.full((1,), np.nan, dtype=torch.float64, device=DEV)
    st = L.zopt_grad_sq_norm(g.data_ptr(), n, bucket, world, rank, sl, out.data_ptr(),
                             ws.data_ptr(), ctypes.byref(size), stream)
    assert st == z.ZOPT_OK
    return out


def noalloc(g, n, bucket, world, rank, out, stream):
    sl = z.shard_len(n, bucket, world)
    st = z.lib().zopt_grad_sq_norm_noalloc(g.data_ptr(), n, bucket, world, rank, sl,
                                           out.data_ptr(), stream)
    assert st == z.ZOPT_OK


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    rng = np.random.default_rng(4321)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    cases = [
        (1 << 26, 1 << 22, 8, 3),     # 2048 partials: the whole scratch array
        (100_003, 8192, 4, 1),        # a few partials, padded last bucket
    ]
    outs = [torch.full((1,), np.nan, dtype=torch.float64, device=DEV) for _ in cases]
    inputs = []
    for (n, bucket, world, rank), out in zip(cases, outs):
        gb = grads(rng, n)
        g = torch.from_numpy(gb.view(np.int16)).to(DEV).view(torch.bfloat16)
        inputs.append((gb, g))
        noalloc(g, n, bucket, world, rank, out, stream)
    torch.cuda.synchronize()
    for (n, bucket, world, rank), out, (gb, g) in zip(cases, outs, inputs):
        ref = with_workspace(g, n, bucket, world, rank, stream).item()
        got = out.item()
        print(f"N={n} bucket={bucket} world={world} rank={rank}: {got!r} vs {ref!r}", flush=True)
        assert np.float64(got).view(np.uint64) == np.float64(ref).view(np.uint64)
        want = oracle.grad_sq_norm(gb, n, bucket, world, rank)
        assert abs(got - want) <= 1e-10 * want


def test_noalloc_rejects_before_any_launch():
    L = z.lib()
    fake = ctypes.c_void_p(0x100000)
    assert L.zopt_grad_sq_norm_noalloc(None, 10, 4, 1, 0, 10, fake, None) == z.ZOPT_ERR_NULL
    assert L.zopt_grad_sq_norm_noalloc(fake, 10, 4, 2, 2, 5, fake, None) == z.ZOPT_ERR_SIZE
    assert L.zopt_grad_sq_norm_noalloc(fake, 10, 4, 2, 0, 7, fake, None) == z.ZOPT_ERR_SIZE
