"""The C ABI of libzopt, without a GPU: the library loads, exports every
function include/zopt.h declares, and rejects bad arguments synchronously,
before any HIP call (so these tests run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

import oracle
import sharded_optimizer_step_adamw_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zopt.h")
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(zopt_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"zopt_adamw_shard_step", "zopt_muon_step", "zopt_round_bf16"} <= set(names)
    lib = z.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = z.lib()
    for s in range(6):
        assert lib.zopt_status_string(s).decode().startswith("ZOPT_")


@pytest.mark.parametrize("n,bucket,world", [(1, 1, 1), (10, 3, 4), (4103, 1000, 4),
                                            (2_000_000_000, 1 << 25, 8), (5, 100, 8),
                                            (1 << 14, 1 << 12, 8), (999, 7, 3)])
def test_shard_len_matches_oracle(n, bucket, world):
    assert z.shard_len(n, bucket, world) == oracle.shard_len(n, bucket, world)


def test_shard_len_rejects_bad_sizes():
    for args in ((0, 4, 1), (10, 0, 1), (10, 4, 0)):
        assert z.lib().zopt_shard_len(*args) == -1


def test_ns_workgroup_limit_checks():
    L = z.lib()
    assert L.zopt_set_ns_workgroup_limit(-1) == z.ZOPT_ERR_SIZE
    assert L.zopt_set_ns_workgroup_limit(16) == z.ZOPT_OK
    assert L.zopt_set_ns_workgroup_limit(0) == z.ZOPT_OK


def test_ns_form_checks():
    L = z.lib()
    assert L.zopt_set_ns_form(3) == z.ZOPT_ERR_HYPER
    assert L.zopt_set_ns_form(-1) == z.ZOPT_ERR_HYPER
    assert L.zopt_set_ns_form(z.NS_FORM_PLAIN) == z.ZOPT_OK
    assert L.zopt_set_ns_form(z.NS_FORM_GRAM_BF16) == z.ZOPT_OK
    assert L.zopt_set_ns_form(z.NS_FORM_AUTO) == z.ZOPT_OK


def adamw(**kw):
    a = dict(master=FAKE, exp_avg=FAKE, exp_avg_sq=FAKE, grad=FAKE, weight=None, N=16,
             bucket=8, world=2, rank=0, shard_len=8, lr=1e-3, beta1=0.9, beta2=0.95,
             eps=1e-8, wd=0.1, step=1, grad_scale=1.0, stream=None)
    a.update(kw)
    return z.lib().zopt_adamw_shard_step(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(master=None), z.ZOPT_ERR_NULL), (dict(exp_avg=None), z.ZOPT_ERR_NULL),
    (dict(exp_avg_sq=None), z.ZOPT_ERR_NULL), (dict(grad=None), z.ZOPT_ERR_NULL),
    (dict(N=0), z.ZOPT_ERR_SIZE), (dict(bucket=0), z.ZOPT_ERR_SIZE),
    (dict(world=0), z.ZOPT_ERR_SIZE), (dict(rank=2), z.ZOPT_ERR_SIZE),
    (dict(rank=-1), z.ZOPT_ERR_SIZE), (dict(shard_len=9), z.ZOPT_ERR_SIZE),
    (dict(shard_len=7), z.ZOPT_ERR_SIZE),
    (dict(lr=-1e-3), z.ZOPT_ERR_HYPER), (dict(lr=float("nan")), z.ZOPT_ERR_HYPER),
    (dict(beta1=1.0), z.ZOPT_ERR_HYPER), (dict(beta2=-0.1), z.ZOPT_ERR_HYPER),
    (dict(eps=0.0), z.ZOPT_ERR_HYPER), (dict(eps=float("inf")), z.ZOPT_ERR_HYPER),
    (dict(wd=-0.1), z.ZOPT_ERR_HYPER), (dict(step=0), z.ZOPT_ERR_HYPER),
    (dict(grad_scale=float("inf")), z.ZOPT_ERR_HYPER),
])
def test_adamw_rejects(kw, status):
    assert adamw(**kw) == status


def adamw_clipped(**kw):
    a = dict(master=FAKE, exp_avg=FAKE, exp_avg_sq=FAKE, grad=FAKE, weight=None, N=16,
             bucket=8, world=2, rank=0, shard_len=8, lr=1e-3, beta1=0.9, beta2=0.95,
             eps=1e-8, wd=0.1, step=1, stats=FAKE, skip=0, stream=None)
    a.update(kw)
    return z.lib().zopt_adamw_shard_step_clipped(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(master=None), z.ZOPT_ERR_NULL), (dict(grad=None), z.ZOPT_ERR_NULL),
    (dict(stats=None), z.ZOPT_ERR_NULL),
    (dict(N=0), z.ZOPT_ERR_SIZE), (dict(rank=2), z.ZOPT_ERR_SIZE),
    (dict(shard_len=9), z.ZOPT_ERR_SIZE),
    (dict(lr=float("nan")), z.ZOPT_ERR_HYPER), (dict(beta1=1.0), z.ZOPT_ERR_HYPER),
    (dict(eps=0.0), z.ZOPT_ERR_HYPER), (dict(step=0), z.ZOPT_ERR_HYPER),
    (dict(skip=2), z.ZOPT_ERR_HYPER), (dict(skip=-1), z.ZOPT_ERR_HYPER),
])
def test_adamw_clipped_rejects(kw, status):
    assert adamw_clipped(**kw) == status


def sq_norm(**kw):
    size = ctypes.c_size_t(1 << 20)
    a = dict(grad=FAKE, N=16, bucket=8, world=2, rank=0, shard_len=8, sq=FAKE,
             ws=ctypes.c_void_p(1 << 20), ws_bytes=ctypes.byref(size), stream=None)
    a.update(kw)
    return z.lib().zopt_grad_sq_norm(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(grad=None), z.ZOPT_ERR_NULL), (dict(sq=None), z.ZOPT_ERR_NULL),
    (dict(ws_bytes=None), z.ZOPT_ERR_NULL),
    (dict(N=0), z.ZOPT_ERR_SIZE), (dict(bucket=0), z.ZOPT_ERR_SIZE),
    (dict(world=0), z.ZOPT_ERR_SIZE), (dict(rank=2), z.ZOPT_ERR_SIZE),
    (dict(shard_len=9), z.ZOPT_ERR_SIZE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), z.ZOPT_ERR_WORKSPACE),
    (dict(ws_bytes=ctypes.byref(ctypes.c_size_t(8))), z.ZOPT_ERR_WORKSPACE),
])
def test_grad_sq_norm_rejects(kw, status):
    assert sq_norm(**kw) == status


@pytest.mark.parametrize("n,bucket,world", [(16, 8, 2), (2_000_000_000, 1 << 25, 8), (1, 1, 1)])
def test_grad_sq_norm_workspace_query(n, bucket, world):
    size = ctypes.c_size_t(0)
    sl = z.shard_len(n, bucket, world)
    st = z.lib().zopt_grad_sq_norm(None, n, bucket, world, 0, sl, None, None,
                                   ctypes.byref(size), None)
    assert st == z.ZOPT_OK
    assert 256 <= size.value <= 16384 and size.value % 256 == 0
    assert z.grad_sq_norm_workspace_bytes(n, bucket, world) == size.value


@pytest.mark.parametrize("kw,status", [
    (dict(sq=None), z.ZOPT_ERR_NULL), (dict(stats=None), z.ZOPT_ERR_NULL),
    (dict(count=0), z.ZOPT_ERR_SIZE), (dict(count=65537), z.ZOPT_ERR_SIZE),
    (dict(max_norm=0.0), z.ZOPT_ERR_HYPER), (dict(max_norm=-1.0), z.ZOPT_ERR_HYPER),
    (dict(max_norm=float("nan")), z.ZOPT_ERR_HYPER),
    (dict(inv_scale=0.0), z.ZOPT_ERR_HYPER), (dict(inv_scale=float("inf")), z.ZOPT_ERR_HYPER),
])
def test_grad_clip_stats_rejects(kw, status):
    a = dict(sq=FAKE, count=1, max_norm=1.0, inv_scale=1.0, stats=FAKE, stream=None)
    a.update(kw)
    assert z.lib().zopt_grad_clip_stats(*a.values()) == status


def test_round_bf16_rejects_and_empty_is_a_noop():
    lib = z.lib()
    assert lib.zopt_round_bf16(FAKE, FAKE, -1, None) == z.ZOPT_ERR_SIZE
    assert lib.zopt_round_bf16(None, FAKE, 4, None) == z.ZOPT_ERR_NULL
    assert lib.zopt_round_bf16(FAKE, None, 4, None) == z.ZOPT_ERR_NULL
    assert lib.zopt_round_bf16(None, None, 0, None) == z.ZOPT_OK  # nothing enqueued


def ptrs(k, null_at=None):
    arr = (ctypes.c_void_p * k)()
    for i in range(k):
        arr[i] = None if i == null_at else 0x100000 + 0x1000 * i
    return arr


def muon(**kw):
    size = ctypes.c_size_t(1 << 40)
    a = dict(batch=2, rows=64, cols=32, master=ptrs(2), momentum=ptrs(2), grad=ptrs(2),
             weight=None, lr=8e-4, mu=0.95, nesterov=1, wd=0.1, ns_steps=5, a=3.4445,
             b=-4.775, c=2.0315, eps=1e-7, adjust=1, ws=ctypes.c_void_p(1 << 20),
             ws_bytes=ctypes.byref(size), stream=None)
    a.update(kw)
    return z.lib().zopt_muon_step(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), z.ZOPT_ERR_SIZE), (dict(batch=65), z.ZOPT_ERR_SIZE),
    (dict(rows=0), z.ZOPT_ERR_SIZE), (dict(cols=-3), z.ZOPT_ERR_SIZE),
    (dict(rows=1 << 16, cols=1 << 15), z.ZOPT_ERR_SIZE),
    # thin, long matrices past the 2^21 side limit (element count below 2^31):
    # 32-bit panel offsets of the Newton-Schulz kernels would wrap
    (dict(rows=8, cols=250_000_000), z.ZOPT_ERR_SIZE),
    (dict(rows=30_000_000, cols=64), z.ZOPT_ERR_SIZE),
    (dict(rows=1, cols=(1 << 31) - 1), z.ZOPT_ERR_SIZE),
    (dict(rows=(1 << 21) + 1, cols=1), z.ZOPT_ERR_SIZE),
    (dict(master=None), z.ZOPT_ERR_NULL), (dict(grad=ptrs(2, null_at=1)), z.ZOPT_ERR_NULL),
    (dict(weight=ptrs(2, null_at=0)), z.ZOPT_ERR_NULL), (dict(ws_bytes=None), z.ZOPT_ERR_NULL),
    (dict(lr=-1.0), z.ZOPT_ERR_HYPER), (dict(mu=1.0), z.ZOPT_ERR_HYPER),
    (dict(nesterov=2), z.ZOPT_ERR_HYPER), (dict(wd=float("nan")), z.ZOPT_ERR_HYPER),
    (dict(ns_steps=-1), z.ZOPT_ERR_HYPER), (dict(ns_steps=101), z.ZOPT_ERR_HYPER),
    (dict(b=float("inf")), z.ZOPT_ERR_HYPER), (dict(eps=-1.0), z.ZOPT_ERR_HYPER),
    (dict(adjust=2), z.ZOPT_ERR_HYPER),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), z.ZOPT_ERR_WORKSPACE),
])
def test_muon_rejects(kw, status):
    assert muon(**kw) == status


def test_muon_side_limit_is_inclusive():
    # 2^21 on the longer side is accepted (the workspace query answers)
    for rows, cols in ((1, 1 << 21), (1 << 21, 512), (1023, 1 << 21)):
        assert z.muon_workspace_bytes(1, rows, cols) > 0


def test_muon_workspace_query_and_too_small():
    need = z.muon_workspace_bytes(2, 64, 32)
    assert need > 0 and need % 256 == 0
    small = ctypes.c_size_t(need - 1)
    assert muon(ws_bytes=ctypes.byref(small)) == z.ZOPT_ERR_WORKSPACE
    # larger problems need more; the query enqueues nothing
    assert z.muon_workspace_bytes(4, 64, 32) > need
    assert z.muon_workspace_bytes(1, 4096, 14336) >= 3 * 4096 * 14336 * 2


def test_output_view_locates_inside_the_workspace():
    lib = z.lib()
    out, ld = ctypes.c_void_p(), ctypes.c_int64()
    base = 1 << 20
    need = z.muon_workspace_bytes(3, 100, 300)
    for rows, cols in ((100, 300), (300, 100)):
        for steps in (0, 1, 5):
            for i in range(3):
                st = lib.zopt_muon_output_view(3, rows, cols, steps, ctypes.c_void_p(base), i,
                                               ctypes.byref(out), ctypes.byref(ld))
                assert st == z.ZOPT_OK
                assert ld.value >= cols
                end = out.value + 2 * ((rows - 1) * ld.value + cols)
                assert base <= out.value and end <= base + need
    assert lib.zopt_muon_output_view(3, 100, 300, 5, ctypes.c_void_p(base), 3,
                                     ctypes.byref(out), ctypes.byref(ld)) == z.ZOPT_ERR_SIZE
    assert lib.zopt_muon_output_view(3, 100, 300, 5, None, 0, ctypes.byref(out),
                                     ctypes.byref(ld)) == z.ZOPT_ERR_NULL


def groups_call(ngroups=2, batch=(2, 1), rows=(64, 300), cols=(32, 100), ws=None, ws_bytes=None):
    lib = z.lib()
    n = len(batch)
    b = (ctypes.c_int32 * n)(*batch)
    r = (ctypes.c_int64 * n)(*rows)
    c = (ctypes.c_int64 * n)(*cols)
    size = ctypes.c_size_t(0) if ws_bytes is None else ws_bytes
    st = lib.zopt_muon_step_groups(ngroups, b, r, c, None, None, None, None, 0.0, 0.0, 0, 0.0, 0,
                                   0.0, 0.0, 0.0, 0.0, 0, ws, ctypes.byref(size), None)
    return st, size.value


def test_groups_workspace_is_the_sum_of_the_groups():
    shapes = [(2, 64, 32), (1, 300, 100), (3, 1100, 1300)]
    total = z.muon_groups_workspace_bytes(shapes)
    assert total == sum(z.muon_workspace_bytes(*s) for s in shapes)
    assert z.muon_groups_workspace_bytes(shapes[:1]) == z.muon_workspace_bytes(*shapes[0])


def test_groups_reject():
    assert groups_call(ngroups=0)[0] == z.ZOPT_ERR_SIZE
    assert groups_call(ngroups=17, batch=(1,) * 17, rows=(8,) * 17, cols=(8,) * 17)[0] == \
        z.ZOPT_ERR_SIZE
    assert groups_call(batch=(2, 0))[0] == z.ZOPT_ERR_SIZE
    assert groups_call(batch=(2, 65))[0] == z.ZOPT_ERR_SIZE
    assert groups_call(rows=(64, 0))[0] == z.ZOPT_ERR_SIZE
    lib = z.lib()
    size = ctypes.c_size_t(0)
    st = lib.zopt_muon_step_groups(1, None, None, None, None, None, None, None, 0.0, 0.0, 0, 0.0,
                                   0, 0.0, 0.0, 0.0, 0.0, 0, None, ctypes.byref(size), None)
    assert st == z.ZOPT_ERR_NULL
    # a non-NULL workspace with NULL matrix pointers is rejected before any launch
    st, _ = groups_call(ws=ctypes.c_void_p(1 << 20), ws_bytes=ctypes.c_size_t(1 << 40))
    assert st == z.ZOPT_ERR_NULL


def test_groups_output_views_are_disjoint_and_in_bounds():
    lib = z.lib()
    shapes = [(2, 100, 300), (3, 300, 100), (1, 1100, 1300)]
    n = len(shapes)
    b = (ctypes.c_int32 * n)(*[s[0] for s in shapes])
    r = (ctypes.c_int64 * n)(*[s[1] for s in shapes])
    c = (ctypes.c_int64 * n)(*[s[2] for s in shapes])
    total = z.muon_groups_workspace_bytes(shapes)
    base = 1 << 20
    out, ld = ctypes.c_void_p(), ctypes.c_int64()
    spans = []
    for steps in (0, 5):
        spans.clear()
        for g, (batch, rows, cols) in enumerate(shapes):
            for i in range(batch):
                st = lib.zopt_muon_groups_output_view(n, b, r, c, steps, ctypes.c_void_p(base), g,
                                                      i, ctypes.byref(out), ctypes.byref(ld))
                assert st == z.ZOPT_OK
                lo = out.value - base
                hi = lo + 2 * ((rows - 1) * ld.value + cols)
                assert 0 <= lo and hi <= total and ld.value >= cols
                spans.append((lo, hi))
        spans.sort()
        assert all(spans[k][1] <= spans[k + 1][0] for k in range(len(spans) - 1))
    assert lib.zopt_muon_groups_output_view(n, b, r, c, 5, ctypes.c_void_p(base), 3, 0,
                                            ctypes.byref(out), ctypes.byref(ld)) == z.ZOPT_ERR_SIZE
    assert lib.zopt_muon_groups_output_view(n, b, r, c, 5, ctypes.c_void_p(base), 1, 3,
                                            ctypes.byref(out), ctypes.byref(ld)) == z.ZOPT_ERR_SIZE


def guarded(**kw):
    size = ctypes.c_size_t(1 << 40)
    a = dict(ngroups=1, batch=(ctypes.c_int32 * 1)(2), rows=(ctypes.c_int64 * 1)(64),
             cols=(ctypes.c_int64 * 1)(32), master=ptrs(2), momentum=ptrs(2), grad=ptrs(2),
             weight=None, lr=8e-4, mu=0.95, nesterov=1, wd=0.1, ns_steps=5, a=3.4445,
             b=-4.775, c=2.0315, eps=1e-7, adjust=1, guard=1000.0, health=FAKE,
             ws=ctypes.c_void_p(1 << 20), ws_bytes=ctypes.byref(size), stream=None)
    a.update(kw)
    return z.lib().zopt_muon_step_groups_guarded(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(health=None), z.ZOPT_ERR_NULL),
    (dict(guard=0.0), z.ZOPT_ERR_HYPER), (dict(guard=-5.0), z.ZOPT_ERR_HYPER),
    (dict(guard=float("nan")), z.ZOPT_ERR_HYPER),
    (dict(batch=(ctypes.c_int32 * 1)(0)), z.ZOPT_ERR_SIZE),
    (dict(master=None), z.ZOPT_ERR_NULL), (dict(lr=-1.0), z.ZOPT_ERR_HYPER),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), z.ZOPT_ERR_WORKSPACE),
])
def test_muon_guarded_rejects(kw, status):
    assert guarded(**kw) == status


def test_muon_guarded_query_needs_no_health():
    size = ctypes.c_size_t(0)
    assert guarded(health=None, guard=0.0, ws=None, ws_bytes=ctypes.byref(size)) == z.ZOPT_OK
    assert size.value == z.muon_workspace_bytes(2, 64, 32)


def graph_create(**kw):
    out = ctypes.c_void_p(0x1234)
    a = dict(ngroups=1, batch=(ctypes.c_int32 * 1)(2), rows=(ctypes.c_int64 * 1)(64),
             cols=(ctypes.c_int64 * 1)(32), master=ptrs(2), momentum=ptrs(2), grad=ptrs(2),
             weight=None, scalars=FAKE, nesterov=1, ns_steps=5, a=3.4445, b=-4.775, c=2.0315,
             eps=1e-7, adjust=1, guard=1000.0, health=None, ws=ctypes.c_void_p(1 << 20),
             ws_bytes=1 << 40, out=ctypes.byref(out))
    a.update(kw)
    st = z.lib().zopt_muon_graph_create(*a.values())
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), z.ZOPT_ERR_NULL), (dict(scalars=None), z.ZOPT_ERR_NULL),
    (dict(ws=None), z.ZOPT_ERR_NULL), (dict(master=None), z.ZOPT_ERR_NULL),
    (dict(grad=ptrs(2, null_at=1)), z.ZOPT_ERR_NULL),
    (dict(batch=(ctypes.c_int32 * 1)(65)), z.ZOPT_ERR_SIZE), (dict(ngroups=0), z.ZOPT_ERR_SIZE),
    (dict(nesterov=3), z.ZOPT_ERR_HYPER), (dict(ns_steps=101), z.ZOPT_ERR_HYPER),
    (dict(c=float("nan")), z.ZOPT_ERR_HYPER), (dict(adjust=-1), z.ZOPT_ERR_HYPER),
    (dict(health=FAKE, guard=0.0), z.ZOPT_ERR_HYPER),
    (dict(ws=ctypes.c_void_p((1 << 20) + 8)), z.ZOPT_ERR_WORKSPACE),
    (dict(ws_bytes=1000), z.ZOPT_ERR_WORKSPACE),
])
def test_muon_graph_create_rejects_before_any_hip_call(kw, status):
    st, handle = graph_create(**kw)
    assert st == status
    if kw.get("out", 1) is not None:
        assert handle is None   # the handle is cleared on every error


def test_muon_graph_launch_and_destroy_null():
    assert z.lib().zopt_muon_graph_launch(None, None) == z.ZOPT_ERR_NULL
    assert z.lib().zopt_muon_graph_destroy(None) == z.ZOPT_OK
