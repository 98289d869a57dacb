"""Python binding of libzopt: one rank's ZeRO-style optimizer step on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libzopt.so`` (built from ``csrc/`` by ``build.py``); this module
checks tensor dtypes, devices and sizes (the C ABI takes plain pointers and
cannot), passes pointers and the current HIP stream, and turns status codes
into exceptions.  PyTorch only supplies device memory and streams.  If the
library is not built, importing the entry points raises -- there is no
fallback.

Entry points (same names as the C ABI in include/zopt.h):
  adamw_shard_step   fused AdamW over a flat bucketed fp32 shard
  muon_step          Muon on a batch of same-shape matrices
  muon_workspace_bytes / muon_output_view
  muon_step_groups   Muon on several such batches in one call (shared launches);
                     with ns_guard: zopt_muon_step_groups_guarded (health checks)
  MuonGraph          a Muon call captured once (zopt_muon_graph_*), replayed per step
                     with lr / momentum / weight decay read from device memory
  muon_groups_workspace_bytes / muon_groups_output_view
  round_bf16         fp32 -> bf16 round-to-nearest-even
  shard_len          the shard length the layout derives (zopt_shard_len)
  grad_sq_norm       sum of squares of a rank's real gradient elements
  grad_sq_norm_noalloc  the same with the library's own scratch (allocates nothing)
  grad_clip_stats    clip statistics (device scalars) from summed squares
  adamw_shard_step_clipped   AdamW taking grad_scale from the clip statistics
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzopt.so")

ZOPT_OK, ZOPT_ERR_NULL, ZOPT_ERR_SIZE, ZOPT_ERR_HYPER, ZOPT_ERR_WORKSPACE, ZOPT_ERR_DEVICE = range(6)
# layout of the clip statistics (ZOPT_CLIP_* in zopt.h)
CLIP_TOTAL_NORM, CLIP_COEF, CLIP_CLIPPED, CLIP_FOUND_INF, CLIP_GRAD_SCALE, CLIP_STATS = range(6)
MAX_BATCH = 64
MAX_GROUPS = 16


class ZoptError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib_or_raise().zopt_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


_lib = None


def _lib_or_raise() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m sharded_optimizer_step_adamw_amd.build` "
                "(or __graft_entry__.build()). There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.zopt_status_string.argtypes = [ctypes.c_int]
        L.zopt_status_string.restype = ctypes.c_char_p
        L.zopt_adamw_shard_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i64,
                                            f32, f32, f32, f32, f32, i64, f32, vp]
        L.zopt_adamw_shard_step.restype = ctypes.c_int
        L.zopt_adamw_shard_step_clipped.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32,
                                                    i64, f32, f32, f32, f32, f32, i64, vp, i32,
                                                    vp]
        L.zopt_adamw_shard_step_clipped.restype = ctypes.c_int
        L.zopt_grad_sq_norm.argtypes = [vp, i64, i64, i32, i32, i64, vp, vp,
                                        ctypes.POINTER(ctypes.c_size_t), vp]
        L.zopt_grad_sq_norm.restype = ctypes.c_int
        L.zopt_grad_sq_norm_noalloc.argtypes = [vp, i64, i64, i32, i32, i64, vp, vp]
        L.zopt_grad_sq_norm_noalloc.restype = ctypes.c_int
        L.zopt_grad_clip_stats.argtypes = [vp, i32, f32, f32, vp, vp]
        L.zopt_grad_clip_stats.restype = ctypes.c_int
        L.zopt_shard_len.argtypes = [i64, i64, i32]
        L.zopt_shard_len.restype = i64
        L.zopt_round_bf16.argtypes = [vp, vp, i64, vp]
        L.zopt_round_bf16.restype = ctypes.c_int
        L.zopt_set_ns_workgroup_limit.argtypes = [i32]
        L.zopt_set_ns_workgroup_limit.restype = ctypes.c_int
        L.zopt_set_ns_form.argtypes = [i32]
        L.zopt_set_ns_form.restype = ctypes.c_int
        pp = ctypes.POINTER(vp)
        L.zopt_muon_step.argtypes = [i32, i64, i64, pp, pp, pp, pp, f32, f32, i32, f32, i32,
                                     f32, f32, f32, f32, i32, vp,
                                     ctypes.POINTER(ctypes.c_size_t), vp]
        L.zopt_muon_step.restype = ctypes.c_int
        L.zopt_muon_output_view.argtypes = [i32, i64, i64, i32, vp, i32, pp,
                                            ctypes.POINTER(i64)]
        L.zopt_muon_output_view.restype = ctypes.c_int
        pi32, pi64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
        L.zopt_muon_step_groups.argtypes = [i32, pi32, pi64, pi64, pp, pp, pp, pp, f32, f32, i32,
                                            f32, i32, f32, f32, f32, f32, i32, vp,
                                            ctypes.POINTER(ctypes.c_size_t), vp]
        L.zopt_muon_step_groups.restype = ctypes.c_int
        L.zopt_muon_step_groups_guarded.argtypes = [
            i32, pi32, pi64, pi64, pp, pp, pp, pp, f32, f32, i32, f32, i32, f32, f32, f32, f32,
            i32, f32, vp, vp, ctypes.POINTER(ctypes.c_size_t), vp]
        L.zopt_muon_step_groups_guarded.restype = ctypes.c_int
        L.zopt_muon_graph_create.argtypes = [
            i32, pi32, pi64, pi64, pp, pp, pp, pp, vp, i32, i32, f32, f32, f32, f32, i32, f32,
            vp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.zopt_muon_graph_create.restype = ctypes.c_int
        L.zopt_muon_graph_launch.argtypes = [vp, vp]
        L.zopt_muon_graph_launch.restype = ctypes.c_int
        L.zopt_muon_graph_destroy.argtypes = [vp]
        L.zopt_muon_graph_destroy.restype = ctypes.c_int
        L.zopt_muon_groups_output_view.argtypes = [i32, pi32, pi64, pi64, i32, vp, i32, i32, pp,
                                                   pi64]
        L.zopt_muon_groups_output_view.restype = ctypes.c_int
        _lib = L
    return _lib


def lib() -> ctypes.CDLL:
    """The loaded libzopt (raises ImportError if it is not built)."""
    return _lib_or_raise()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, numel: int, name: str, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, need {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: has {t.numel()} elements, needs {numel}")


def _check(status: int, where: str) -> None:
    if status != ZOPT_OK:
        raise ZoptError(status, where)


def shard_len(n: int, bucket: int, world: int) -> int:
    """Shard length every rank holds (zopt_shard_len)."""
    v = lib().zopt_shard_len(n, bucket, world)
    if v < 0:
        raise ValueError("shard_len: need n, bucket, world >= 1")
    return int(v)


def adamw_shard_step(master, exp_avg, exp_avg_sq, grad, weight, n, bucket, world, rank,
                     lr, beta1, beta2, eps, weight_decay, step, grad_scale=1.0,
                     shard_len_=None, stream=None) -> None:
    """One fused AdamW step over rank `rank`'s shard (zopt_adamw_shard_step).
    master/exp_avg/exp_avg_sq: fp32 [shard_len]; grad: bf16 [n]; weight:
    bf16 [n] or None."""
    sl = shard_len(n, bucket, world) if shard_len_ is None else shard_len_
    dev = master.device
    _need(master, torch.float32, sl, "master")
    _need(exp_avg, torch.float32, sl, "exp_avg", dev)
    _need(exp_avg_sq, torch.float32, sl, "exp_avg_sq", dev)
    _need(grad, torch.bfloat16, n, "grad", dev)
    if weight is not None:
        _need(weight, torch.bfloat16, n, "weight", dev)
    st = lib().zopt_adamw_shard_step(
        master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), grad.data_ptr(),
        None if weight is None else weight.data_ptr(), n, bucket, world, rank, sl,
        lr, beta1, beta2, eps, weight_decay, step, grad_scale, _stream(dev, stream))
    _check(st, "zopt_adamw_shard_step")


def adamw_shard_step_clipped(master, exp_avg, exp_avg_sq, grad, weight, n, bucket, world, rank,
                             lr, beta1, beta2, eps, weight_decay, step, clip_stats,
                             skip_nonfinite=False, shard_len_=None, stream=None) -> None:
    """adamw_shard_step with grad_scale read from the device clip statistics
    (fp32 [CLIP_STATS]) when the kernel runs (zopt_adamw_shard_step_clipped)."""
    sl = shard_len(n, bucket, world) if shard_len_ is None else shard_len_
    dev = master.device
    _need(master, torch.float32, sl, "master")
    _need(exp_avg, torch.float32, sl, "exp_avg", dev)
    _need(exp_avg_sq, torch.float32, sl, "exp_avg_sq", dev)
    _need(grad, torch.bfloat16, n, "grad", dev)
    _need(clip_stats, torch.float32, CLIP_STATS, "clip_stats", dev)
    if weight is not None:
        _need(weight, torch.bfloat16, n, "weight", dev)
    st = lib().zopt_adamw_shard_step_clipped(
        master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), grad.data_ptr(),
        None if weight is None else weight.data_ptr(), n, bucket, world, rank, sl,
        lr, beta1, beta2, eps, weight_decay, step, clip_stats.data_ptr(), int(skip_nonfinite),
        _stream(dev, stream))
    _check(st, "zopt_adamw_shard_step_clipped")


def grad_sq_norm_workspace_bytes(n: int, bucket: int, world: int, rank: int = 0) -> int:
    size = ctypes.c_size_t(0)
    st = lib().zopt_grad_sq_norm(None, n, bucket, world, rank, shard_len(n, bucket, world),
                                 None, None, ctypes.byref(size), None)
    _check(st, "zopt_grad_sq_norm(workspace query)")
    return int(size.value)


def grad_sq_norm(grad, n, bucket, world, rank, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sum of squares of rank `rank`'s real gradient elements, as a float64
    [1] device tensor (zopt_grad_sq_norm); nothing is read back."""
    dev = grad.device
    _need(grad, torch.bfloat16, n, "grad")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=dev)
    _need(out, torch.float64, 1, "out", dev)
    need = grad_sq_norm_workspace_bytes(n, bucket, world, rank)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, need, "workspace", dev)
    size = ctypes.c_size_t(workspace.numel())
    st = lib().zopt_grad_sq_norm(grad.data_ptr(), n, bucket, world, rank,
                                 shard_len(n, bucket, world), out.data_ptr(),
                                 workspace.data_ptr(), ctypes.byref(size), _stream(dev, stream))
    _check(st, "zopt_grad_sq_norm")
    return out


def grad_sq_norm_noalloc(grad, n, bucket, world, rank, out: torch.Tensor,
                         stream=None) -> torch.Tensor:
    """grad_sq_norm with the library's own 16 KiB scratch per GPU instead of
    a workspace (zopt_grad_sq_norm_noalloc): `out` is a float64 [1] device
    tensor the caller provides, and the call allocates nothing.  Calls that
    overlap on one GPU race on the scratch."""
    _need(grad, torch.bfloat16, n, "grad")
    _need(out, torch.float64, 1, "out", grad.device)
    st = lib().zopt_grad_sq_norm_noalloc(grad.data_ptr(), n, bucket, world, rank,
                                         shard_len(n, bucket, world), out.data_ptr(),
                                         _stream(grad.device, stream))
    _check(st, "zopt_grad_sq_norm_noalloc")
    return out


def grad_clip_stats(sq: torch.Tensor, max_norm: float, inv_scale: float = 1.0,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Clip statistics (fp32 [CLIP_STATS] device tensor: total_norm,
    clip_coef, clipped, found_inf, grad_scale) from the float64 sums of
    squares in `sq`, added in order (zopt_grad_clip_stats)."""
    dev = sq.device
    _need(sq, torch.float64, 1, "sq")
    if out is None:
        out = torch.empty(CLIP_STATS, dtype=torch.float32, device=dev)
    _need(out, torch.float32, CLIP_STATS, "out", dev)
    st = lib().zopt_grad_clip_stats(sq.data_ptr(), sq.numel(), max_norm, inv_scale,
                                    out.data_ptr(), _stream(dev, stream))
    _check(st, "zopt_grad_clip_stats")
    return out


def round_bf16(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst = bf16(src), round to nearest even (zopt_round_bf16)."""
    n = src.numel()
    _need(src, torch.float32, n, "src")
    _need(dst, torch.bfloat16, n, "dst", src.device)
    st = lib().zopt_round_bf16(src.data_ptr(), dst.data_ptr(), n, _stream(src.device, stream))
    _check(st, "zopt_round_bf16")


def set_ns_workgroup_limit(n: int) -> None:
    """Caps the workgroups the persistent Newton-Schulz B X launches keep
    resident (0: a full round of the device); process-wide
    (zopt_set_ns_workgroup_limit)."""
    _check(lib().zopt_set_ns_workgroup_limit(int(n)), "zopt_set_ns_workgroup_limit")


NS_FORM_AUTO, NS_FORM_PLAIN, NS_FORM_GRAM_BF16 = 0, 1, 2


def set_ns_form(form: int) -> None:
    """Newton-Schulz form of later calls: NS_FORM_AUTO (segments on the Gram
    matrix for groups with n >= 2 m, m <= 4096 and batch m^2 (n - m) >= 2^29, the m x m
    chain in fp16 where the coefficients allow), NS_FORM_PLAIN (plain
    iterations throughout) or NS_FORM_GRAM_BF16 (as AUTO, chain in bf16)
    (zopt_set_ns_form)."""
    _check(lib().zopt_set_ns_form(int(form)), "zopt_set_ns_form")


def _ptr_array(tensors) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _check_matrices(lists, shape, device, prefix=""):
    """Every tensor of `lists` [(tensors, dtype, name)] is a contiguous GPU
    tensor of that dtype and `shape` on `device`: one combined test per
    tensor, and the detailed checks (for the error message) only where it
    fails."""
    index = device.index if device.type == "cuda" else -2
    for tensors, dt, nm in lists:
        for i, t in enumerate(tensors):
            if not (isinstance(t, torch.Tensor) and t.dtype == dt and t.is_cuda
                    and t.get_device() == index and t.shape == shape and t.is_contiguous()):
                name = f"{prefix}{nm}[{i}]"
                _need(t, dt, shape[0] * shape[1], name, device)
                raise ValueError(f"{name}: shape {tuple(t.shape)}, need {tuple(shape)}")


def muon_workspace_bytes(batch: int, rows: int, cols: int) -> int:
    size = ctypes.c_size_t(0)
    st = lib().zopt_muon_step(batch, rows, cols, None, None, None, None, 0.0, 0.0, 0, 0.0, 0,
                              0.0, 0.0, 0.0, 0.0, 0, None, ctypes.byref(size), None)
    _check(st, "zopt_muon_step(workspace query)")
    return int(size.value)


def muon_step(master: Sequence[torch.Tensor], momentum: Sequence[torch.Tensor],
              grad: Sequence[torch.Tensor], weight: Optional[Sequence[torch.Tensor]],
              lr: float, momentum_beta: float = 0.95, nesterov: bool = True,
              weight_decay: float = 0.1, ns_steps: int = 5,
              ns_coeffs=(3.4445, -4.7750, 2.0315), ns_eps: float = 1e-7,
              adjust_lr: int = 1, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """One Muon step on a batch of same-shape [rows, cols] matrices
    (zopt_muon_step).  master, momentum: fp32; grad, weight: bf16.  Returns
    the workspace (allocated with torch if not given), which holds the
    orthogonalised updates (see muon_output_view)."""
    batch = len(master)
    if not (1 <= batch <= MAX_BATCH) or len(momentum) != batch or len(grad) != batch or (
            weight is not None and len(weight) != batch):
        raise ValueError("muon_step: need 1..64 matrices and equal-length lists")
    shape = master[0].shape
    rows, cols = shape
    dev = master[0].device
    _check_matrices(((master, torch.float32, "master"), (momentum, torch.float32, "momentum"),
                     (grad, torch.bfloat16, "grad"))
                    + (((weight, torch.bfloat16, "weight"),) if weight is not None else ()),
                    shape, dev)
    need = muon_workspace_bytes(batch, rows, cols)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, need, "workspace", dev)
    size = ctypes.c_size_t(workspace.numel())
    a, b, c = (float(x) for x in ns_coeffs)
    st = lib().zopt_muon_step(
        batch, rows, cols, _ptr_array(master), _ptr_array(momentum), _ptr_array(grad),
        None if weight is None else _ptr_array(weight), lr, momentum_beta, int(nesterov),
        weight_decay, ns_steps, a, b, c, ns_eps, adjust_lr, workspace.data_ptr(),
        ctypes.byref(size), _stream(dev, stream))
    _check(st, "zopt_muon_step")
    return workspace


def muon_output_view(workspace: torch.Tensor, batch: int, rows: int, cols: int,
                     ns_steps: int, index: int) -> torch.Tensor:
    """The bf16 [rows, cols] orthogonalised update of matrix `index` inside a
    workspace filled by muon_step (a strided view, not a copy)."""
    out = ctypes.c_void_p(0)
    ld = ctypes.c_int64(0)
    st = lib().zopt_muon_output_view(batch, rows, cols, ns_steps, workspace.data_ptr(), index,
                                     ctypes.byref(out), ctypes.byref(ld))
    _check(st, "zopt_muon_output_view")
    off = out.value - workspace.data_ptr()
    assert off % 2 == 0 and off >= 0
    flat = workspace.view(torch.bfloat16)
    return flat.as_strided((rows, cols), (ld.value, 1), off // 2)


def _shape_arrays(shapes):
    n = len(shapes)
    if not (1 <= n <= MAX_GROUPS):
        raise ValueError(f"need 1..{MAX_GROUPS} groups, got {n}")
    b = (ctypes.c_int32 * n)(*[int(x[0]) for x in shapes])
    r = (ctypes.c_int64 * n)(*[int(x[1]) for x in shapes])
    c = (ctypes.c_int64 * n)(*[int(x[2]) for x in shapes])
    return n, b, r, c


def muon_groups_workspace_bytes(shapes: Sequence[tuple]) -> int:
    """Workspace bytes of a zopt_muon_step_groups call over groups given as
    (batch, rows, cols)."""
    n, b, r, c = _shape_arrays(shapes)
    size = ctypes.c_size_t(0)
    st = lib().zopt_muon_step_groups(n, b, r, c, None, None, None, None, 0.0, 0.0, 0, 0.0, 0,
                                     0.0, 0.0, 0.0, 0.0, 0, None, ctypes.byref(size), None)
    _check(st, "zopt_muon_step_groups(workspace query)")
    return int(size.value)


def muon_step_groups(groups: Sequence[tuple], lr: float, momentum_beta: float = 0.95,
                     nesterov: bool = True, weight_decay: float = 0.1, ns_steps: int = 5,
                     ns_coeffs=(3.4445, -4.7750, 2.0315), ns_eps: float = 1e-7,
                     adjust_lr: int = 1, workspace: Optional[torch.Tensor] = None,
                     stream=None, ns_guard: Optional[float] = None,
                     ns_health: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Muon step on several groups of same-shape matrices in one call
    (zopt_muon_step_groups).  Each group is (master, momentum, grad, weight)
    with lists of equal length; weight may be None for every group or for
    none.  Returns the workspace (see muon_groups_output_view).

    With ns_guard (and ns_health, fp32 [2 + 3 * matrices] on the device) the
    call is zopt_muon_step_groups_guarded: ns_health receives the number of
    rejected matrices, the worst passing ratio and [ratio, absmax, rejected]
    per matrix, and a rejected matrix is not updated."""
    shapes, M, Mo, G, W, with_w, dev = _muon_group_tables(groups)
    need = muon_groups_workspace_bytes(shapes)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, need, "workspace", dev)
    n, b, r, c = _shape_arrays(shapes)
    size = ctypes.c_size_t(workspace.numel())
    ca, cb, cc = (float(x) for x in ns_coeffs)
    common = (n, b, r, c, _ptr_array(M), _ptr_array(Mo), _ptr_array(G),
              _ptr_array(W) if with_w else None, lr, momentum_beta, int(nesterov), weight_decay,
              ns_steps, ca, cb, cc, ns_eps, adjust_lr)
    if ns_guard is None:
        if ns_health is not None:
            raise ValueError("muon_step_groups: ns_health needs ns_guard")
        st = lib().zopt_muon_step_groups(*common, workspace.data_ptr(), ctypes.byref(size),
                                         _stream(dev, stream))
        _check(st, "zopt_muon_step_groups")
        return workspace
    if ns_health is None:
        raise ValueError("muon_step_groups: ns_guard needs an ns_health tensor")
    _need(ns_health, torch.float32, 2 + 3 * len(M), "ns_health", dev)
    st = lib().zopt_muon_step_groups_guarded(*common, ns_guard, ns_health.data_ptr(),
                                             workspace.data_ptr(), ctypes.byref(size),
                                             _stream(dev, stream))
    _check(st, "zopt_muon_step_groups_guarded")
    return workspace


def _muon_group_tables(groups):
    """Checks the (master, momentum, grad, weight) groups of a Muon call and
    flattens them: (shapes, masters, momenta, grads, weights, with_weights,
    device)."""
    if not groups:
        raise ValueError("muon_step_groups: no groups")
    with_w = groups[0][3] is not None
    shapes, M, Mo, G, W = [], [], [], [], []
    dev = groups[0][0][0].device
    for gi, (master, momentum, grad, weight) in enumerate(groups):
        batch = len(master)
        if not (1 <= batch <= MAX_BATCH) or len(momentum) != batch or len(grad) != batch:
            raise ValueError(f"group {gi}: need 1..64 matrices and equal-length lists")
        if (weight is not None) != with_w or (weight is not None and len(weight) != batch):
            raise ValueError(f"group {gi}: weight lists must be given for all groups or none")
        shape = master[0].shape
        rows, cols = shape
        _check_matrices(((master, torch.float32, "master"), (momentum, torch.float32, "momentum"),
                         (grad, torch.bfloat16, "grad"))
                        + (((weight, torch.bfloat16, "weight"),) if weight is not None else ()),
                        shape, dev, f"group {gi} ")
        shapes.append((batch, rows, cols))
        M += list(master)
        Mo += list(momentum)
        G += list(grad)
        if with_w:
            W += list(weight)
    return shapes, M, Mo, G, W, with_w, dev


class MuonGraph:
    """One Muon call over `groups` captured as a hipGraph
    (zopt_muon_graph_create), replayed by launch() (zopt_muon_graph_launch).
    lr, momentum_beta and weight_decay are read from `scalars` (fp32 [3] on
    the device) each time the graph runs: write new values there (a copy or
    fill on the stream) to change them.  The tensors given are kept alive
    while the graph exists; close() (or garbage collection) synchronises the
    device and frees the graph."""

    def __init__(self, groups, scalars: torch.Tensor, nesterov: bool = True, ns_steps: int = 5,
                 ns_coeffs=(3.4445, -4.7750, 2.0315), ns_eps: float = 1e-7, adjust_lr: int = 1,
                 workspace: Optional[torch.Tensor] = None, ns_guard: Optional[float] = None,
                 ns_health: Optional[torch.Tensor] = None):
        shapes, M, Mo, G, W, with_w, dev = _muon_group_tables(groups)
        _need(scalars, torch.float32, 3, "scalars", dev)
        need = muon_groups_workspace_bytes(shapes)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _need(workspace, torch.uint8, need, "workspace", dev)
        if (ns_guard is None) != (ns_health is None):
            raise ValueError("MuonGraph: give ns_guard and ns_health together")
        if ns_health is not None:
            _need(ns_health, torch.float32, 2 + 3 * len(M), "ns_health", dev)
        n, b, r, c = _shape_arrays(shapes)
        ca, cb, cc = (float(x) for x in ns_coeffs)
        handle = ctypes.c_void_p()
        st = lib().zopt_muon_graph_create(
            n, b, r, c, _ptr_array(M), _ptr_array(Mo), _ptr_array(G),
            _ptr_array(W) if with_w else None, scalars.data_ptr(), int(nesterov), ns_steps,
            ca, cb, cc, ns_eps, adjust_lr, 0.0 if ns_guard is None else ns_guard,
            None if ns_health is None else ns_health.data_ptr(), workspace.data_ptr(),
            workspace.numel(), ctypes.byref(handle))
        _check(st, "zopt_muon_graph_create")
        self._handle = handle
        self.device = dev
        self.shapes = shapes
        self.ns_steps = ns_steps
        self.workspace = workspace
        self._keep = (groups, scalars, ns_health)

    def launch(self, stream=None) -> None:
        if self._handle is None:
            raise RuntimeError("MuonGraph: closed")
        _check(lib().zopt_muon_graph_launch(self._handle, _stream(self.device, stream)),
               "zopt_muon_graph_launch")

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None:
            torch.cuda.synchronize(self.device)
            _check(lib().zopt_muon_graph_destroy(self._handle), "zopt_muon_graph_destroy")
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def muon_groups_output_view(workspace: torch.Tensor, shapes: Sequence[tuple], ns_steps: int,
                            group: int, index: int) -> torch.Tensor:
    """The bf16 [rows, cols] orthogonalised update of matrix `index` of group
    `group` inside a workspace filled by muon_step_groups (a strided view)."""
    n, b, r, c = _shape_arrays(shapes)
    out = ctypes.c_void_p(0)
    ld = ctypes.c_int64(0)
    st = lib().zopt_muon_groups_output_view(n, b, r, c, ns_steps, workspace.data_ptr(), group,
                                            index, ctypes.byref(out), ctypes.byref(ld))
    _check(st, "zopt_muon_groups_output_view")
    off = out.value - workspace.data_ptr()
    assert off % 2 == 0 and off >= 0
    rows, cols = int(shapes[group][1]), int(shapes[group][2])
    return workspace.view(torch.bfloat16).as_strided((rows, cols), (ld.value, 1), off // 2)


__all__ = ["adamw_shard_step", "muon_step", "muon_workspace_bytes", "muon_output_view",
           "muon_step_groups", "muon_groups_workspace_bytes", "muon_groups_output_view",
           "round_bf16", "shard_len", "lib", "ZoptError", "LIB_PATH", "MAX_BATCH", "MAX_GROUPS"]
