"""CPU oracle for one rank's ZeRO-style optimizer step.

TEST INFRASTRUCTURE ONLY.  The plain, slow, obviously correct definition of
what the GPU library computes.  Only the test suite, the smoke check
(``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code with the GPU library and the GPU library never
calls it.

* ``zopt_oracle.c`` (built to ``liboracle.so`` with gcc, no FMA contraction):
  the flat bucketed shard layout, binary32 AdamW, round-to-nearest-even
  bf16, the Muon momentum pre-step and the Muon post-step.
  It also holds the squared gradient norm of a shard with the clip
  statistics derived from it, and the Newton-Schulz health figures (update
  ratio, divergence guard).
* ``ns.py``: Newton-Schulz in float64.

Every array argument is a numpy array of the stated dtype; bf16 values are
carried as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .ns import (NS_COEFFS, NS_EPS, NS_STEPS, frobenius_prescale, newton_schulz,
                 ns_scalar_map)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zopt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-shared", "-fPIC"]


def build() -> str:
    """Compile zopt_oracle.c into liboracle.so next to it; return the path."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, f32, vp = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_void_p)
        L.orc_rne_bf16.argtypes = [f32]
        L.orc_rne_bf16.restype = ctypes.c_uint16
        L.orc_rne_bf16_array.argtypes = [vp, vp, i64]
        L.orc_bucket_adjust.argtypes = [i64, i32]
        L.orc_bucket_adjust.restype = i64
        L.orc_num_buckets.argtypes = [i64, i64, i32]
        L.orc_num_buckets.restype = i64
        L.orc_shard_len.argtypes = [i64, i64, i32]
        L.orc_shard_len.restype = i64
        L.orc_shard_index_map.argtypes = [i64, i64, i32, i32, i64, vp, vp, vp]
        L.orc_shard_index_map.restype = ctypes.c_int
        L.orc_adamw_scalars.argtypes = [f32, f32, f32, f32, i64, vp]
        L.orc_adamw_shard_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32,
                                           f32, f32, f32, f32, f32, i64, f32]
        L.orc_adamw_points.argtypes = [i64, vp, vp, vp, vp, vp, f32, f32, f32, f32,
                                       f32, i64]
        L.orc_muon_pre.argtypes = [i64, vp, vp, f32, ctypes.c_int, vp]
        L.orc_muon_scale.argtypes = [i64, i64, ctypes.c_int]
        L.orc_muon_scale.restype = ctypes.c_double
        L.orc_muon_post.argtypes = [i64, i64, vp, vp, vp, f32, f32, ctypes.c_int]
        L.orc_grad_sq_norm.argtypes = [vp, i64, i64, i32, i32]
        L.orc_grad_sq_norm.restype = ctypes.c_double
        L.orc_clip_stats.argtypes = [vp, i32, f32, f32, vp]
        L.orc_ns_health.argtypes = [i64, i64, vp, f32, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a: np.ndarray, dtype, name: str) -> None:
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a contiguous {np.dtype(dtype)} array")


# ----------------------------------------------------------------- bf16

def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (ties to even), returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_rne_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to binary32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- layout

def bucket_adjust(bucket: int, world: int) -> int:
    return int(lib().orc_bucket_adjust(bucket, world))


def num_buckets(n: int, bucket: int, world: int) -> int:
    return int(lib().orc_num_buckets(n, bucket, world))


def shard_len(n: int, bucket: int, world: int) -> int:
    return int(lib().orc_shard_len(n, bucket, world))


def shard_index_map(n: int, bucket: int, world: int, rank: int, j: np.ndarray):
    """(flat index, is_real) for each shard index j of `rank`."""
    j = np.ascontiguousarray(j, dtype=np.int64)
    flat = np.empty(j.shape, dtype=np.int64)
    real = np.empty(j.shape, dtype=np.uint8)
    rc = lib().orc_shard_index_map(n, bucket, world, rank, j.size, _ptr(j),
                                   _ptr(flat), _ptr(real))
    if rc != 0:
        raise IndexError("shard index outside [0, shard_len)")
    return flat, real.astype(bool)


# ----------------------------------------------------------------- AdamW

def adamw_scalars(lr, beta1, beta2, wd, step) -> np.ndarray:
    """[step_size, sqrt(bias_correction2), decay, 1 - beta1, 1 - beta2]."""
    out = np.empty(5, dtype=np.float32)
    lib().orc_adamw_scalars(lr, beta1, beta2, wd, step, _ptr(out))
    return out


def adamw_shard_step(master, exp_avg, exp_avg_sq, grad, weight, n, bucket, world,
                     rank, lr, beta1, beta2, eps, wd, step, grad_scale=1.0):
    """One AdamW step over rank `rank`'s shard, in place (see zopt_oracle.c)."""
    _check(master, np.float32, "master")
    _check(exp_avg, np.float32, "exp_avg")
    _check(exp_avg_sq, np.float32, "exp_avg_sq")
    _check(grad, np.uint16, "grad")
    if weight is not None:
        _check(weight, np.uint16, "weight")
        assert weight.size == n
    assert grad.size == n
    sl = shard_len(n, bucket, world)
    assert master.size == exp_avg.size == exp_avg_sq.size == sl
    lib().orc_adamw_shard_step(_ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq),
                               _ptr(grad), _ptr(weight), n, bucket, world, rank,
                               lr, beta1, beta2, eps, wd, step, grad_scale)


def adamw_points(p, m, v, g, lr, beta1, beta2, eps, wd, step):
    """AdamW on independent elements with binary32 gradients; in place.
    Returns the bf16 bits of the new p."""
    for a, nm in ((p, "p"), (m, "m"), (v, "v"), (g, "g")):
        _check(a, np.float32, nm)
    w = np.empty(p.shape, dtype=np.uint16)
    lib().orc_adamw_points(p.size, _ptr(p), _ptr(m), _ptr(v), _ptr(g), _ptr(w), lr,
                           beta1, beta2, eps, wd, step)
    return w


# ----------------------------------------------------------------- clipping

CLIP_FIELDS = ("total_norm", "clip_coef", "clipped", "found_inf", "grad_scale")


def grad_sq_norm(grad, n, bucket, world, rank) -> float:
    """Sum of squares of rank `rank`'s real gradient elements (see zopt_oracle.c)."""
    _check(grad, np.uint16, "grad")
    assert grad.size == n
    return float(lib().orc_grad_sq_norm(_ptr(grad), n, bucket, world, rank))


def clip_stats(sq, max_norm, inv_scale=1.0) -> np.ndarray:
    """[total_norm, clip_coef, clipped, found_inf, grad_scale] (binary32) from
    the partial sums of squares `sq`, added in order."""
    sq = np.ascontiguousarray(np.atleast_1d(np.asarray(sq, dtype=np.float64)))
    out = np.empty(5, dtype=np.float32)
    lib().orc_clip_stats(_ptr(sq), sq.size, max_norm, inv_scale, _ptr(out))
    return out


# ----------------------------------------------------------------- Muon

def muon_pre(momentum, grad, mu, nesterov=True) -> np.ndarray:
    """Momentum EMA + Nesterov, in place on `momentum`; returns U (binary32,
    the caller's orientation)."""
    _check(momentum, np.float32, "momentum")
    _check(grad, np.uint16, "grad")
    assert momentum.shape == grad.shape
    u = np.empty(momentum.shape, dtype=np.float32)
    lib().orc_muon_pre(momentum.size, _ptr(momentum), _ptr(grad), mu, int(nesterov),
                       _ptr(u))
    return u


def muon_scale(rows, cols, adjust=1) -> float:
    return float(lib().orc_muon_scale(rows, cols, adjust))


def muon_post(master, o, lr, wd, adjust=1, want_weight=True):
    """P <- P*fp32(1-lr*wd) - fp32(lr*scale)*O in place; returns bf16 bits of P."""
    _check(master, np.float32, "master")
    o = np.ascontiguousarray(o, dtype=np.float32)
    assert master.shape == o.shape and master.ndim == 2
    rows, cols = master.shape
    w = np.empty(master.shape, dtype=np.uint16) if want_weight else None
    lib().orc_muon_post(rows, cols, _ptr(master), _ptr(o), _ptr(w), lr, wd, adjust)
    return w


NS_GUARD = 1000.0  # element magnitude above which an update is refused


def ns_health(o, guard=NS_GUARD) -> np.ndarray:
    """[ratio, absmax, rejected] of one orthogonalised update O [rows, cols]
    (binary32): ratio = ||O||_F / sqrt(min(rows, cols)), rejected = 1 unless
    every |O_ij| <= guard."""
    o = np.ascontiguousarray(o, dtype=np.float32)
    assert o.ndim == 2
    out = np.empty(3, dtype=np.float32)
    lib().orc_ns_health(o.shape[0], o.shape[1], _ptr(o), guard, _ptr(out))
    return out


def ns_call_health(os_, guard=NS_GUARD):
    """Health of the updates of one Muon call: (number rejected, worst ratio
    among the updates that passed (0 if none did), per-matrix [ratio, absmax,
    rejected] rows)."""
    rows = np.array([ns_health(o, guard) for o in os_], dtype=np.float32).reshape(-1, 3)
    passed = rows[rows[:, 2] == 0, 0]
    worst = np.float32(passed.max()) if passed.size else np.float32(0.0)
    return int(rows[:, 2].sum()), worst, rows


def muon_step(master, momentum, grad, lr, mu, nesterov, wd, ns_steps=NS_STEPS,
              coeffs=NS_COEFFS, ns_eps=NS_EPS, adjust=1, o_override=None, guard=None):
    """The whole Muon step of one matrix, in place on master and momentum.

    Returns (weight bits, O in float64).  With ``o_override`` (binary32 O from
    another implementation) the post-step uses it instead of this oracle's own
    float64 Newton-Schulz result -- stage-wise, teacher-forced checking.  With
    a ``guard``, an update the divergence guard rejects is not applied: master
    keeps its value and the weight bits returned are None (momentum has still
    taken its step)."""
    u = muon_pre(momentum, grad, mu, nesterov)
    o64 = newton_schulz(u, ns_steps, coeffs, ns_eps)
    o = o64.astype(np.float32) if o_override is None else o_override
    if guard is not None and ns_health(o, guard)[2]:
        return None, o64
    w = muon_post(master, o, lr, wd, adjust)
    return w, o64


__all__ = [
    "NS_COEFFS", "NS_EPS", "NS_STEPS", "frobenius_prescale", "newton_schulz",
    "ns_scalar_map", "build", "lib", "rne_bf16", "bf16_bits_to_f32",
    "bucket_adjust", "num_buckets", "shard_len", "shard_index_map", "adamw_scalars",
    "adamw_shard_step", "adamw_points", "CLIP_FIELDS", "grad_sq_norm", "clip_stats",
    "muon_pre", "muon_scale", "muon_post", "NS_GUARD", "ns_health", "ns_call_health",
    "muon_step",
]
