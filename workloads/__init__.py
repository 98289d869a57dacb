"""Seeded synthetic inputs for one rank's optimizer step.

This module holds the workload definitions (sizes, shapes, hyperparameters,
value distributions) and the seeded random draws that feed both the GPU
library and the CPU oracle.  It holds none of the optimizer's arithmetic: no
layout math, no AdamW, no rounding of results, no Newton-Schulz.  bf16 inputs
are made with torch's own float32 -> bfloat16 cast.

Seeds: numpy ``SeedSequence([1234, workload_id, tensor_id, step])`` -- 1234 is
the initialisation seed of the BluScript trainer's GPT constructor.  Large
inputs are drawn on the GPU with a torch CUDA generator seeded from the same
sequence.

Workloads (all synthetic; the pages train on public text corpora that are not
needed here, and no dataset stands in for anything):

  tiny        AdamW on N = 1,048,576 (bucket 262,144, world 4, rank 0,
              10 steps) + Muon on 2 x [128, 512]
  gpt2_small  one GPT-2-small-shaped optimizer step at world 1: AdamW on the
              tied 50304 x 768 embedding + 25 vectors of 768, Muon on 12
              layers x {Wq, Wk, Wv, Wo 768 x 768, fc 3072 x 768,
              proj 768 x 3072}; gradients carry 1% outliers x100
  zero2_2b    the flat AdamW shard of rank 3 of 8 over a 2.0e9-parameter
              backbone in buckets of 1 << 25 (2.5e8 shard elements)
  llama1b_r0  rank 0's matrices of a d=2048, 16-layer GQA decoder
              (round-robin by size over 8 ranks)
  llama8b_r0  rank 0's matrices of a 32-layer d=4096 decoder; Student-t(3)
              gradients
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np
import torch

BASE_SEED = 1234


# ---------------------------------------------------------------- definitions

@dataclasses.dataclass(frozen=True)
class AdamWPart:
    """One zopt_adamw_shard_step call per step, over [offset, offset + n) of a
    flat parameter vector."""
    n: int
    bucket: int
    world: int
    rank: int
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    offset: int = 0


@dataclasses.dataclass(frozen=True)
class AdamWWorkload:
    name: str
    wid: int
    n_total: int
    parts: Tuple[AdamWPart, ...]
    steps: int
    master_std: float = 0.02
    grad_std: float = 1e-3
    outlier_frac: float = 0.0
    outlier_mult: float = 100.0


@dataclasses.dataclass(frozen=True)
class MuonGroup:
    """count matrices of one stored shape [rows, cols] (PyTorch [out, in])."""
    count: int
    rows: int
    cols: int


@dataclasses.dataclass(frozen=True)
class MuonWorkload:
    name: str
    wid: int
    groups: Tuple[MuonGroup, ...]
    lr: float = 8e-4
    momentum: float = 0.95
    nesterov: bool = True
    weight_decay: float = 0.1
    ns_steps: int = 5
    ns_coeffs: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
    ns_eps: float = 1e-7
    adjust_lr: int = 1            # 1: match AdamW's update RMS (0.2); 0: original
    master_std: float = 0.02
    grad_std: float = 1e-3
    grad_dist: str = "normal"     # "normal" | "normal_outliers" | "student_t3"
    steps: int = 1

    @property
    def n_matrices(self) -> int:
        return sum(g.count for g in self.groups)


def round_robin_owned(shapes: Sequence[Tuple[str, int, int]], world: int,
                      rank: int) -> List[Tuple[str, int, int]]:
    """Whole-matrix ownership, round-robin by size: a stable sort of the
    matrices by element count (largest first, model order among equals), then
    matrix i goes to rank i mod world."""
    order = sorted(range(len(shapes)), key=lambda i: -shapes[i][1] * shapes[i][2])
    return [shapes[i] for k, i in enumerate(order) if k % world == rank]


def _groups(owned: Sequence[Tuple[str, int, int]]) -> Tuple[MuonGroup, ...]:
    counts = {}
    for _, r, c in owned:
        counts[(r, c)] = counts.get((r, c), 0) + 1
    return tuple(MuonGroup(k, r, c) for (r, c), k in counts.items())


def _llama_shapes(layers, d, q_heads, kv_heads, head_dim, ffn, fused_gate_up):
    out = []
    for layer in range(layers):
        out += [(f"L{layer}.wq", q_heads * head_dim, d),
                (f"L{layer}.wk", kv_heads * head_dim, d),
                (f"L{layer}.wv", kv_heads * head_dim, d),
                (f"L{layer}.wo", d, q_heads * head_dim)]
        if fused_gate_up:
            out += [(f"L{layer}.gate_up", 2 * ffn, d)]
        else:
            out += [(f"L{layer}.gate", ffn, d), (f"L{layer}.up", ffn, d)]
        out += [(f"L{layer}.down", d, ffn)]
    return out


# cfg: tiny
TINY_ADAMW = AdamWWorkload(
    name="tiny_adamw", wid=1, n_total=1_048_576,
    parts=(AdamWPart(1_048_576, 262_144, 4, 0, 1e-3, 0.9, 0.95, 1e-8, 0.1),),
    steps=10)
TINY_MUON = MuonWorkload(name="tiny_muon", wid=1, groups=(MuonGroup(2, 128, 512),),
                         steps=10)

# cfg: GPT-2-small optimizer step (world 1).  Embedding takes weight decay,
# the 25 vectors of 768 (norm gains / scales) do not.
_EMB = 50304 * 768
_VEC = 25 * 768
GPT2_ADAMW = AdamWWorkload(
    name="gpt2_small_adamw", wid=2, n_total=_EMB + _VEC,
    parts=(AdamWPart(_EMB, 1 << 25, 1, 0, 6e-4, 0.9, 0.95, 1e-8, 0.1, offset=0),
           AdamWPart(_VEC, 1 << 25, 1, 0, 6e-4, 0.9, 0.95, 1e-8, 0.0, offset=_EMB)),
    steps=1, outlier_frac=0.01)
GPT2_MUON = MuonWorkload(
    name="gpt2_small_muon", wid=2,
    groups=(MuonGroup(48, 768, 768), MuonGroup(12, 3072, 768), MuonGroup(12, 768, 3072)),
    grad_dist="normal_outliers")

# cfg: ZeRO-2 flat AdamW shard, rank 3 of 8
ZERO2_ADAMW = AdamWWorkload(
    name="zero2_2b_rank3_adamw", wid=3, n_total=2_000_000_000,
    parts=(AdamWPart(2_000_000_000, 1 << 25, 8, 3, 3e-4, 0.9, 0.95, 1e-8, 0.1),),
    steps=100)

# cfg: Llama-style 1B, rank 0 of 8 (gate and up fused as one [11264, 2048])
LLAMA1B_MUON = MuonWorkload(
    name="llama1b_rank0_muon", wid=4,
    groups=_groups(round_robin_owned(_llama_shapes(16, 2048, 16, 4, 128, 5632, True), 8, 0)))

# cfg: 8B-scale, rank 0 of 8
LLAMA8B_MUON = MuonWorkload(
    name="llama8b_rank0_muon", wid=5,
    groups=_groups(round_robin_owned(_llama_shapes(32, 4096, 32, 8, 128, 14336, False), 8, 0)),
    master_std=0.01, grad_dist="student_t3")

ADAMW_WORKLOADS = {w.name: w for w in (TINY_ADAMW, GPT2_ADAMW, ZERO2_ADAMW)}
MUON_WORKLOADS = {w.name: w for w in (TINY_MUON, GPT2_MUON, LLAMA1B_MUON, LLAMA8B_MUON)}


# ---------------------------------------------------------------- host draws

def seed_seq(wid: int, tensor_id: int, step: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([BASE_SEED, wid, tensor_id, step])


def rng(wid: int, tensor_id: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq(wid, tensor_id, step)))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns with torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def host_normal(wid, tensor_id, shape, std, step=0) -> np.ndarray:
    return (rng(wid, tensor_id, step).standard_normal(shape) * std).astype(np.float32)


def host_grad_bf16(wid, tensor_id, shape, std, dist="normal", step=0,
                   outlier_frac=0.01, outlier_mult=100.0) -> np.ndarray:
    """bf16 gradient bits: N(0, std), or with a seeded Bernoulli(outlier_frac)
    mask multiplied by outlier_mult, or std * Student-t(3)."""
    r = rng(wid, tensor_id, step)
    if dist == "student_t3":
        x = r.standard_t(3, size=shape) * std
    else:
        x = r.standard_normal(shape) * std
        if dist == "normal_outliers":
            x = np.where(r.random(shape) < outlier_frac, x * outlier_mult, x)
    return to_bf16_bits(x.astype(np.float32))


# ---------------------------------------------------------------- device draws

def _device_gen(wid, tensor_id, step, device):
    seed = int(seed_seq(wid, tensor_id, step).generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal(wid, tensor_id, shape, std, device, dtype=torch.float32, step=0):
    g = _device_gen(wid, tensor_id, step, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x if dtype == torch.float32 else x.to(dtype)


def device_grad_bf16(wid, tensor_id, shape, std, device, dist="normal", step=0,
                     outlier_frac=0.01, outlier_mult=100.0):
    """bf16 gradient tensor drawn on the device (same distributions as
    host_grad_bf16, a different random stream)."""
    g = _device_gen(wid, tensor_id, step, device)
    if dist == "student_t3":
        z = torch.randn(shape, generator=g, device=device)
        chi = torch.randn((3,) + tuple(shape if isinstance(shape, tuple) else (shape,)),
                          generator=g, device=device).pow_(2).sum(0).div_(3.0)
        x = z.div_(chi.sqrt_()).mul_(std)
    else:
        x = torch.randn(shape, generator=g, device=device).mul_(std)
        if dist == "normal_outliers":
            mask = torch.rand(shape, generator=g, device=device) < outlier_frac
            x = torch.where(mask, x * outlier_mult, x)
    return x.to(torch.bfloat16)
