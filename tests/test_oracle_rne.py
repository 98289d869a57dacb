"""Pins for the oracle's fp32 -> bf16 round-to-nearest-even.

The write-back rounds the updated fp32 shard to bf16 exactly as a cast of the
fp32 master to bf16 does [DEG zero.py, ZeroMaster docstring and
gather_params].  Pins: hand-worked cases (ties, overflow, subnormals, NaN),
agreement with torch's CPU float32 -> bfloat16 cast (a library routine) on
every upper half-word, and the printed reason fp32 masters are needed.
"""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


def rne_bits(bits):
    return int(oracle.rne_bf16(f32(bits))[0])


def test_hand_cases():
    assert rne_bits(0x3F800000) == 0x3F80              # 1.0
    assert rne_bits(0x3F808000) == 0x3F80              # 1 + 2^-8: tie -> even
    assert rne_bits(0x3F818000) == 0x3F82              # 1 + 3*2^-8: tie -> even (up)
    assert rne_bits(0x3F808001) == 0x3F81              # just above the tie
    assert rne_bits(0x3F807FFF) == 0x3F80              # just below the tie
    assert rne_bits(0x7F7FFFFF) == 0x7F80              # max finite fp32 -> +inf
    assert rne_bits(0xFF7FFFFF) == 0xFF80              # -> -inf
    assert rne_bits(0x7F7F7FFF) == 0x7F7F              # largest that stays finite
    assert rne_bits(0x7F800000) == 0x7F80              # +inf stays
    assert rne_bits(0xFF800000) == 0xFF80              # -inf stays
    assert rne_bits(0x7FC00000) == 0x7FC0              # NaN
    assert rne_bits(0xFFC00001) == 0x7FC0              # negative NaN: sign dropped
    assert rne_bits(0x7F800001) == 0x7FC0              # signalling NaN quieted
    assert rne_bits(0x00000001) == 0x0000              # smallest subnormal -> 0
    assert rne_bits(0x00010000) == 0x0001              # smallest bf16 subnormal kept
    assert rne_bits(0x00018000) == 0x0002              # subnormal tie -> even
    assert rne_bits(0x80000000) == 0x8000              # -0 keeps its sign
    assert rne_bits(0x00000000) == 0x0000


def test_matches_torch_cast_on_every_upper_half():
    """All 2^16 upper halves, each with low halves around the rounding
    boundary, against torch's CPU float32 -> bfloat16 conversion."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF,
                     0xC000, 0xFFFE, 0xFFFF, 0x1234, 0x9ABC], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    ours = oracle.rne_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    ref = ref.view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_random_patterns_match_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = oracle.rne_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref.view(np.uint16)[~nan])


def test_bf16_master_would_lose_the_decay():
    """The decay factor 1 - lr*wd = 1 - 6e-5 is far below bf16's relative
    grid of 2^-8, so rounding a decayed bf16 value gives the value back, while
    in fp32 the decay is kept."""
    fig = json.load(open(GOLDEN))["decay_vs_bf16_grid"]
    lr, wd = fig["lr"], fig["weight_decay"]
    assert abs(lr * wd - fig["printed_decay_term"]) < 1e-12
    assert abs(2.0 ** -8 - fig["printed_bf16_grid"]) < 1e-4
    decay = np.float32(1.0 - lr * wd)
    # every positive normal bf16 value
    h = np.arange(0x0080, 0x7F80, dtype=np.uint16)
    p = oracle.bf16_bits_to_f32(h)
    decayed = p * decay
    assert np.array_equal(oracle.rne_bf16(decayed), h)
    assert np.all(decayed != p)
