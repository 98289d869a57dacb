"""Pins for the oracle's flat bucketed shard layout.

The layout is the one of DEG zero.py (ZeroMaster module docstring and
__init__): parameters end to end in a flat vector, cut into buckets whose
length is lowered to a multiple of world, the last bucket padded to a multiple
of world; rank r owns the r-th of world equal pieces of every bucket, and its
shard is those pieces concatenated.

The pins build that layout a second way -- by literally materialising every
bucket as a Python list, padding it, slicing it into pieces and
concatenating -- and check the oracle's closed-form index map against it, plus
the partition invariants the description implies.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def materialised_shards(n, bucket, world):
    """Every rank's shard as a list of flat indices (None = padding), built by
    cutting a Python list [0, n) exactly as the page describes."""
    flat = list(range(n))
    size = bucket - bucket % world
    if size < world:
        size = world
    shards = [[] for _ in range(world)]
    for start in range(0, n, size):
        chunk = flat[start:start + size]
        while len(chunk) % world:
            chunk.append(None)
        piece = len(chunk) // world
        for r in range(world):
            shards[r].extend(chunk[r * piece:(r + 1) * piece])
    return shards


CASES = [
    (1, 1, 1), (7, 3, 1), (10, 4, 4), (10, 3, 4), (3, 100, 4), (1, 5, 8),
    (1000, 64, 8), (1001, 64, 8), (1000, 65, 8), (999, 7, 3), (12345, 1000, 6),
    (4096, 4096, 1), (4097, 4096, 2), (50, 1, 2), (64, 8, 16),
]


@pytest.mark.parametrize("n,bucket,world", CASES)
def test_index_map_matches_materialised_layout(n, bucket, world):
    shards = materialised_shards(n, bucket, world)
    assert oracle.shard_len(n, bucket, world) == len(shards[0])
    for r in range(world):
        sl = len(shards[r])
        flat, real = oracle.shard_index_map(n, bucket, world, r, np.arange(sl))
        for j, want in enumerate(shards[r]):
            if want is None:
                assert not real[j], (r, j)
            else:
                assert real[j] and flat[j] == want, (r, j, flat[j], want)


@pytest.mark.parametrize("n,bucket,world", CASES)
def test_partition_invariants(n, bucket, world):
    sl = oracle.shard_len(n, bucket, world)
    seen = np.zeros(n, dtype=np.int64)
    pads = 0
    for r in range(world):
        flat, real = oracle.shard_index_map(n, bucket, world, r, np.arange(sl))
        np.add.at(seen, flat[real], 1)
        pads += int((~real).sum())
    # every real element is owned by exactly one rank, once
    assert np.all(seen == 1)
    nb = oracle.num_buckets(n, bucket, world)
    assert nb == math.ceil(n / oracle.bucket_adjust(bucket, world))
    # padding only fills the last bucket up to a multiple of world
    assert sl * world == n + pads and pads < world
    assert sl == math.ceil(n / world) or pads > 0 or sl * world == n


def test_bucket_adjust_rule():
    # lowered to a multiple of world, never below world
    assert oracle.bucket_adjust(10, 4) == 8
    assert oracle.bucket_adjust(3, 4) == 4
    assert oracle.bucket_adjust(8, 4) == 8
    assert oracle.bucket_adjust(1, 1) == 1


def test_out_of_range_index_rejected():
    with pytest.raises(IndexError):
        oracle.shard_index_map(10, 4, 2, 0, np.array([oracle.shard_len(10, 4, 2)]))


def test_zero2_backbone_layout_numbers():
    """2.0e9 parameters, buckets of 1 << 25 over 8 ranks (the page's default
    bucket constant): 60 buckets, 250,000,000 elements per shard, no padding."""
    fig = json.load(open(GOLDEN))["zero_bucket"]
    bucket = fig["bucket_elems"]
    assert bucket == 1 << 25 and bucket * 4 // 2**20 == fig["printed_fp32_MB"]
    n = 2_000_000_000
    assert oracle.num_buckets(n, bucket, 8) == 60
    assert oracle.shard_len(n, bucket, 8) == 250_000_000
    # rank 3: the last bucket starts at 59 << 25 and has piece 20,288,512 / 8
    last_piece = (n - 59 * bucket) // 8
    j = np.array([0, 59 * (bucket // 8), 250_000_000 - 1])
    flat, real = oracle.shard_index_map(n, bucket, 8, 3, j)
    assert real.all()
    assert flat[0] == 3 * (bucket // 8)
    assert flat[1] == 59 * bucket + 3 * last_piece == 1_987_319_680
    assert flat[2] == 59 * bucket + 4 * last_piece - 1
