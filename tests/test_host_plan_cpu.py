"""Host-side split planning of the decode attention (no GPU): the chunk length
is the smallest multiple of the 32-token tile, at least two tiles, whose split
count fits the concurrent workgroups."""

import numpy as np
import pytest

import mla_latent_kv_partial_amd as mla


def _splits(n, chunk):
    return sum(mla.split_count(v, chunk) for v in n)


@pytest.mark.parametrize("n,slots,expect", [
    ([4096], 256, 64),              # one short row: two tiles per split, 64 splits
    ([4096] * 64, 256, 1024),       # 64 equal rows: four splits each, every CU busy
    ([2048], 256, 64),              # a DSA selection of 2048 positions
    ([1], 256, 64),
    ([100000], 256, 416),           # ceil(100000 / 256) = 391 -> 416 (multiple of 32)
])
def test_plan_chunk_len_cases(n, slots, expect):
    assert mla.plan_chunk_len(n, slots) == expect


@pytest.mark.parametrize("seed", range(6))
def test_plan_chunk_len_is_minimal_and_fits(seed):
    rng = np.random.default_rng(seed)
    n = [int(v) for v in rng.integers(1024, 32769, size=int(rng.integers(1, 12)))]
    slots = 256
    c = mla.plan_chunk_len(n, slots)
    assert c % 32 == 0 and c >= 64
    assert _splits(n, c) <= slots
    # one tile less would exceed the slots (or drop below two tiles)
    assert c - 32 < 64 or _splits(n, c - 32) > slots


def test_plan_chunk_len_more_rows_than_slots_stops_at_longest_row():
    n = [50] * 300
    c = mla.plan_chunk_len(n, 256)
    assert c >= max(n)
