"""Pins of the DSA top-k selector oracle (page "mlx-bun 0.2.0 -> 0.4.0",
glm52-dsa.ts, selectGlm52DsaDevice) against a hand-worked example of the
page's rule (the page prints no values), brute force on tiny inputs, and
closed forms."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dsa_topk_hand_example.json")


def test_hand_example():
    with open(GOLDEN) as f:
        fix = json.load(f)
    for case in fix["cases"]:
        got = oracle.dsa_select(np.array(case["scores"], dtype=np.float32), case["top_k"])
        if case["expected"] is None:
            assert got is None
        else:
            assert got.tolist() == case["expected"]


def _brute(scores, k):
    """Selection by Python float comparisons: sort by (-score, position), then
    order the top k by (not strictly above the k-th score, position)."""
    n = len(scores)
    if n <= k:
        return None
    ranked = sorted(range(n), key=lambda i: (-float(scores[i]), i))
    top = ranked[:k]
    thr = min(float(scores[i]) for i in top)
    return sorted(top, key=lambda i: (not float(scores[i]) > thr, i))


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 40))
    k = int(rng.integers(1, n + 2))
    # few distinct values, so ties at the threshold are common
    scores = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.75)
    got = oracle.dsa_select(scores, k)
    ref = _brute(scores, k)
    assert (got is None) == (ref is None)
    if ref is not None:
        assert got.tolist() == ref


def test_distinct_scores_closed_form():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(5000).astype(np.float32)
    k = 300
    got = oracle.dsa_select(s, k)
    top = set(np.argpartition(-s.astype(np.float64), k - 1)[:k].tolist())
    lowest = min(top, key=lambda i: s[i])
    assert got.tolist() == sorted(top - {lowest}) + [lowest]


def test_keys_order_like_floats():
    vals = np.array([-np.inf, -1e30, -2.5, -1e-30, -0.0, 0.0, 1e-30, 3.0, 1e30, np.inf], dtype=np.float32)
    keys = oracle.dsa_rank_keys(vals).astype(np.int64)
    assert np.all(np.diff(keys) < 0), "keys must strictly decrease as the scores increase"


def test_signed_zeros_rank_by_bits_and_tie_by_value():
    # +0 ranks above -0 (bits), but they are equal for the threshold comparison
    s = np.array([-0.0, 0.0, -1.0, -0.0], dtype=np.float32)
    assert oracle.dsa_select(s, 2).tolist() == [0, 1]
    s = np.array([-0.0, 1.0, 0.0, -0.0], dtype=np.float32)
    assert oracle.dsa_select(s, 2).tolist() == [1, 2]


def test_rows_concatenate_and_dense_rows_count_minus_one():
    s = np.zeros((3, 10), dtype=np.float32)
    s[0, :8] = np.arange(8)
    s[2, :10] = -np.arange(10)
    idx, cnt = oracle.dsa_select_rows(s, [8, 3, 10], 4)
    assert cnt.tolist() == [4, -1, 4]
    assert idx.tolist() == [5, 6, 7, 4] + [0, 1, 2, 3]


def test_rejections():
    with pytest.raises(oracle.OracleError):
        oracle.dsa_select(np.array([1.0, np.nan], dtype=np.float32), 1)
    with pytest.raises(oracle.OracleError):
        oracle.dsa_select(np.array([1.0, 2.0], dtype=np.float32), 0)
