"""Pins of the oracle's partial interleaved RoPE against closed forms and invariants.

Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx.
"""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import OracleError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_ulp(x: float) -> float:
    x32 = np.float32(x)
    return float(np.spacing(np.abs(x32)))


@pytest.mark.parametrize("rotary_dims,theta", [(2, 10000.0), (16, 10000.0), (64, 10000.0), (64, 500000.0), (10, 3.0)])
def test_inverse_frequency_is_nearest_f32_of_closed_form(rotary_dims, theta):
    getcontext().prec = 60
    inv = oracle.rope_inverse_frequencies(rotary_dims, theta)
    assert inv.dtype == np.float32 and inv.shape == (rotary_dims // 2,)
    assert inv[0] == np.float32(1.0)
    assert np.all(np.diff(inv.astype(np.float64)) < 0) if rotary_dims > 2 else True
    t = Decimal(repr(float(np.float32(theta))))
    for p in range(rotary_dims // 2):
        exact = float(t ** (Decimal(-2 * p) / Decimal(rotary_dims)))
        assert abs(float(inv[p]) - exact) <= _f32_ulp(exact)


def test_inverse_frequency_exact_values_theta_10000():
    # 10000^(-2p/8) = 10^(-p): the exponent -2p/8 is exact in f32 for p < 4.
    inv = oracle.rope_inverse_frequencies(8, 10000.0)
    assert inv.tolist() == [np.float32(1.0), np.float32(0.1), np.float32(0.01), np.float32(0.001)]


def test_angle_of_pair_zero_is_the_position():
    inv = oracle.rope_inverse_frequencies(64, 10000.0)
    pos = np.array([0, 1, 7, 4096, 131072, (1 << 24) - 1])
    ang = oracle.rope_angles(pos, inv)
    assert ang.dtype == np.float32
    assert np.array_equal(ang[:, 0], pos.astype(np.float32))


def test_angle_is_rounded_product():
    inv = oracle.rope_inverse_frequencies(64, 10000.0)
    pos = np.arange(0, 200000, 997)
    ang = oracle.rope_angles(pos, inv)
    exact = pos[:, None].astype(np.float64) * inv.astype(np.float64)[None, :]
    # correctly rounded: within half an ulp of the exact double product
    assert np.all(np.abs(ang.astype(np.float64) - exact) <= 0.5 * np.spacing(np.abs(ang)).astype(np.float64))


def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "rope_hand_example.json")))
    x = np.array(g["input"])[None, None, :]                     # [1 row, 1 token, 5]
    inv = oracle.rope_inverse_frequencies(g["rotary_dims"], g["theta"])
    assert inv.tolist() == [np.float32(v) for v in g["inverse_frequencies_f32"]]
    y = oracle.rope_partial_interleaved(x, g["position"], g["rotary_dims"], g["theta"])[0, 0]
    a1 = float(np.float32(0.01))
    expected = [math.cos(1.0), -math.sin(a1), math.sin(1.0), math.cos(a1), 7.0]
    np.testing.assert_allclose(y, expected, rtol=0, atol=1e-15)


def test_position_zero_is_the_deinterleave_permutation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 1, 3, 20))
    y = oracle.rope_partial_interleaved(x, 0, 16, 10000.0)
    perm = list(range(0, 16, 2)) + list(range(1, 16, 2)) + list(range(16, 20))
    assert np.array_equal(y, x[..., perm])


def test_matches_complex_multiplication():
    """(a + i b) * exp(i angle): real part first half, imaginary part second half."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 2, 64))
    off = [11, 0, 40000]
    y = oracle.rope_partial_interleaved(x, off, 64, 10000.0)
    inv = oracle.rope_inverse_frequencies(64, 10000.0)
    for b in range(3):
        for t in range(5):
            ang = oracle.rope_angles(np.array(off[b] + t), inv).astype(np.float64)
            z = (x[b, t, :, 0::2] + 1j * x[b, t, :, 1::2]) * np.exp(1j * ang)
            np.testing.assert_allclose(y[b, t, :, :32], z.real, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(y[b, t, :, 32:], z.imag, rtol=1e-13, atol=1e-13)


def test_pair_norms_preserved_and_tail_untouched():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 7, 4, 24))
    y = oracle.rope_partial_interleaved(x, [3, 100000], 16, 10000.0)
    n_in = x[..., 0:16:2] ** 2 + x[..., 1:16:2] ** 2
    n_out = y[..., :8] ** 2 + y[..., 8:16] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)
    assert np.array_equal(y[..., 16:], x[..., 16:])


def test_relative_position_property():
    """<rot(q,m), rot(k,n)> depends on n - m only (up to the f32 angle rounding)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)

    def rot(v, pos):
        return oracle.rope_partial_interleaved(v[None, None, :], pos, 64, 10000.0)[0, 0]

    scale = np.linalg.norm(q) * np.linalg.norm(k)
    for m, n, d in [(0, 5, 17), (3, 3, 100), (10, 2, 250)]:
        a = rot(q, m) @ rot(k, n)
        b = rot(q, m + d) @ rot(k, n + d)
        assert abs(a - b) <= 1e-4 * scale


def test_per_row_offsets_equal_separate_calls_and_tokens_advance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 6, 2, 16))
    off = [0, 9, 123456]
    y = oracle.rope_partial_interleaved(x, off, 16, 10000.0)
    for b in range(3):
        yb = oracle.rope_partial_interleaved(x[b:b + 1], off[b], 16, 10000.0)
        assert np.array_equal(y[b:b + 1], yb)
        for t in range(6):
            yt = oracle.rope_partial_interleaved(x[b:b + 1, t:t + 1], off[b] + t, 16, 10000.0)
            assert np.array_equal(y[b:b + 1, t:t + 1], yt)


def test_token_axis_other_than_one():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 5, 8))          # token axis 2
    y = oracle.rope_partial_interleaved(x, 4, 8, 10000.0, token_axis=2)
    y_ref = np.swapaxes(oracle.rope_partial_interleaved(np.swapaxes(x, 1, 2), 4, 8, 10000.0), 1, 2)
    assert np.array_equal(y, y_ref)


@pytest.mark.parametrize("kwargs", [
    dict(x=np.zeros(4), position_offset=0, rotary_dims=4, theta=1e4),                  # rank < 2
    dict(x=np.zeros((2, 4)), position_offset=0, rotary_dims=4, theta=1e4, token_axis=1),  # token axis = feature axis
    dict(x=np.zeros((2, 3, 4)), position_offset=[0, 1], rotary_dims=4, theta=1e4, token_axis=0),
    dict(x=np.zeros((2, 3, 4)), position_offset=[0, 1, 2], rotary_dims=4, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=-1, rotary_dims=4, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=1.5, rotary_dims=4, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=0, rotary_dims=3, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=0, rotary_dims=6, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=0, rotary_dims=0, theta=1e4),
    dict(x=np.zeros((2, 3, 4)), position_offset=0, rotary_dims=4, theta=0.0),
    dict(x=np.zeros((2, 3, 4)), position_offset=0, rotary_dims=4, theta=float("inf")),
])
def test_rejections(kwargs):
    with pytest.raises(OracleError):
        oracle.rope_partial_interleaved(**kwargs)
