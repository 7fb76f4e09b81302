"""Pins of the fused-append oracle (page "mlx-bun 0.0.11 -> 0.0.13",
glm52-mla.ts: rmsNormF32Mlx and the kv_a split of Glm52Mla.project)."""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rms_norm_hand_example.json")
SPLIT = os.path.join(os.path.dirname(__file__), "golden", "append_split_hand_example.json")

# closed forms of the append golden file
_FORMS = {
    "6/sqrt12.5": 6 / math.sqrt(12.5),
    "2/sqrt12.5": 2 / math.sqrt(12.5),
    "cos(1)": math.cos(1.0),
    "sin(1)": math.sin(1.0),
    "cos(f32(0.01))": math.cos(float(np.float32(0.01))),
    "-sin(f32(0.01))": -math.sin(float(np.float32(0.01))),
}


def _vals(x):
    if isinstance(x, list):
        return np.array([_vals(v) for v in x])
    return _FORMS[x] if isinstance(x, str) else float(x)


def test_append_split_hand_example():
    """kv_a = [latent (first r) | rope key (last dr)]: RMSNorm on the first, RoPE on the second."""
    g = json.load(open(SPLIT))
    lat, rope = oracle.append_compressed(_vals(g["kv_a"]), _vals(g["weight"]), g["eps"], g["positions"], g["theta"],
                                         g["kv_lora_rank"], g["rope_dim"])
    np.testing.assert_allclose(lat, _vals(g["expected_latent"]), rtol=1e-15, atol=0)
    np.testing.assert_allclose(rope, _vals(g["expected_rope"]), rtol=1e-15, atol=1e-16)


def test_rms_norm_hand_example():
    with open(GOLDEN) as f:
        fix = json.load(f)
    for c in fix["cases"]:
        got = oracle.rms_norm(np.array(c["x"]), np.array(c["weight"]), c["eps"])
        assert np.allclose(got, c["expected"], rtol=1e-14, atol=0)


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64))
    y = oracle.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt((y * y).mean(axis=-1)), 1.0, rtol=1e-13)
    assert np.allclose(oracle.rms_norm(-7.5 * x, np.ones(64), 0.0), -y, rtol=1e-12)


def test_rms_norm_brute_force_loop():
    rng = np.random.default_rng(4)
    x, w = rng.standard_normal(9), rng.standard_normal(9)
    s = 0.0
    for v in x:
        s += v * v
    inv = 1.0 / (s / 9 + 1e-3) ** 0.5
    assert np.allclose(oracle.rms_norm(x, w, 1e-3), [x[i] * inv * w[i] for i in range(9)], rtol=1e-13)


def test_append_splits_latent_and_rope():
    rng = np.random.default_rng(5)
    r, dr = 16, 8
    kv_a = rng.standard_normal((2, 3, r + dr))
    w = rng.standard_normal(r)
    lat, rope = oracle.append_compressed(kv_a, w, 1e-6, [5, 0], 10000.0, r, dr)
    assert np.allclose(lat, oracle.rms_norm(kv_a[..., :r], w, 1e-6))
    # row 1 starts at position 0: token 0 is the plain de-interleave of its pairs
    assert np.array_equal(rope[1, 0], np.concatenate([kv_a[1, 0, r::2], kv_a[1, 0, r + 1::2]]))
    # pair norms are preserved at every position
    a, b = kv_a[..., r::2], kv_a[..., r + 1::2]
    assert np.allclose(a * a + b * b, rope[..., :dr // 2] ** 2 + rope[..., dr // 2:] ** 2)


@pytest.mark.parametrize("eps", [-1.0, float("nan"), float("inf")])
def test_rms_norm_rejects_bad_epsilon(eps):
    with pytest.raises(oracle.OracleError):
        oracle.rms_norm(np.ones(4), np.ones(4), eps)


def test_o_proj_brute_force_and_unit_rows():
    rng = np.random.default_rng(6)
    ctx, w = rng.standard_normal((3, 7)), rng.standard_normal((5, 7))
    ref = [[sum(ctx[m, k] * w[n, k] for k in range(7)) for n in range(5)] for m in range(3)]
    assert np.allclose(oracle.o_proj(ctx, w), ref, rtol=1e-13)
    # a unit context row selects a column of w_o (an input feature across outputs)
    e = np.zeros((1, 7))
    e[0, 4] = 1.0
    assert np.array_equal(oracle.o_proj(e, w)[0], w[:, 4])
    with pytest.raises(oracle.OracleError):
        oracle.o_proj(ctx, w[:, :6])
