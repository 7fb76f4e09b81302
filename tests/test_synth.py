"""The seeded generators: bf16 rounding against torch, determinism, draw ranges."""

import numpy as np
import torch

from synth import configs, generators as g


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(10000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 10000).astype(np.float32),
        # exact ties: mantissa low half = 0x8000, with even and odd kept bit
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00008000], dtype=np.uint32)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf], dtype=np.float32),
    ])
    ours = g.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(g.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_nan_stays_nan():
    b = g.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(g.bf16_bits_to_f32(b))[0]


def test_determinism_and_independent_streams():
    a = g.normal_f32(2, g.T_LATENT, (4, 8))
    b = g.normal_f32(2, g.T_LATENT, (4, 8))
    c = g.normal_f32(2, g.T_ROPE, (4, 8))
    d = g.normal_f32(2, g.T_LATENT, (4, 8), layer=1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_std_scaling():
    w = g.normal_f32(2, g.T_W_KVB, (512, 512), std=1 / np.sqrt(512))
    assert abs(w.std() - 1 / np.sqrt(512)) < 2e-3 / np.sqrt(512) * 10


def test_ragged_lengths_inclusive_range():
    x = g.ragged_lengths(3, 20000, 1024, 32768)
    assert x.min() == 1024 and x.max() == 32768
    assert x.dtype == np.int32


def test_dsa_positions_sorted_unique_with_newest():
    p = g.dsa_positions(4, 131072, 2048)
    assert p.dtype == np.int32 and p.size == 2048
    assert np.all(np.diff(p) > 0)
    assert p[-1] == 131071 and p[0] >= 0


def test_decode_inputs_layout():
    inp = configs.decode_inputs(configs.TINY_F32)
    assert inp.latent.shape == (1, 128, 64) and inp.latent.dtype == np.float32
    assert inp.rope.shape == (1, 128, 16) and inp.w_kvb.shape == (256, 64)
    assert inp.offsets.tolist() == [128]
    small = configs.with_shape(configs.RAGGED_BF16, ragged=(3, 40))
    r = configs.decode_inputs(small, batch=5)
    w = r.width
    assert w == r.kv_len.max() and r.latent.dtype == np.uint16
    for b in range(5):
        pad = w - int(r.kv_len[b])
        assert np.all(r.latent[b, :pad] == g.BF16_QUIET_NAN)
        assert not np.any(r.latent[b, pad:] == g.BF16_QUIET_NAN)
    assert np.array_equal(r.offsets, r.kv_len.astype(np.int64))
