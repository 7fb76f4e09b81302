"""Seeded synthetic inputs for the MLA latent-KV decode / prefill workloads.

This module only draws random numbers and converts fp32 to bf16 storage.  It
holds none of the attention arithmetic, so both the CPU oracle (through the
tests) and the HIP path consume exactly the same bytes from it.

Recipe:
  * generator: NumPy PCG64 seeded with SeedSequence([config_id, tensor_id, layer]);
  * activations (q_nope, q_rope_raw, c_q, latent, rope, k_rope_raw) ~ N(0, 1);
  * weights ~ N(0, std = 1/sqrt(fan_in)), fan_in = input width of the linear
    layer as stored [out, in];
  * bf16 storage by round-to-nearest-even of the fp32 draw.
"""

from __future__ import annotations

import numpy as np

# Tensor identifiers used in the seed sequence.  Stable: changing one changes
# every stored expectation that depends on it.
T_Q_NOPE = 1
T_Q_ROPE_RAW = 2
T_LATENT = 3
T_ROPE = 4
T_W_KVB = 5
T_LENGTHS = 6
T_SELECTION = 7
T_C_Q = 8
T_W_QB = 9
T_K_ROPE_RAW = 10
T_MISC = 11
T_DSA_SCORES = 12

BF16_QUIET_NAN = np.uint16(0x7FC0)


def rng_for(config_id: int, tensor_id: int, layer: int = 0, row: int | None = None) -> np.random.Generator:
    """Independent, reproducible stream per (config, tensor, layer[, row])."""
    entropy = [int(config_id), int(tensor_id), int(layer)]
    if row is not None:
        entropy.append(int(row))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy)))


def normal_f32(config_id: int, tensor_id: int, shape, std: float = 1.0, layer: int = 0,
               row: int | None = None) -> np.ndarray:
    g = rng_for(config_id, tensor_id, layer, row)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN; finite values that round past the largest
    bf16 become +-inf, as in IEEE conversion.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QUIET_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of a bf16 bit pattern to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def ragged_lengths(config_id: int, batch: int, low: int, high: int, layer: int = 0) -> np.ndarray:
    """Per-row cache lengths drawn uniformly from the integers [low, high], both ends included."""
    g = rng_for(config_id, T_LENGTHS, layer)
    return g.integers(low, high, size=batch, endpoint=True).astype(np.int32)


def dsa_positions(config_id: int, tokens: int, count: int, layer: int = 0) -> np.ndarray:
    """Sorted unique int32 positions in [0, tokens) that always include tokens-1.

    count-1 positions are drawn without replacement from [0, tokens-1), then the
    newest position tokens-1 is added.
    """
    if count < 1 or count > tokens:
        raise ValueError("selection count must lie in [1, tokens]")
    g = rng_for(config_id, T_SELECTION, layer)
    picked = g.choice(tokens - 1, size=count - 1, replace=False) if count > 1 else np.empty(0, np.int64)
    out = np.sort(np.concatenate([picked, [tokens - 1]])).astype(np.int32)
    return out


def right_aligned(values: np.ndarray, lengths: np.ndarray, width: int, pad_value) -> np.ndarray:
    """Place row b's first lengths[b] entries of `values` right-aligned in `width` slots.

    values: [B, >=max(lengths), F]; the pad region [0, width-lengths[b]) holds pad_value.
    """
    b, _, f = values.shape
    out = np.empty((b, width, f), dtype=values.dtype)
    for row in range(b):
        n = int(lengths[row])
        out[row, : width - n] = pad_value
        out[row, width - n :] = values[row, :n]
    return out
