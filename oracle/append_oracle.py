"""Plain CPU oracle of the fused cache append.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts: Glm52Mla.project splits the
kv_a_proj_with_mqa output [B, T, r + dr] into the latent part (first r) and
the rope part (last dr); the latent goes through rmsNormF32Mlx with the
kv_a_layernorm weight, the rope part through partialInterleavedRopeMlx at the
row's position offset; Glm52Mla.forward then appends both to the cache.
rmsNormF32Mlx: x * rsqrt(mean(x^2) + eps) * w, computed in float32 on the
page, in float64 here; eps must be finite and >= 0.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import OracleError, rope_partial_interleaved


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis in float64."""
    if not np.isfinite(eps) or eps < 0:
        raise OracleError(f"eps={eps}: need a finite value >= 0")
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (x.shape[-1],):
        raise OracleError("RMSNorm weight must match the feature width")
    mean = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(mean + eps) * w


def append_compressed(kv_a: np.ndarray, weight: np.ndarray, eps: float, positions, theta: float,
                      kv_lora_rank: int, rope_dim: int):
    """kv_a [B, T, r + dr] -> (latent [B, T, r], rotated rope [B, T, dr]) as appended to the cache;
    token t of row b is rotated at position positions[b] + t."""
    kv_a = np.asarray(kv_a, dtype=np.float64)
    if kv_a.ndim != 3 or kv_a.shape[-1] != kv_lora_rank + rope_dim:
        raise OracleError("kv_a must be [B, T, kv_lora_rank + rope_dim]")
    latent = rms_norm(kv_a[..., :kv_lora_rank], weight, eps)
    rope = rope_partial_interleaved(kv_a[..., kv_lora_rank:], [int(p) for p in positions], rope_dim, theta)
    return latent, rope


def o_proj(ctx: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, the o_proj linear after
    attendReconstructed / attendAbsorbed: out[m, :] = ctx[m, :] . w_o^T with
    w_o stored [hidden, heads * v_head] (out features, in features)."""
    ctx = np.asarray(ctx, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    if ctx.shape[-1] != w_o.shape[1]:
        raise OracleError("o_proj: context width != weight input width")
    return ctx @ w_o.T
