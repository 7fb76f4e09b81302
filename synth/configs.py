"""The five MLA workloads, as concrete seeded inputs.

Names say what each workload is:
  tiny_f32          B=1, H=4, dn=32, dr=16, dv=32, r=64, T=128, fp32
  dense_bf16        B=1, H=64, dn=128, dr=64, dv=128, r=512, T=4096, bf16 cache
  ragged_bf16       as dense_bf16 with B=8, per-row lengths ~ U{1024..32768}
  dsa_bf16          B=1, T=131072 bf16 cache, 2048 selected positions
  prefill_bf16      B=1, 4096 new tokens, H=64, q_lora_rank=1536, causal

Storage arrays are NumPy: bf16 tensors as uint16 bit patterns, fp32 tensors as
float32.  `values()` widens either exactly to float64 for the oracle.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import generators as g

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    config_id: int
    dtype: str
    batch: int
    heads: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora_rank: int
    tokens: int                      # cache width for dense rows
    ragged: tuple | None = None      # (low, high) inclusive length draw
    selected: int | None = None      # DSA selected positions (B == 1)
    theta: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.qk_nope + self.qk_rope)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    config_id: int
    dtype: str
    batch: int
    tokens: int                      # new query tokens T
    keys: int                        # cached + new keys K (K >= T)
    heads: int
    q_lora_rank: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora_rank: int
    theta: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.qk_nope + self.qk_rope)


TINY_F32 = DecodeConfig("tiny_f32", 1, F32, 1, 4, 32, 16, 32, 64, 128)
DENSE_BF16 = DecodeConfig("dense_bf16", 2, BF16, 1, 64, 128, 64, 128, 512, 4096)
RAGGED_BF16 = DecodeConfig("ragged_bf16", 3, BF16, 8, 64, 128, 64, 128, 512, 32768, ragged=(1024, 32768))
DSA_BF16 = DecodeConfig("dsa_bf16", 4, BF16, 1, 64, 128, 64, 128, 512, 131072, selected=2048)
PREFILL_BF16 = PrefillConfig("prefill_bf16", 5, BF16, 1, 4096, 4096, 64, 1536, 128, 64, 128, 512)

DECODE_CONFIGS = (TINY_F32, DENSE_BF16, RAGGED_BF16, DSA_BF16)
ALL_CONFIGS = DECODE_CONFIGS + (PREFILL_BF16,)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draw -> storage array of the config's dtype."""
    if dtype == BF16:
        return g.f32_to_bf16_bits(x)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def values(x: np.ndarray) -> np.ndarray:
    """Storage array -> exact float64 values."""
    if x.dtype == np.uint16:
        return g.bf16_bits_to_f32(x).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    raise TypeError(x.dtype)


def pad_value(dtype: str):
    """Pad slots hold NaN so that any read of them that reaches arithmetic shows."""
    return g.BF16_QUIET_NAN if dtype == BF16 else np.float32(np.nan)


@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q_nope: np.ndarray        # [B,H,dn]
    q_rope_raw: np.ndarray    # [B,H,dr]   pair-interleaved, not yet rotated
    latent: np.ndarray        # [B,W,r]    right-aligned, pad = NaN
    rope: np.ndarray          # [B,W,dr]   already-rotated keys
    w_kvb: np.ndarray         # [H*(dn+dv), r]
    kv_len: np.ndarray        # int32 [B]
    offsets: np.ndarray       # int64 [B]  RoPE position of the query token
    sel_idx: np.ndarray | None = None    # int32, concatenated per row
    sel_count: np.ndarray | None = None  # int32 [B]; -1 = dense row

    @property
    def width(self) -> int:
        return self.latent.shape[1]

    def attended(self, row: int) -> np.ndarray:
        """Indices into row's valid slice that the row attends, in list order."""
        if self.sel_count is None or self.sel_count[row] < 0:
            return np.arange(int(self.kv_len[row]), dtype=np.int64)
        start = int(np.sum(np.maximum(self.sel_count[:row], 0)))
        return self.sel_idx[start : start + int(self.sel_count[row])].astype(np.int64)


def decode_inputs(cfg: DecodeConfig, layer: int = 0, batch: int | None = None,
                  lengths=None) -> DecodeInputs:
    """Seeded inputs of a decode workload.

    `batch` overrides the row count (ragged draws); `lengths` fixes the per-row
    cache lengths instead of drawing them (smaller parity cases).
    """
    cid = cfg.config_id
    b = cfg.batch if batch is None else batch
    h, dn, dr, dv, r = cfg.heads, cfg.qk_nope, cfg.qk_rope, cfg.v_head, cfg.kv_lora_rank
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int32)
        b = len(lengths)
        width = int(lengths.max())
    elif cfg.ragged is not None:
        lengths = g.ragged_lengths(cid, b, cfg.ragged[0], cfg.ragged[1], layer)
        width = int(lengths.max())
    else:
        lengths = np.full(b, cfg.tokens, dtype=np.int32)
        width = cfg.tokens
    q_nope = store(g.normal_f32(cid, g.T_Q_NOPE, (b, h, dn), layer=layer), cfg.dtype)
    q_rope_raw = store(g.normal_f32(cid, g.T_Q_ROPE_RAW, (b, h, dr), layer=layer), cfg.dtype)
    w_kvb = store(g.normal_f32(cid, g.T_W_KVB, (h * (dn + dv), r), std=1.0 / math.sqrt(r), layer=layer), cfg.dtype)
    storage = np.uint16 if cfg.dtype == BF16 else np.float32
    latent = np.empty((b, width, r), dtype=storage)
    rope = np.empty((b, width, dr), dtype=storage)
    pad = pad_value(cfg.dtype)
    for row in range(b):
        n = int(lengths[row])
        latent[row, : width - n] = pad
        rope[row, : width - n] = pad
        latent[row, width - n :] = store(g.normal_f32(cid, g.T_LATENT, (n, r), layer=layer, row=row), cfg.dtype)
        rope[row, width - n :] = store(g.normal_f32(cid, g.T_ROPE, (n, dr), layer=layer, row=row), cfg.dtype)
    offsets = lengths.astype(np.int64)
    sel_idx = sel_count = None
    if cfg.selected is not None:
        if b != 1:
            raise ValueError("the DSA workload has one row")
        sel_idx = g.dsa_positions(cid, int(lengths[0]), cfg.selected, layer)
        sel_count = np.array([cfg.selected], dtype=np.int32)
    return DecodeInputs(cfg, q_nope, q_rope_raw, latent, rope, w_kvb, lengths, offsets, sel_idx, sel_count)


@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    c_q: np.ndarray           # [B,T,ql]   normalized q-LoRA state
    w_qb: np.ndarray          # [H*(dn+dr), ql]
    latent: np.ndarray        # [B,K,r]
    k_rope_raw: np.ndarray    # [B,K,dr]   pair-interleaved, rotated at positions 0..K-1 before use
    w_kvb: np.ndarray         # [H*(dn+dv), r]
    q_offsets: np.ndarray     # int64 [B]  position of query token 0 (= K - T)
    left_pad: np.ndarray | None = None   # int32 [B]


def prefill_inputs(cfg: PrefillConfig, layer: int = 0, tokens: int | None = None,
                   keys: int | None = None) -> PrefillInputs:
    """Seeded prefill inputs.  `tokens` / `keys` override T and K (smaller parity
    sizes; keys defaults to tokens when only tokens is given)."""
    cid = cfg.config_id
    t = cfg.tokens if tokens is None else tokens
    k = (cfg.keys if tokens is None else tokens) if keys is None else keys
    if k < t:
        raise ValueError("keys must be >= tokens")
    b, h, ql = cfg.batch, cfg.heads, cfg.q_lora_rank
    dn, dr, dv, r = cfg.qk_nope, cfg.qk_rope, cfg.v_head, cfg.kv_lora_rank
    c_q = store(g.normal_f32(cid, g.T_C_Q, (b, t, ql), layer=layer), cfg.dtype)
    w_qb = store(g.normal_f32(cid, g.T_W_QB, (h * (dn + dr), ql), std=1.0 / math.sqrt(ql), layer=layer), cfg.dtype)
    latent = store(g.normal_f32(cid, g.T_LATENT, (b, k, r), layer=layer), cfg.dtype)
    k_rope_raw = store(g.normal_f32(cid, g.T_K_ROPE_RAW, (b, k, dr), layer=layer), cfg.dtype)
    w_kvb = store(g.normal_f32(cid, g.T_W_KVB, (h * (dn + dv), r), std=1.0 / math.sqrt(r), layer=layer), cfg.dtype)
    q_offsets = np.full(b, k - t, dtype=np.int64)
    return PrefillInputs(cfg, c_q, w_qb, latent, k_rope_raw, w_kvb, q_offsets)


def with_shape(cfg, **changes):
    """A copy of a config with some geometry changed (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)
