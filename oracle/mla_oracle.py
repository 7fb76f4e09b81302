"""Plain fp64 CPU oracle for GLM-5.2-style multi-head latent attention (MLA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library and its
Python binding never import it, and it imports nothing from them.

What it computes follows the three "mlx-bun" diff pages (my.diffend.io):
  * "mlx-bun 0.0.11 -> 0.0.13", file glm52-mla.ts: partial interleaved RoPE
    (partialInterleavedRopeMlx), the reconstructed attention path
    (Glm52Mla.attendReconstructed), the weight-absorbed single-token decode
    (Glm52Mla.attendAbsorbed, including the DSA selected-position gather) and
    the ragged-row dispatch of Glm52Mla.forward;
  * "mlx-bun 0.2.0 -> 0.4.0", file glm52-mla.ts: the left-padding mask added to
    attendReconstructed; file glm52-cache.ts: right-aligned rows with per-row
    lengths and left padding.

Everything is float64.  Inputs are the exact values the GPU consumes (bf16 or
fp32 widened without rounding).  Where the pages leave a step open the reading
taken is stated at the function.  The split-softmax partials and their combine
are not on the pages; they are the exact decomposition of the page's softmax
and are defined here from the mathematics (log-sum-exp algebra).
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np


class OracleError(ValueError):
    """An argument the pages reject (they throw an Error with a message)."""


# ---------------------------------------------------------------------------
# Partial interleaved RoPE
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx.
# ---------------------------------------------------------------------------

def rope_inverse_frequencies(rotary_dims: int, theta: float) -> np.ndarray:
    """Per-pair inverse frequency, float32, built the way the page builds it.

    For pair p the exponent is the f32 rounding of the double quotient -2p/R;
    the inverse frequency is the f32 rounding of the double power
    f32(theta) ** exponent.
    """
    half = rotary_dims // 2
    out = np.empty(half, dtype=np.float32)
    theta32 = float(np.float32(theta))
    for p in range(half):
        exponent = float(np.float32(float(-2 * p) / float(rotary_dims)))
        out[p] = np.float32(math.pow(theta32, exponent))
    return out


def rope_angles(positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """f32 angle = f32 rounding of the double product position * inverse frequency.

    positions: integer array [...]; returns float32 [..., half].
    """
    pos = np.asarray(positions, dtype=np.float64)[..., None]
    return (pos * inv_freq.astype(np.float64)).astype(np.float32)


def rope_rotate(x: np.ndarray, angles: np.ndarray, rotary_dims: int) -> np.ndarray:
    """Rotate the pair-interleaved prefix of the last axis by `angles`.

    x: [..., D] float64; angles: broadcastable to [..., R/2] (float32 values).
    Input prefix [a0,b0,a1,b1,...]; output [a*c - b*s ..., b*c + a*s ...],
    the real parts first, then the imaginary parts; x[..., R:] is copied.
    cos and sin are evaluated in float64 at the f32 angle.
    """
    half = rotary_dims // 2
    c = np.cos(angles.astype(np.float64))
    s = np.sin(angles.astype(np.float64))
    a = x[..., 0:rotary_dims:2]
    b = x[..., 1:rotary_dims:2]
    y = np.array(x, dtype=np.float64, copy=True)
    y[..., :half] = a * c - b * s
    y[..., half:rotary_dims] = b * c + a * s
    return y


def rope_partial_interleaved(x: np.ndarray, position_offset, rotary_dims: int, theta: float,
                             token_axis: int = 1) -> np.ndarray:
    """The page's partial interleaved RoPE, with its argument checks.

    Positions advance along `token_axis`: token t sits at offset + t.  The
    offset is one non-negative integer, or one per entry of axis 0 (then the
    token axis must not be axis 0).
    """
    x = np.asarray(x, dtype=np.float64)
    rank = x.ndim
    # The page rejects these inputs before rotating (partialInterleavedRopeMlx);
    # the conditions are restated here, the messages are this oracle's own.
    width = x.shape[-1] if rank else 0
    if (not isinstance(rotary_dims, (int, np.integer)) or isinstance(rotary_dims, bool)
            or not 0 < rotary_dims <= width or rotary_dims % 2):
        raise OracleError(f"rotary_dims={rotary_dims}: need an even count in (0, {width}]")
    if not (math.isfinite(theta) and theta > 0):
        raise OracleError(f"theta={theta}: need a finite value > 0")
    if rank < 2:
        raise OracleError(f"input of ndim {rank}: need a token axis and a feature axis")
    axis = token_axis + rank if token_axis < 0 else token_axis
    if not 0 <= axis < rank - 1:
        raise OracleError(f"token_axis={token_axis}: need an axis before the last (feature) axis of a {rank}-d input")
    per_row = not np.isscalar(position_offset) and not isinstance(position_offset, (int, np.integer))
    offsets = list(position_offset) if per_row else [position_offset]
    if per_row and (axis == 0 or len(offsets) != x.shape[0]):
        raise OracleError(f"{len(offsets)} per-row offsets with tokens on axis {axis}: need one offset for each "
                          f"of the {x.shape[0]} entries of axis 0, and the tokens on another axis")
    if any(isinstance(o, bool) or not isinstance(o, (int, np.integer)) or int(o) < 0 for o in offsets):
        raise OracleError("position offsets: need integers >= 0")

    tokens = x.shape[axis]
    half = rotary_dims // 2
    inv = rope_inverse_frequencies(rotary_dims, theta)
    rows = len(offsets)
    pos = np.array([[int(offsets[r]) + t for t in range(tokens)] for r in range(rows)], dtype=np.int64)
    ang = rope_angles(pos, inv)                      # [rows, tokens, half]
    shape = [1] * rank
    if per_row:
        shape[0] = rows
    shape[axis] = tokens
    shape[-1] = half
    ang = ang.reshape(shape)
    return rope_rotate(x, ang, rotary_dims)


# ---------------------------------------------------------------------------
# kv_b_proj row layout
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, attendAbsorbed: per head h the
# key block W_UK is rows [h(dn+dv), h(dn+dv)+dn) ([qk_nope, latent]) and the
# value block W_UV is the next dv rows ([value, latent]).
# ---------------------------------------------------------------------------

def split_kv_b(w_kvb: np.ndarray, heads: int, qk_nope: int, v_head: int):
    w = np.asarray(w_kvb, dtype=np.float64)
    rows, rank = w.shape
    if rows != heads * (qk_nope + v_head):
        raise OracleError("kv_b_proj rows != heads * (qk_nope + v_head)")
    w = w.reshape(heads, qk_nope + v_head, rank)
    return w[:, :qk_nope, :], w[:, qk_nope:, :]


def absorb_q(q_nope: np.ndarray, w_kvb: np.ndarray, qk_nope: int, v_head: int) -> np.ndarray:
    """Latent-space query q_lat[b,h,:] = q_nope[b,h,:] @ W_UK[h]  ([B,H,dn] -> [B,H,r])."""
    q = np.asarray(q_nope, dtype=np.float64)
    w_uk, _ = split_kv_b(w_kvb, q.shape[1], qk_nope, v_head)
    return np.einsum("bhd,hdr->bhr", q, w_uk)


def absorb_v(o_lat: np.ndarray, w_kvb: np.ndarray, qk_nope: int, v_head: int) -> np.ndarray:
    """Per-head output ctx[b,h,:] = o_lat[b,h,:] @ W_UV[h]^T, heads concatenated ([B,H,r] -> [B,H*dv])."""
    o = np.asarray(o_lat, dtype=np.float64)
    b, h, _ = o.shape
    _, w_uv = split_kv_b(w_kvb, h, qk_nope, v_head)
    return np.einsum("bhr,hvr->bhv", o, w_uv).reshape(b, h * v_head)


# ---------------------------------------------------------------------------
# Attended tokens of a row
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, Glm52Mla.forward (each row
# sliced from its left pad) and attendAbsorbed (DSA gather along the token axis
# of the row's valid slice; host lists non-empty and inside the prefix).
# Page "mlx-bun 0.2.0 -> 0.4.0", glm52-cache.ts: rows are right-aligned, so
# row b's valid tokens occupy [W - len_b, W).
# ---------------------------------------------------------------------------

def attended_positions(kv_len: int, selection) -> np.ndarray:
    """Indices into the row's valid slice, in the order attended.

    selection None means every valid token in order.  A selection is checked as
    the page checks a host list: non-empty, every entry an integer in [0, kv_len).
    Duplicates are attended once per occurrence (a gather keeps them).
    """
    if kv_len < 1:
        raise OracleError(f"kv_len={kv_len}: a decode row holds at least one token")
    if selection is None:
        return np.arange(kv_len, dtype=np.int64)
    sel = np.asarray(selection)
    if sel.ndim != 1 or sel.size == 0:
        raise OracleError("selection list: need a 1-d list with at least one entry")
    if not np.issubdtype(sel.dtype, np.integer):
        raise OracleError("selection list: need integer entries")
    if sel.min() < 0 or sel.max() >= kv_len:
        raise OracleError(f"selection list: entries must lie in [0, {kv_len})")
    return sel.astype(np.int64)


def row_tokens(cache: np.ndarray, row: int, kv_len: int, positions: np.ndarray) -> np.ndarray:
    """Gather the attended tokens of one right-aligned row: cache[row, W-len+positions]."""
    width = cache.shape[1]
    if kv_len > width:
        raise OracleError("row length exceeds the cache width")
    valid = np.asarray(cache[row, width - kv_len:], dtype=np.float64)
    return valid[positions]


def softmax(scores: np.ndarray, axis: int = -1) -> np.ndarray:
    """Max-subtracted softmax; -inf entries get probability zero."""
    m = np.max(scores, axis=axis, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def _selections(batch: int, selections):
    if selections is None:
        return [None] * batch
    if len(selections) != batch:
        raise OracleError(f"{len(selections)} selection entries for {batch} rows")
    return list(selections)


# ---------------------------------------------------------------------------
# Decode, reconstructed definition (the plain definition of the result).
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, attendReconstructed at one
# query token: per-head K_nope and V from kv_b_proj, the rope key broadcast over
# heads, scores scaled by 1/sqrt(qk_head_dim) (passed as `scale`), softmax,
# P.V, heads concatenated.  Rows are independent (forward's per-row loop).
# ---------------------------------------------------------------------------

def decode_reconstructed(q_nope, q_rope, latent, rope, w_kvb, kv_len, selections, scale,
                         qk_nope: int, v_head: int) -> np.ndarray:
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    batch, heads, _ = q_nope.shape
    w_uk, w_uv = split_kv_b(w_kvb, heads, qk_nope, v_head)
    out = np.zeros((batch, heads * v_head))
    for b, sel in enumerate(_selections(batch, selections)):
        pos = attended_positions(int(kv_len[b]), sel)
        c = row_tokens(latent, b, int(kv_len[b]), pos)            # [n, r]
        rho = row_tokens(rope, b, int(kv_len[b]), pos)            # [n, dr]
        k_nope = np.einsum("nr,hdr->hnd", c, w_uk)                # [H, n, dn]
        v = np.einsum("nr,hvr->hnv", c, w_uv)                     # [H, n, dv]
        key = np.concatenate([k_nope, np.broadcast_to(rho, (heads,) + rho.shape)], axis=-1)
        query = np.concatenate([q_nope[b], q_rope[b]], axis=-1)   # [H, dn+dr]
        s = scale * np.einsum("hk,hnk->hn", query, key)
        p = softmax(s, axis=-1)
        out[b] = np.einsum("hn,hnv->hv", p, v).reshape(-1)
    return out


# ---------------------------------------------------------------------------
# Decode, absorbed form.
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, attendAbsorbed: q_lat =
# q_nope.W_UK, scores = q_lat.latent^T + q_rope.rope^T (scaled), softmax,
# latent context = P.latent, output = latent context . W_UV^T.
# ---------------------------------------------------------------------------

def latent_attention(q_lat, q_rope, latent, rope, kv_len, selections, scale):
    """Softmax attention of latent-space queries over latent||rope tokens.

    Returns o_lat [B,H,r] (the normalised latent context) and lse [B,H]
    (natural-log normaliser of the scaled scores).
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    batch, heads, rank = q_lat.shape
    o_lat = np.zeros((batch, heads, rank))
    lse = np.zeros((batch, heads))
    for b, sel in enumerate(_selections(batch, selections)):
        pos = attended_positions(int(kv_len[b]), sel)
        c = row_tokens(latent, b, int(kv_len[b]), pos)
        rho = row_tokens(rope, b, int(kv_len[b]), pos)
        s = scale * (q_lat[b] @ c.T + q_rope[b] @ rho.T)          # [H, n]
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=-1, keepdims=True)
        o_lat[b] = (e @ c) / l
        lse[b] = (m + np.log(l))[:, 0]
    return o_lat, lse


def decode_absorbed(q_nope, q_rope, latent, rope, w_kvb, kv_len, selections, scale,
                    qk_nope: int, v_head: int) -> dict:
    q_lat = absorb_q(q_nope, w_kvb, qk_nope, v_head)
    o_lat, lse = latent_attention(q_lat, q_rope, latent, rope, kv_len, selections, scale)
    ctx = absorb_v(o_lat, w_kvb, qk_nope, v_head)
    return {"q_lat": q_lat, "o_lat": o_lat, "lse": lse, "ctx": ctx}


# ---------------------------------------------------------------------------
# Split-T partials and their combine (flash-decoding).  Not on the pages: the
# exact decomposition of the softmax above.  The attended list of a row is cut,
# in list order, into contiguous chunks of `chunk_len`; chunk s yields
#   m_s = max score, l_s = sum exp(score - m_s),
#   o_s = sum exp(score - m_s) c / l_s,   lse_s = m_s + ln l_s.
# Combining: LSE = ln sum_s exp(lse_s);  o = sum_s exp(lse_s - LSE) o_s.
# ---------------------------------------------------------------------------

def split_count(n_attended: int, chunk_len: int) -> int:
    if chunk_len < 1:
        raise OracleError("chunk_len must be positive")
    return -(-n_attended // chunk_len)


def latent_attention_partials(q_lat, q_rope, latent, rope, kv_len, selections, scale, chunk_len: int,
                              s_max: int | None = None):
    """Per-split partials: part_o [B,H,S,r], part_lse [B,H,S], n_splits [B].

    Unused split slots (s >= n_splits[b]) hold lse = -inf and o = 0.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    batch, heads, rank = q_lat.shape
    sels = _selections(batch, selections)
    positions = [attended_positions(int(kv_len[b]), sels[b]) for b in range(batch)]
    n_splits = np.array([split_count(len(p), chunk_len) for p in positions], dtype=np.int32)
    s_total = int(n_splits.max()) if s_max is None else int(s_max)
    if s_total < n_splits.max():
        raise OracleError("s_max smaller than the number of splits")
    part_o = np.zeros((batch, heads, s_total, rank))
    part_lse = np.full((batch, heads, s_total), -np.inf)
    for b in range(batch):
        pos = positions[b]
        for s in range(n_splits[b]):
            chunk = pos[s * chunk_len:(s + 1) * chunk_len]
            c = row_tokens(latent, b, int(kv_len[b]), chunk)
            rho = row_tokens(rope, b, int(kv_len[b]), chunk)
            sc = scale * (q_lat[b] @ c.T + q_rope[b] @ rho.T)
            m = sc.max(axis=-1, keepdims=True)
            e = np.exp(sc - m)
            l = e.sum(axis=-1, keepdims=True)
            part_o[b, :, s] = (e @ c) / l
            part_lse[b, :, s] = (m + np.log(l))[:, 0]
    return part_o, part_lse, n_splits


def combine_partials(part_o, part_lse, n_splits):
    """Merge split partials into o_lat [B,H,r] and lse [B,H]."""
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    batch, heads, _, rank = part_o.shape
    o = np.zeros((batch, heads, rank))
    lse = np.full((batch, heads), -np.inf)
    for b in range(batch):
        n = int(n_splits[b])
        if n < 1:
            raise OracleError("a row needs at least one split")
        l = part_lse[b, :, :n]                                    # [H, n]
        m = l.max(axis=-1, keepdims=True)
        finite = np.isfinite(m[:, 0])
        w = np.where(np.isfinite(l), np.exp(l - np.where(np.isfinite(m), m, 0.0)), 0.0)
        tot = w.sum(axis=-1, keepdims=True)
        safe = np.where(tot > 0, tot, 1.0)
        o[b] = np.einsum("hs,hsr->hr", w / safe, part_o[b, :, :n])
        lse[b] = np.where(finite, (m + np.log(safe))[:, 0], -np.inf)
    return o, lse


# ---------------------------------------------------------------------------
# Reconstructed causal prefill.
# Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts: project (q_b_proj from the
# normalised q-LoRA state, reshape [B,T,H,dn+dr], split, RoPE on the rope part
# at offset + t) and attendReconstructed (kv_b_proj expansion, rope key
# broadcast over heads, scaled scores, causal mask with last visible key
# prefix + t, softmax, P.V).  Page "mlx-bun 0.2.0 -> 0.4.0", glm52-mla.ts: keys
# before the row's left pad are masked as well.
# ---------------------------------------------------------------------------

def prefill_queries(c_q, w_qb, q_offsets, theta, heads: int, qk_nope: int, qk_rope: int,
                    query_rows: Sequence[int] | None = None):
    """The prefill queries of page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
    Glm52Mla.project, from the normalised q-LoRA state on.

    q = c_q . w_qb^T ([B, T', H*(dn+dr)]), viewed as [B, T', H, dn+dr]: head h
    owns features [h(dn+dr), (h+1)(dn+dr)) of the projection.  Within a head the
    first dn features are q_nope and the last dr the rope part, which is rotated
    by partial interleaved RoPE at position q_offsets[b] + t.
    Returns (q_nope [B, T', H, dn], q_rope [B, T', H, dr]).
    """
    c_q = np.asarray(c_q, dtype=np.float64)
    w_qb = np.asarray(w_qb, dtype=np.float64)
    batch, tokens, _ = c_q.shape
    qk = qk_nope + qk_rope
    if w_qb.shape[0] != heads * qk:
        raise OracleError("q_b_proj rows != heads * (qk_nope + qk_rope)")
    rows = np.arange(tokens) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    inv = rope_inverse_frequencies(qk_rope, theta)
    q_nope = np.zeros((batch, len(rows), heads, qk_nope))
    q_rope = np.zeros((batch, len(rows), heads, qk_rope))
    for b in range(batch):
        q = (c_q[b, rows] @ w_qb.T).reshape(len(rows), heads, qk)
        q_nope[b] = q[..., :qk_nope]
        ang = rope_angles(int(q_offsets[b]) + rows, inv)[:, None, :]   # [T', 1, dr/2]
        q_rope[b] = rope_rotate(q[..., qk_nope:], ang, qk_rope)
    return q_nope, q_rope


def prefill_reconstructed(c_q, w_qb, latent, rope, w_kvb, q_offsets, theta, left_pad, scale,
                          heads: int, qk_nope: int, qk_rope: int, v_head: int,
                          query_rows: Sequence[int] | None = None) -> np.ndarray:
    """Context [B, T', H*dv] for query tokens `query_rows` (default all T).

    c_q [B,T,ql] normalised q-LoRA state; w_qb [H*(dn+dr), ql]; latent [B,K,r];
    rope [B,K,dr] already-rotated keys; q_offsets[b] = RoPE position of query
    token 0 of row b; left_pad[b] = masked leading keys of row b (None = 0).
    """
    c_q = np.asarray(c_q, dtype=np.float64)
    w_qb = np.asarray(w_qb, dtype=np.float64)
    latent = np.asarray(latent, dtype=np.float64)
    rope = np.asarray(rope, dtype=np.float64)
    batch, tokens, _ = c_q.shape
    keys = latent.shape[1]
    if keys < tokens:
        raise OracleError(f"keys={keys} < tokens={tokens}: the key block includes the query block")
    qk = qk_nope + qk_rope
    if w_qb.shape[0] != heads * qk:
        raise OracleError("q_b_proj rows != heads * (qk_nope + qk_rope)")
    rows = np.arange(tokens) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    prefix = keys - tokens
    pads = np.zeros(batch, dtype=np.int64) if left_pad is None else np.asarray(left_pad, dtype=np.int64)
    w_uk, w_uv = split_kv_b(w_kvb, heads, qk_nope, v_head)
    q_nope_all, q_rope_all = prefill_queries(c_q, w_qb, q_offsets, theta, heads, qk_nope, qk_rope, rows)
    out = np.zeros((batch, len(rows), heads * v_head))
    for b in range(batch):
        q_nope, q_rope = q_nope_all[b], q_rope_all[b]
        k_nope = np.einsum("kr,hdr->hkd", latent[b], w_uk)              # [H, K, dn]
        v = np.einsum("kr,hvr->hkv", latent[b], w_uv)                   # [H, K, dv]
        kidx = np.arange(keys)
        visible = (kidx[None, :] >= pads[b]) & (kidx[None, :] <= prefix + rows[:, None])   # [T', K]
        for h in range(heads):
            s = scale * (q_nope[:, h] @ k_nope[h].T + q_rope[:, h] @ rope[b].T)
            s = np.where(visible, s, -np.inf)
            with np.errstate(invalid="ignore"):
                p = softmax(s, axis=-1)       # a query that sees no key has no defined output (NaN)
            out[b, :, h * v_head:(h + 1) * v_head] = p @ v[h]
    return out
