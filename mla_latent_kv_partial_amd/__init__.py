"""Python binding of libmla.so: MLA latent-KV decode and reconstructed prefill on MI355X.

Each function marshals torch tensors (device memory) and the current HIP
stream into the C entry point of the same name in include/mla.h; all
arithmetic runs in the library's HIP kernels.  Outputs not passed in are
allocated with torch on the inputs' device.
"""

from __future__ import annotations

import ctypes
import math
import numbers

import torch

from ._lib import (EXPORTS, LIB_PATH, MLA_DTYPE_BF16, MLA_DTYPE_F32, MlaError, check, i32_array, i64_array,
                   lib)

__all__ = [
    "MlaError", "LIB_PATH", "EXPORTS", "mla_rope_partial_interleaved", "mla_absorb_q", "mla_decode_latent_attn",
    "mla_decode_combine", "mla_absorb_v", "mla_prefill_reconstructed", "mla_version", "split_count",
    "plan_chunk_len", "prefill_workspace_bytes", "mla_dsa_topk_select", "mla_append_compressed",
    "mla_o_proj", "mla_decode_query", "mla_dsa_topk_select_noalloc",
]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16 expected")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _host_list(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return [int(v) for v in x.detach().cpu().reshape(-1).tolist()]
    if isinstance(x, (int,)):
        return [int(x)]
    return [int(v) for v in x]


def _collapse(shape, strides, lo, hi):
    """(size, stride) of axes [lo, hi) viewed as one axis, or None if not viewable."""
    size, stride = 1, 0
    dims = [(shape[i], strides[i]) for i in range(lo, hi) if shape[i] != 1]
    if not dims:
        return 1, 0
    size, stride = dims[-1]
    for n, s in reversed(dims[:-1]):
        if s != stride * size:
            return None
        size *= n
    return size, stride


def mla_version() -> int:
    return int(lib.mla_version())


def split_count(n_attended: int, chunk_len: int) -> int:
    return -(-int(n_attended) // int(chunk_len))


def plan_chunk_len(n_attended, slots: int, tile: int = 32, min_tiles: int = 2) -> int:
    """Smallest multiple of `tile`, and at least `min_tiles` tiles, whose split
    count over all rows fits `slots` concurrent workgroups (the decode kernel
    runs one workgroup per CU), so the launch finishes in one round.  Two tiles
    at least: a split's fixed cost (first-tile wait, partial write) then covers
    two tiles, and the merge reads half as many partials (a 4096-token row:
    31.4 instead of 34.8 us per decode layer).  Host-side scheduling only."""
    n = [int(v) for v in n_attended]
    total = sum(n)
    if not n or total == 0:
        return tile
    chunk = max(tile * min_tiles, -(-total // max(slots, 1)))
    chunk = -(-chunk // tile) * tile
    while sum(split_count(v, chunk) for v in n) > slots and chunk < max(n):
        chunk += tile
    return chunk


def mla_rope_partial_interleaved(x: torch.Tensor, position_offset, rotary_dims: int, theta: float,
                                 token_axis: int = 1, out: torch.Tensor | None = None) -> torch.Tensor:
    """Partial interleaved RoPE of `x` (rank >= 2, feature axis last); `out=x` rotates in place."""
    if x.dim() < 2:
        raise ValueError(f"x has ndim {x.dim()}: a token axis and a feature axis are needed")
    rank = x.dim()
    axis = token_axis + rank if token_axis < 0 else token_axis
    if not 0 <= axis < rank - 1:
        raise ValueError("RoPE token axis must lie before the feature axis")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.stride() != x.stride() or out.dtype != x.dtype:
        raise ValueError("out must match x in shape, strides and dtype")
    if x.stride(-1) != 1:
        raise ValueError("the feature axis must have stride 1")
    offsets = _host_list(position_offset)
    per_row = not isinstance(position_offset, numbers.Integral)
    shape, strides = list(x.shape), list(x.stride())
    lead = _collapse(shape, strides, 0, axis)
    inner = _collapse(shape, strides, axis + 1, rank - 1)
    if lead is None or inner is None:
        raise ValueError("x cannot be viewed as [batch, tokens, inner, feat]; make it contiguous")
    batch, sb = lead
    if per_row:
        if axis == 0:
            raise ValueError("per-row offsets index axis 0: put the tokens on another axis")
        if len(offsets) != shape[0]:
            raise ValueError(f"{len(offsets)} offsets for {shape[0]} rows")
        rep = batch // shape[0] if shape[0] else 1
        offsets = [o for o in offsets for _ in range(rep)]
    tokens, st = shape[axis], strides[axis]
    n_inner, si = inner
    offs = i64_array(offsets)
    check(lib.mla_rope_partial_interleaved(
        _dtype_code(x), _ptr(x), _ptr(out), batch, tokens, n_inner, shape[-1], sb, st, si, int(rotary_dims),
        float(theta), offs, len(offsets), _stream(x)), "mla_rope_partial_interleaved")
    return out


def mla_absorb_q(q_nope: torch.Tensor, w_kv_b: torch.Tensor, v_head: int,
                 q_lat: torch.Tensor | None = None) -> torch.Tensor:
    """q_nope [B,H,dn] (strided, last stride 1), w_kv_b [H*(dn+dv), r] -> q_lat [B,H,r] of q_nope's dtype."""
    b, h, dn = q_nope.shape
    r = w_kv_b.shape[1]
    if q_nope.dtype != w_kv_b.dtype:
        raise TypeError("q_nope and w_kv_b must share a dtype")
    if q_nope.stride(2) != 1 or not w_kv_b.is_contiguous():
        raise ValueError("q_nope needs feature stride 1 and w_kv_b must be contiguous")
    if q_lat is None:
        q_lat = torch.empty((b, h, r), dtype=q_nope.dtype, device=q_nope.device)
    if q_lat.dtype != q_nope.dtype or not q_lat.is_contiguous() or tuple(q_lat.shape) != (b, h, r):
        raise ValueError("q_lat must be a contiguous [B,H,r] tensor of q_nope's dtype")
    check(lib.mla_absorb_q(_dtype_code(q_nope), _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(w_kv_b),
                           _ptr(q_lat), b, h, dn, int(v_head), r, _stream(q_nope)), "mla_absorb_q")
    return q_lat


def mla_decode_query(q_nope: torch.Tensor, q_rope: torch.Tensor, w_kv_b: torch.Tensor, v_head: int, positions,
                     theta: float, q_lat: torch.Tensor | None = None,
                     q_rope_out: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """The decode query in one call: q_nope [B,H,dn] -> q_lat [B,H,r] (as mla_absorb_q) and
    q_rope [B,H,dr] -> q_rope_out rotated at positions[b] (as mla_rope_partial_interleaved over the
    whole rope part).  q_rope_out=q_rope rotates in place; otherwise it must match q_rope's strides."""
    b, h, dn = q_nope.shape
    r = w_kv_b.shape[1]
    if q_nope.dtype != w_kv_b.dtype or q_rope.dtype != q_nope.dtype:
        raise TypeError("q_nope, q_rope and w_kv_b must share a dtype")
    if q_rope.dim() != 3 or tuple(q_rope.shape[:2]) != (b, h):
        raise ValueError("q_rope must be [B,H,dr] with q_nope's B and H")
    if q_nope.stride(2) != 1 or q_rope.stride(2) != 1 or not w_kv_b.is_contiguous():
        raise ValueError("q_nope and q_rope need feature stride 1 and w_kv_b must be contiguous")
    if q_lat is None:
        q_lat = torch.empty((b, h, r), dtype=q_nope.dtype, device=q_nope.device)
    if q_lat.dtype != q_nope.dtype or not q_lat.is_contiguous() or tuple(q_lat.shape) != (b, h, r):
        raise ValueError("q_lat must be a contiguous [B,H,r] tensor of q_nope's dtype")
    if q_rope_out is None:   # the same strides as q_rope (the ABI takes one stride pair for both)
        q_rope_out = torch.empty_strided(q_rope.shape, q_rope.stride(), dtype=q_rope.dtype, device=q_rope.device)
    if (q_rope_out.shape != q_rope.shape or q_rope_out.stride() != q_rope.stride()
            or q_rope_out.dtype != q_rope.dtype):
        raise ValueError("q_rope_out must match q_rope in shape, strides and dtype")
    pos = _host_list(positions)
    if len(pos) != b:
        raise ValueError("one position per row is required")
    check(lib.mla_decode_query(_dtype_code(q_nope), _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_rope),
                               _ptr(q_rope_out), q_rope.stride(0), q_rope.stride(1), _ptr(w_kv_b), _ptr(q_lat), b, h,
                               dn, q_rope.shape[2], int(v_head), r, i64_array(pos), float(theta), _stream(q_nope)),
          "mla_decode_query")
    return q_lat, q_rope_out


def mla_decode_latent_attn(q_lat: torch.Tensor, q_rope: torch.Tensor, latent: torch.Tensor, rope: torch.Tensor,
                           kv_len, softmax_scale: float, chunk_len: int, sel_idx: torch.Tensor | None = None,
                           sel_count=None, part_o: torch.Tensor | None = None,
                           part_lse: torch.Tensor | None = None, s_max: int | None = None,
                           dev_err: torch.Tensor | None = None, part_dtype: torch.dtype = torch.float32):
    """Split-T latent attention partials.  Returns (part_o, part_lse, n_splits list).

    latent [B,W,r] and rope [B,W,dr] (strided views of a cache; feature stride 1);
    kv_len and sel_count are host sequences; sel_idx an int32 device tensor.
    part_o is float32 or bfloat16 (its dtype when given, else part_dtype).
    """
    b, h, r = q_lat.shape
    w = latent.shape[1]
    dr = rope.shape[2]
    lens = _host_list(kv_len)
    counts = _host_list(sel_count)
    n_att = [c if counts is not None and c > 0 else n for n, c in zip(lens, counts or [-1] * b)]
    n_splits = [split_count(n, chunk_len) for n in n_att]
    if s_max is None:
        s_max = max(n_splits) if n_splits else 1
    dev = q_lat.device
    if part_o is None:
        part_o = torch.empty((b, h, s_max, r), dtype=part_dtype, device=dev)
    if part_lse is None:
        part_lse = torch.empty((b, h, s_max), dtype=torch.float32, device=dev)
    if sel_idx is not None and sel_idx.dtype != torch.int32:
        raise TypeError("sel_idx must be int32")
    if latent.stride(2) != 1 or rope.stride(2) != 1 or q_rope.stride(2) != 1:
        raise ValueError("feature axes must have stride 1")
    if q_lat.dtype != latent.dtype or not q_lat.is_contiguous():
        raise ValueError("q_lat must be contiguous and share the cache dtype")
    check(lib.mla_decode_latent_attn(
        _dtype_code(latent), _ptr(q_lat), _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(latent), latent.stride(0), latent.stride(1), _ptr(rope), rope.stride(0), rope.stride(1),
        b, h, r, dr, w, i32_array(lens), _ptr(sel_idx), None if counts is None else i32_array(counts),
        float(softmax_scale), int(chunk_len), _dtype_code(part_o), _ptr(part_o), _ptr(part_lse), int(s_max),
        _ptr(dev_err), _stream(q_lat)), "mla_decode_latent_attn")
    return part_o, part_lse, n_splits


def mla_decode_combine(part_o: torch.Tensor, part_lse: torch.Tensor, n_splits, o_lat: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, want_lse: bool = True):
    """Merge partials (float32 or bfloat16) into o_lat [B,H,r] (and lse [B,H])."""
    b, h, s_max, r = part_o.shape
    if o_lat is None:
        o_lat = torch.empty((b, h, r), dtype=torch.float32, device=part_o.device)
    if lse is None and want_lse:
        lse = torch.empty((b, h), dtype=torch.float32, device=part_o.device)
    check(lib.mla_decode_combine(_dtype_code(part_o), _ptr(part_o), _ptr(part_lse), b, h, r, s_max,
                                 i32_array(_host_list(n_splits)), _ptr(o_lat), _ptr(lse), _stream(part_o)),
          "mla_decode_combine")
    return o_lat, lse


def mla_absorb_v(o_lat: torch.Tensor, w_kv_b: torch.Tensor, qk_nope: int, v_head: int,
                 ctx: torch.Tensor | None = None) -> torch.Tensor:
    """o_lat fp32 [B,H,r] -> ctx fp32 [B,H*dv]."""
    b, h, r = o_lat.shape
    if ctx is None:
        ctx = torch.empty((b, h * v_head), dtype=torch.float32, device=o_lat.device)
    if not (o_lat.is_contiguous() and w_kv_b.is_contiguous()):
        raise ValueError("o_lat and w_kv_b must be contiguous")
    check(lib.mla_absorb_v(_dtype_code(w_kv_b), _ptr(o_lat), _ptr(w_kv_b), _ptr(ctx), b, h, int(qk_nope),
                           int(v_head), r, _stream(o_lat)), "mla_absorb_v")
    return ctx


def mla_decode_stream_probe(latent: torch.Tensor, rope: torch.Tensor, kv_len, chunk_len: int):
    """Measurement: stream the cache bytes mla_decode_latent_attn reads for these
    dense rows, with its launch geometry and copy schedule, computing nothing
    (packed bf16 [B, W, 576] cache only)."""
    b, w, r = latent.shape
    check(lib.mla_decode_stream_probe(_dtype_code(latent), _ptr(latent), latent.stride(0), latent.stride(1),
                                      _ptr(rope), rope.stride(0), rope.stride(1), b, r, rope.shape[2], w,
                                      i32_array(_host_list(kv_len)), int(chunk_len), _stream(latent)),
          "mla_decode_stream_probe")


def mla_decode_combine_v(part_o: torch.Tensor, part_lse: torch.Tensor, n_splits, w_kv_b: torch.Tensor, qk_nope: int,
                         v_head: int, ctx: torch.Tensor | None = None, o_lat: torch.Tensor | None = None,
                         lse: torch.Tensor | None = None):
    """Merge partials and project through W_UV in one launch: ctx fp32 [B,H*dv]
    (o_lat [B,H,r] and lse [B,H] are written too when given)."""
    b, h, s_max, r = part_o.shape
    if ctx is None:
        ctx = torch.empty((b, h * v_head), dtype=torch.float32, device=part_o.device)
    if not w_kv_b.is_contiguous():
        raise ValueError("w_kv_b must be contiguous")
    check(lib.mla_decode_combine_v(_dtype_code(w_kv_b), _dtype_code(part_o), _ptr(part_o), _ptr(part_lse), b, h, r,
                                   s_max,
                                   i32_array(_host_list(n_splits)), _ptr(w_kv_b), int(qk_nope), int(v_head), _ptr(ctx),
                                   _ptr(o_lat), _ptr(lse), _stream(part_o)), "mla_decode_combine_v")
    return ctx


def prefill_workspace_bytes(dtype: torch.dtype, batch, tokens, keys, heads, q_lora_rank, kv_lora_rank, qk_nope,
                            qk_rope, v_head) -> int:
    need = ctypes.c_size_t(0)
    code = MLA_DTYPE_BF16 if dtype == torch.bfloat16 else MLA_DTYPE_F32
    offs = i64_array([0] * max(1, batch))
    check(lib.mla_prefill_reconstructed(code, batch, tokens, keys, heads, q_lora_rank, kv_lora_rank, qk_nope, qk_rope,
                                        v_head, None, None, None, None, None, offs, 10000.0, None, 1.0, None,
                                        ctypes.byref(need), None, None), "mla_prefill_reconstructed")
    return int(need.value)


def mla_prefill_reconstructed(q_c: torch.Tensor, w_q_b: torch.Tensor, latent: torch.Tensor, rope: torch.Tensor,
                              w_kv_b: torch.Tensor, heads: int, qk_nope: int, qk_rope: int, v_head: int, q_offsets,
                              theta: float, softmax_scale: float | None = None, left_pad=None,
                              workspace: torch.Tensor | None = None, ctx: torch.Tensor | None = None) -> torch.Tensor:
    """Causal prefill: q_c [B,T,ql], latent [B,K,r], rope [B,K,dr] (rotated) -> ctx fp32 [B,T,H*dv]."""
    b, t, ql = q_c.shape
    k, r = latent.shape[1], latent.shape[2]
    for name, ten in (("q_c", q_c), ("w_q_b", w_q_b), ("latent", latent), ("rope", rope), ("w_kv_b", w_kv_b)):
        if not ten.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(qk_nope + qk_rope)
    need = prefill_workspace_bytes(q_c.dtype, b, t, k, heads, ql, r, qk_nope, qk_rope, v_head)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_c.device)
    if ctx is None:
        ctx = torch.empty((b, t, heads * v_head), dtype=torch.float32, device=q_c.device)
    size = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    pads = _host_list(left_pad)
    check(lib.mla_prefill_reconstructed(
        _dtype_code(q_c), b, t, k, heads, ql, r, int(qk_nope), int(qk_rope), int(v_head), _ptr(q_c), _ptr(w_q_b),
        _ptr(latent), _ptr(rope), _ptr(w_kv_b), i64_array(_host_list(q_offsets)), float(theta),
        None if pads is None else i32_array(pads), float(softmax_scale), _ptr(workspace), ctypes.byref(size),
        _ptr(ctx), _stream(q_c)), "mla_prefill_reconstructed")
    return ctx


def dsa_topk_workspace_bytes(row_len, top_k: int) -> int:
    """Workspace bytes mla_dsa_topk_select needs for rows of these lengths (0
    when every row runs on one workgroup)."""
    lens = _host_list(row_len)
    size = ctypes.c_size_t(0)
    counts = i32_array([0] * max(len(lens), 1))
    stride = max(lens) if lens else 1
    check(lib.mla_dsa_topk_select(ctypes.c_void_p(16), stride, len(lens), i32_array(lens), int(top_k), None, counts,
                                  None, ctypes.byref(size), None), "mla_dsa_topk_select")
    return int(size.value)


def mla_dsa_topk_select(scores: torch.Tensor, row_len, top_k: int, sel_idx: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, two_stage: bool = True):
    """DSA top-k positions of each row of fp32 scores [B, W] (row b: scores[b, :row_len[b]]).

    Returns (sel_idx int32 device tensor, sel_count host list): the form
    mla_decode_latent_attn takes (rows with row_len <= top_k stay dense, -1).
    two_stage: long rows run on several workgroups with a workspace (allocated
    here unless given); False keeps every row on one workgroup."""
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    if scores.dim() == 1:
        scores = scores.view(1, -1)
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be [B, W] with a unit feature stride")
    lens = _host_list(row_len)
    b = scores.shape[0]
    if len(lens) != b:
        raise ValueError("row_len needs one entry per score row")
    total = sum(int(top_k) for n in lens if n > top_k)
    if sel_idx is None:
        sel_idx = torch.empty(max(total, 1), dtype=torch.int32, device=scores.device)
    elif sel_idx.dtype != torch.int32 or sel_idx.numel() < total:
        raise ValueError("sel_idx must be int32 with room for every selected index")
    counts = i32_array([0] * b)
    size = None
    if two_stage:
        size = ctypes.c_size_t(0)
        check(lib.mla_dsa_topk_select(_ptr(scores), scores.stride(0), b, i32_array(lens), int(top_k), None, counts,
                                      None, ctypes.byref(size), _stream(scores)), "mla_dsa_topk_select")
        if workspace is None:
            workspace = torch.empty(max(size.value, 1), dtype=torch.uint8, device=scores.device)
        elif workspace.numel() * workspace.element_size() < size.value:
            raise ValueError("workspace too small")
        size = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    check(lib.mla_dsa_topk_select(_ptr(scores), scores.stride(0), b, i32_array(lens), int(top_k), _ptr(sel_idx),
                                  counts, _ptr(workspace) if two_stage else None,
                                  ctypes.byref(size) if two_stage else None, _stream(scores)), "mla_dsa_topk_select")
    return sel_idx[:total], [int(c) for c in counts]


def mla_dsa_topk_select_noalloc(scores: torch.Tensor, row_len, top_k: int, sel_idx: torch.Tensor):
    """mla_dsa_topk_select without a workspace: the library's fixed device
    scratch serves the long rows (at most 32 of them per call).  sel_idx (int32,
    room for top_k per selected row) is the caller's; nothing is allocated.
    Returns (sel_idx[:selected], sel_count host list)."""
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    if scores.dim() == 1:
        scores = scores.view(1, -1)
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be [B, W] with a unit feature stride")
    lens = _host_list(row_len)
    b = scores.shape[0]
    if len(lens) != b:
        raise ValueError("row_len needs one entry per score row")
    total = sum(int(top_k) for n in lens if n > top_k)
    if sel_idx.dtype != torch.int32 or sel_idx.numel() < total:
        raise ValueError("sel_idx must be int32 with room for every selected index")
    counts = i32_array([0] * b)
    check(lib.mla_dsa_topk_select_noalloc(_ptr(scores), scores.stride(0), b, i32_array(lens), int(top_k),
                                          _ptr(sel_idx), counts, _stream(scores)), "mla_dsa_topk_select_noalloc")
    return sel_idx[:total], [int(c) for c in counts]


def mla_append_compressed(kv_a: torch.Tensor, norm_weight: torch.Tensor, eps: float, positions, theta: float,
                          latent: torch.Tensor, rope: torch.Tensor, slot: int) -> None:
    """RMSNorm(kv_a[..., :r]) and RoPE(kv_a[..., r:]) written to latent[:, slot:slot+T] / rope[:, slot:slot+T].

    kv_a [B, T, r + dr]; latent [B, W, r] and rope [B, W, dr] are cache views
    (feature stride 1); positions: host sequence, RoPE position of token 0 per row."""
    b, t, width = kv_a.shape
    r, dr = latent.shape[2], rope.shape[2]
    if width != r + dr:
        raise ValueError("kv_a must hold kv_lora_rank + rope_dim features")
    if not (kv_a.dtype == norm_weight.dtype == latent.dtype == rope.dtype):
        raise TypeError("kv_a, norm_weight and the cache must share a dtype")
    if kv_a.stride(2) != 1 or latent.stride(2) != 1 or rope.stride(2) != 1 or not norm_weight.is_contiguous():
        raise ValueError("feature axes must have stride 1")
    if slot < 0 or slot + t > latent.shape[1] or slot + t > rope.shape[1]:
        raise ValueError("slot + tokens must fit the cache")
    check(lib.mla_append_compressed(
        _dtype_code(kv_a), _ptr(kv_a), kv_a.stride(0), kv_a.stride(1), b, t, r, dr, _ptr(norm_weight),
        float(eps), i64_array(_host_list(positions)), float(theta), _ptr(latent), latent.stride(0),
        latent.stride(1), _ptr(rope), rope.stride(0), rope.stride(1), int(slot), _stream(kv_a)),
        "mla_append_compressed")


def mla_o_proj(ctx: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """ctx fp32 [..., in] (contiguous), w_o [hidden, in] -> out fp32 [..., hidden]."""
    if ctx.dtype != torch.float32 or not ctx.is_contiguous() or not w_o.is_contiguous():
        raise ValueError("ctx must be contiguous fp32 and w_o contiguous")
    hidden, width = w_o.shape
    if ctx.shape[-1] != width:
        raise ValueError("ctx width != w_o input width")
    rows = ctx.numel() // width
    if out is None:
        out = torch.empty((*ctx.shape[:-1], hidden), dtype=torch.float32, device=ctx.device)
    need = ctypes.c_size_t(0)
    check(lib.mla_o_proj_workspace_bytes(_dtype_code(w_o), rows, width, hidden, ctypes.byref(need)),
          "mla_o_proj_workspace_bytes")
    if need.value and (workspace is None or workspace.numel() * workspace.element_size() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=ctx.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.mla_o_proj(_dtype_code(w_o), _ptr(ctx), rows, width, _ptr(w_o), hidden, _ptr(out), _ptr(workspace),
                         nbytes, _stream(ctx)), "mla_o_proj")
    return out

