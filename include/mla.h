/*
 * mla.h - C ABI of libmla.so: the hot path of GLM-5.2-style multi-head latent
 * attention (MLA) over a compressed KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Definitions follow the three "mlx-bun" diff pages on my.diffend.io:
 *   [P1] "mlx-bun 0.0.11 -> 0.0.13", package/src/model/glm52-mla.ts
 *   [P2] "mlx-bun 0.2.0 -> 0.4.0", glm52-mla.ts (left-padding mask) and
 *        glm52-cache.ts (right-aligned rows, per-row lengths, left pad)
 *   [P2] also glm52-dsa.ts (selectGlm52DsaDevice, the DSA top-k selection)
 *   [P3] "mlx-bun 0.4.0 -> 1.0.0", glm52.ts (the DSA indexer's dense fallback)
 *
 * A decode step is the chain
 *   mla_rope_partial_interleaved (q rope part)  ->  mla_absorb_q  ->
 *   mla_decode_latent_attn  ->  mla_decode_combine  ->  mla_absorb_v
 * (mla_decode_query does the first two in one call, mla_decode_combine_v the
 * last two)
 * and a prefill block is one call of mla_prefill_reconstructed.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the comment says [host].
 *   - Ownership: the caller owns every buffer.  The library never allocates,
 *     frees or keeps a pointer beyond the work it enqueues on `stream`; the
 *     caller keeps buffers alive until that work completes (the pages' rule
 *     that returned arrays are caller-owned, [P1] Glm52Mla.project).
 *   - No entry point synchronises the device or the stream.  Work is enqueued
 *     on `stream` (NULL = the default stream) and runs in stream order.
 *   - Element strides are in elements, not bytes; the innermost (feature)
 *     stride is always 1.
 *   - dtype: MLA_DTYPE_F32 or MLA_DTYPE_BF16 names the storage type of the
 *     activations, cache and weights an entry reads, and of the absorbed query
 *     q_lat (the bf16 path rounds its fp32 accumulation to nearest even once;
 *     the MFMA score operand is bf16 either way).  Accumulation is always
 *     fp32; partials, o_lat, lse and ctx are always fp32.
 *   - Errors: arguments are checked on the host before anything is enqueued,
 *     as the pages throw synchronously.  A failed check returns a negative
 *     mla_status and enqueues nothing; mla_last_error() then returns a
 *     message (thread-local, valid until the next call on that thread).  A
 *     launch failure returns MLA_ERR_DEVICE.  Entry points are re-entrant.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1
} mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_ARG = -1,        /* null pointer, bad dtype, non-positive geometry */
  MLA_ERR_SHAPE = -2,      /* shapes that do not fit one another */
  MLA_ERR_ROPE = -3,       /* RoPE argument rules of [P1] partialInterleavedRopeMlx */
  MLA_ERR_SELECTION = -4,  /* DSA selection counts */
  MLA_ERR_WORKSPACE = -5,  /* workspace missing or too small */
  MLA_ERR_DEVICE = -6,     /* a HIP call or kernel launch failed */
  MLA_ERR_UNSUPPORTED = -7 /* valid by the pages, outside this library's limits */
} mla_status;

/* Message of the last failed call on this thread ("" after success). */
const char* mla_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int mla_version(void);

/*
 * Partial interleaved RoPE.  [P1] partialInterleavedRopeMlx.
 *
 * x and y are logical [batch, tokens, inner, feat] arrays of `dtype` with the
 * same element strides (stride_b, stride_t, stride_i, 1); y may equal x (in
 * place), otherwise they must not overlap.  For each row vector v = x[b,t,i,:]
 * the first rotary_dims features hold pairs (a_p, b_p) = (v[2p], v[2p+1]),
 * p < rotary_dims/2, and
 *     y[p]          = a_p cos(ang) - b_p sin(ang)
 *     y[R/2 + p]    = b_p cos(ang) + a_p sin(ang)
 *     y[R .. feat)  = v[R .. feat)            (non-rotary tail kept)
 * with position = offsets[b or 0] + t, inverse frequency
 * f32(pow(f32(theta), f32(-2p/R))) and ang = f32(position * inverse frequency),
 * all as on the page.  cos/sin and the rotation are evaluated in double and
 * rounded once to `dtype`.
 *
 * offsets [host] int64: n_offsets == 1 (one offset for every row) or
 * n_offsets == batch (one per row).  Rules of the page, MLA_ERR_ROPE when
 * broken: offsets >= 0; rotary_dims > 0, even, <= feat; theta finite and > 0.
 * Limits (MLA_ERR_UNSUPPORTED): rotary_dims <= 512; offset + tokens <= 2^53.
 * Any of batch, tokens, inner may be 0 (nothing is enqueued).
 */
int mla_rope_partial_interleaved(int32_t dtype, const void* x, void* y,
                                 int32_t batch, int32_t tokens, int32_t inner, int32_t feat,
                                 int64_t stride_b, int64_t stride_t, int64_t stride_i,
                                 int32_t rotary_dims, double theta,
                                 const int64_t* offsets, int32_t n_offsets,
                                 hipStream_t stream);

/*
 * Absorb the no-PE query into latent space.  [P1] Glm52Mla.attendAbsorbed:
 * the key block of head h is W_UK[h] = w_kv_b rows [h(dn+dv), h(dn+dv)+dn),
 * a [dn, r] matrix, and the latent-space query is q_nope . W_UK.
 *
 *   q_lat[b,h,c] = sum_d q_nope[b,h,d] * w_kv_b[h*(dn+dv) + d, c]
 *
 * q_nope: [batch, heads, qk_nope] of `dtype`, strides (q_stride_b, q_stride_h, 1).
 * w_kv_b: [heads*(qk_nope+v_head), kv_lora_rank] of `dtype`, row-major, contiguous.
 * q_lat:  [batch, heads, kv_lora_rank] of `dtype`, contiguous.
 */
int mla_absorb_q(int32_t dtype, const void* q_nope, int64_t q_stride_b, int64_t q_stride_h,
                 const void* w_kv_b, void* q_lat,
                 int32_t batch, int32_t heads, int32_t qk_nope, int32_t v_head, int32_t kv_lora_rank,
                 hipStream_t stream);

/*
 * The decode query in one call: the page's query split into its no-PE part,
 * absorbed as in mla_absorb_q, and its rope part, rotated as in
 * mla_rope_partial_interleaved ([P1] Glm52Mla.project and attendAbsorbed:
 * q_pe takes RoPE at the row's position before the scores).  The results are
 * those of the two entries:
 *   q_lat      = mla_absorb_q(q_nope)
 *   q_rope_out = mla_rope_partial_interleaved(q_rope_in) with tokens = 1,
 *                inner = heads, feat = rotary_dims = qk_rope, offsets = positions
 * computed in one launch where the bf16 MFMA absorb applies (the rotation runs
 * while the weight tiles are in flight), else in two launches.
 *
 * q_nope:     [batch, heads, qk_nope] of `dtype`, strides (qn_stride_b, qn_stride_h, 1).
 * q_rope_in:  [batch, heads, qk_rope] of `dtype`, strides (qr_stride_b, qr_stride_h, 1);
 * q_rope_out: same strides; may equal q_rope_in (in place), else must not overlap it.
 * w_kv_b, q_lat as in mla_absorb_q.
 * positions [host] int64[batch]: the RoPE position of each row's query token.
 * Errors as in the two entries (MLA_ERR_ROPE: odd or non-positive qk_rope,
 * negative position, theta not finite and > 0; MLA_ERR_UNSUPPORTED: qk_rope > 512,
 * position >= 2^53).  batch may be 0 (nothing is enqueued).
 */
int mla_decode_query(int32_t dtype, const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                     const void* q_rope_in, void* q_rope_out, int64_t qr_stride_b, int64_t qr_stride_h,
                     const void* w_kv_b, void* q_lat,
                     int32_t batch, int32_t heads, int32_t qk_nope, int32_t qk_rope, int32_t v_head,
                     int32_t kv_lora_rank, const int64_t* positions, double theta,
                     hipStream_t stream);

/*
 * Latent decode attention, split-T partials.  [P1] Glm52Mla.attendAbsorbed
 * (scores = scale*(q_lat.latent^T + q_rope.rope^T), softmax, P.latent) with
 * the DSA gather of the same function and the ragged rows of Glm52Mla.forward;
 * [P2] glm52-cache.ts for the right-aligned cache.
 *
 * Cache: row b holds kv_len[b] valid tokens right-aligned in `width` slots,
 * i.e. token j (0 <= j < kv_len[b]) of the row's valid slice is slot
 * width - kv_len[b] + j.  latent [batch, width, kv_lora_rank] and
 * rope [batch, width, rope_dim] are `dtype` arrays with element strides
 * (latent_stride_b, latent_stride_t, 1) and (rope_stride_b, rope_stride_t, 1);
 * a packed [batch, width, r+dr] cache passes rope = latent + r and equal
 * strides.  Pad slots are never read.
 *
 * Attended list A_b of row b: all valid tokens in order when sel_count is
 * NULL or sel_count[b] == -1; otherwise sel_count[b] >= 1 indices
 * into the valid slice, read from sel_idx starting at the sum of the positive
 * sel_count entries of the rows before b (rows concatenated), attended in list
 * order, duplicates once per occurrence.  An index outside [0, kv_len[b]) is
 * skipped (it contributes nothing) and, when dev_err is not NULL, *dev_err is
 * set to a non-zero value on the device.  sel_count[b] == 0 is
 * MLA_ERR_SELECTION (the page rejects an empty selection).
 *
 * A_b is cut in list order into n_b = ceil(|A_b| / chunk_len) splits of
 * chunk_len tokens (the last may be shorter).  For split s of row b and head h
 *   score_j  = softmax_scale * (q_lat[b,h,:] . latent_j + q_rope[b,h,:] . rope_j)
 *   m        = max_j score_j,   l = sum_j exp(score_j - m)
 *   part_o[b,h,s,:] = sum_j exp(score_j - m) latent_j / l
 *   part_lse[b,h,s] = m + ln l
 * A split whose indices were all skipped stores o = 0 and lse = -inf.
 * Slots s >= n_b are left untouched.
 *
 * q_lat [batch, heads, kv_lora_rank] of `dtype`, contiguous; q_rope [batch, heads,
 * rope_dim] of `dtype`, strides (qr_stride_b, qr_stride_h, 1), already rotated.
 * kv_len [host] int32[batch], each in [1, width] (MLA_ERR_SHAPE otherwise).
 * sel_count [host] int32[batch] or NULL.  sel_idx device int32 (may be NULL
 * only if no row is selected).  part_o [batch, heads, s_max, r] of
 * part_dtype (MLA_DTYPE_F32, or MLA_DTYPE_BF16: each normalised split context
 * rounded once to bf16, round to nearest even; half the bytes that the
 * attention writes and the merge reads back) and part_lse [batch, heads,
 * s_max] fp32; s_max >= max_b n_b (MLA_ERR_SHAPE).
 * Limits (MLA_ERR_UNSUPPORTED): kv_lora_rank <= 1024, rope_dim <= 256.
 */
int mla_decode_latent_attn(int32_t dtype, const void* q_lat,
                           const void* q_rope, int64_t qr_stride_b, int64_t qr_stride_h,
                           const void* latent, int64_t latent_stride_b, int64_t latent_stride_t,
                           const void* rope, int64_t rope_stride_b, int64_t rope_stride_t,
                           int32_t batch, int32_t heads, int32_t kv_lora_rank, int32_t rope_dim,
                           int32_t width, const int32_t* kv_len,
                           const int32_t* sel_idx, const int32_t* sel_count,
                           float softmax_scale, int32_t chunk_len,
                           int32_t part_dtype, void* part_o, float* part_lse, int32_t s_max,
                           int32_t* dev_err, hipStream_t stream);

/*
 * Measurement, not part of the path: for a caller who wants the copy-path
 * floor of mla_decode_latent_attn at a given shape (roofline reporting).  It
 * reads exactly the cache bytes the attention reads for dense rows of a packed
 * bf16 [B, W, 576] cache (rope = latent + 512, equal strides), with the same
 * launch geometry (one workgroup per split of chunk_len attended tokens) and
 * the same HBM -> LDS copy schedule, and computes and writes nothing.
 * Arguments as in mla_decode_latent_attn.  Errors: MLA_ERR_ARG, MLA_ERR_SHAPE
 * (kv_len), MLA_ERR_UNSUPPORTED (any other layout or geometry).
 */
int mla_decode_stream_probe(int32_t dtype, const void* latent, int64_t latent_stride_b, int64_t latent_stride_t,
                            const void* rope, int64_t rope_stride_b, int64_t rope_stride_t, int32_t batch,
                            int32_t kv_lora_rank, int32_t rope_dim, int32_t width, const int32_t* kv_len,
                            int32_t chunk_len, hipStream_t stream);

/*
 * Combine split partials (flash-decoding merge).  The exact log-sum-exp
 * decomposition of the page's softmax ([P1] attendAbsorbed):
 *   LSE = ln sum_{s<n_b} exp(part_lse[b,h,s])
 *   o_lat[b,h,:] = sum_{s<n_b} exp(part_lse[b,h,s] - LSE) part_o[b,h,s,:]
 * Splits with lse = -inf contribute nothing; if every split of (b,h) is
 * empty, o_lat = 0 and lse = -inf.
 * n_splits [host] int32[batch], each in [1, s_max].  lse may be NULL.
 * part_o of part_dtype (fp32 or bf16) and the other layouts as in
 * mla_decode_latent_attn; o_lat fp32 [batch, heads, r], lse [batch, heads].
 */
int mla_decode_combine(int32_t part_dtype, const void* part_o, const float* part_lse,
                       int32_t batch, int32_t heads, int32_t kv_lora_rank, int32_t s_max,
                       const int32_t* n_splits, float* o_lat, float* lse, hipStream_t stream);

/*
 * mla_decode_combine followed by mla_absorb_v in one launch: the merged latent
 * context of each (row, head) stays on chip and is projected through the
 * head's value block ([P1] attendAbsorbed: o_lat . W_UV[h]^T, heads
 * concatenated).
 *   ctx[b, h*dv + v] = sum_c o_lat[b,h,c] * w_kv_b[h*(dn+dv) + dn + v, c]
 * with o_lat as defined for mla_decode_combine.  `dtype` is the dtype of
 * w_kv_b (layout as in mla_absorb_q); the projection accumulates in fp32 over
 * the fp32 o_lat.  part_dtype, part_o, part_lse, n_splits as in mla_decode_combine;
 * ctx fp32 [batch, heads*v_head] contiguous.  o_lat [batch, heads, r] and
 * lse [batch, heads] may be NULL; when given they receive the merge.
 * Limits (MLA_ERR_UNSUPPORTED): kv_lora_rank <= 1024.
 */
int mla_decode_combine_v(int32_t dtype, int32_t part_dtype, const void* part_o, const float* part_lse,
                         int32_t batch, int32_t heads, int32_t kv_lora_rank, int32_t s_max,
                         const int32_t* n_splits, const void* w_kv_b, int32_t qk_nope, int32_t v_head,
                         float* ctx, float* o_lat, float* lse, hipStream_t stream);

/*
 * Project the latent context out through the value block.  [P1]
 * attendAbsorbed: W_UV[h] = w_kv_b rows [h(dn+dv)+dn, (h+1)(dn+dv)), a
 * [dv, r] matrix; the head output is o_lat . W_UV^T and heads are
 * concatenated into [batch, heads*dv].
 *   ctx[b, h*dv + v] = sum_c o_lat[b,h,c] * w_kv_b[h*(dn+dv) + dn + v, c]
 * o_lat fp32 [batch, heads, r] contiguous; w_kv_b as in mla_absorb_q;
 * ctx fp32 [batch, heads*v_head] contiguous.
 */
int mla_absorb_v(int32_t dtype, const float* o_lat, const void* w_kv_b, float* ctx,
                 int32_t batch, int32_t heads, int32_t qk_nope, int32_t v_head, int32_t kv_lora_rank,
                 hipStream_t stream);

/*
 * Fused cache append.  [P1] Glm52Mla.project: the kv_a_proj_with_mqa output
 * of a token splits into the latent part (first kv_lora_rank features) and
 * the rope part (last rope_dim); the latent goes through rmsNormF32Mlx with
 * the kv_a_layernorm weight, the rope part through partialInterleavedRopeMlx
 * at the token's position; Glm52Mla.forward appends both to the cache.
 *
 *   latent[b, slot + t, :] = x * rsqrt(mean(x^2) + eps) * norm_weight,
 *                            x = kv_a[b, t, 0 .. kv_lora_rank)
 *   rope[b, slot + t, :]   = RoPE(kv_a[b, t, kv_lora_rank ..), positions[b] + t)
 *
 * In the right-aligned cache of mla_decode_latent_attn every row appends at
 * the same slot (the width before the append: slot = width) while each row's
 * RoPE position is its own length ([P2] glm52-cache.ts).
 * kv_a [batch, tokens, kv_lora_rank + rope_dim] of `dtype`, strides
 * (kv_a_stride_b, kv_a_stride_t, 1); norm_weight [kv_lora_rank] of `dtype`;
 * positions [host] int64[batch]; latent / rope: the cache arrays as in
 * mla_decode_latent_attn (the caller guarantees slot + tokens fits the
 * buffer).  The mean square is accumulated in fp32, the rotation in double;
 * each output is rounded once to `dtype`.
 * Errors: MLA_ERR_ARG (eps negative or not finite, NULL, bad strides),
 * MLA_ERR_ROPE (odd rope_dim, theta, negative positions).
 */
int mla_append_compressed(int32_t dtype, const void* kv_a, int64_t kv_a_stride_b, int64_t kv_a_stride_t,
                          int32_t batch, int32_t tokens, int32_t kv_lora_rank, int32_t rope_dim,
                          const void* norm_weight, float eps, const int64_t* positions, double theta,
                          void* latent, int64_t latent_stride_b, int64_t latent_stride_t, void* rope,
                          int64_t rope_stride_b, int64_t rope_stride_t, int32_t slot, hipStream_t stream);

/*
 * o_proj linear after the attention.  [P1] the o_proj of
 * Glm52Mla.attendReconstructed / attendAbsorbed: the per-head contexts
 * concatenated [rows, heads*v_head] times the o_proj weight, stored
 * [hidden, heads*v_head] (out features, in features):
 *
 *   out[m, n] = sum_k ctx[m, k] * w_o[n, k]
 *
 * ctx fp32 [rows, in_features] contiguous (the ctx of mla_absorb_v or of
 * mla_prefill_reconstructed); w_o [hidden, in_features] of `dtype`,
 * contiguous; out fp32 [rows, hidden].  bf16 weights: up to 64 rows stream
 * the weight once on MFMA with the fp32 context split into two bf16 parts;
 * more rows round the context to bf16 once (in the workspace) and run an MFMA
 * GEMM.  The workspace size depends on the shapes only:
 * mla_o_proj_workspace_bytes writes it (0 when none is needed, and then
 * workspace may be NULL).  Errors: MLA_ERR_ARG, MLA_ERR_WORKSPACE.
 */
int mla_o_proj_workspace_bytes(int32_t dtype, int64_t rows, int32_t in_features, int32_t hidden, size_t* bytes);
int mla_o_proj(int32_t dtype, const float* ctx, int64_t rows, int32_t in_features, const void* w_o, int32_t hidden,
               float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * DSA top-k position selection.  [P2] glm52-dsa.ts, selectGlm52DsaDevice,
 * with the dense fallback of the [P3] indexer (a context not longer than top_k is
 * attended densely).  For row b with n = row_len[b] > top_k, over the fp32
 * scores s[0..n) at scores + b * score_stride:
 *   rank key  = bitwise NOT of the order-preserving uint32 image of s[i]
 *               (negative values: all bits flipped; others: sign bit flipped)
 *   selection = the top_k positions of smallest key, equal keys (equal score
 *               bits) taken in ascending position order
 *   threshold = the minimum selected score
 *   output    = the selected positions with s[i] > threshold in ascending
 *               order, then the other selected positions in ascending order
 * Positions are relative to the row's score slice, i.e. to the valid slice of
 * the row's cache, which is what mla_decode_latent_attn takes.
 *
 * scores: device fp32, row b at scores + b * score_stride (score_stride >=
 *         max row_len when batch > 1).  Scores must not be NaN (the selection
 *         of a NaN is not defined by the page; no error is raised).
 * row_len [host] int32[batch], each in [1, 2^30].
 * sel_count [host, written] int32[batch]: top_k for a selected row, -1 for a
 *         dense row (row_len[b] <= top_k), as mla_decode_latent_attn takes it.
 * sel_idx: device int32, written with top_k entries per selected row,
 *         concatenated in row order; may be NULL only if no row is selected.
 * workspace / workspace_bytes: a row of 16385 to 131072 scores with
 *         top_k <= 16384 / ceil(row_len / 16384) (the multi-workgroup,
 *         "two-stage" rows) runs on one workgroup per 8192-score segment and
 *         then one for the row, in three launches, in caller memory of
 *         131328 bytes per such row (256-byte aligned).  workspace == NULL with
 *         workspace_bytes != NULL writes the size needed (0 when no row
 *         qualifies) and returns MLA_OK without launching.  workspace_bytes
 *         == NULL: every row runs on one workgroup.  Both ways give the same
 *         positions.
 * Errors: MLA_ERR_ARG (NULL pointers, top_k < 1, batch < 0), MLA_ERR_SHAPE
 * (row_len out of range or above score_stride), MLA_ERR_WORKSPACE (too small
 * or misaligned).
 */
int mla_dsa_topk_select(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len,
                        int32_t top_k, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                        size_t* workspace_bytes, hipStream_t stream);

/*
 * mla_dsa_topk_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The positions and sel_count are those of
 * mla_dsa_topk_select with a workspace (bit-identical).  The two-stage rows
 * (see workspace above) use a fixed scratch array in the library's device
 * memory instead: 32 such rows at most (4 MiB; each device holds its own copy
 * until the process ends), and every other row runs on one workgroup.  The
 * call allocates and frees nothing.  All calls on one device share the
 * scratch: calls that overlap on one device (several streams or threads)
 * race and must be serialised by the caller.
 * Errors: as mla_dsa_topk_select, and MLA_ERR_WORKSPACE when more than 32
 * rows take the two-stage form (split the batch); MLA_ERR_DEVICE if the
 * scratch address cannot be obtained on the current device.
 */
int mla_dsa_topk_select_noalloc(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len,
                                int32_t top_k, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream);

/*
 * Reconstructed causal prefill.  [P1] Glm52Mla.project (q_b_proj of the
 * normalised q-LoRA state, reshape [B,T,H,dn+dr], split no-PE / rope, RoPE of
 * the rope part at q_offsets[b] + t) and Glm52Mla.attendReconstructed
 * (kv_b_proj expansion to per-head K_nope / V, rope key broadcast over heads,
 * scores scaled by softmax_scale, causal mask, softmax, P.V); [P2] left pad.
 *
 *   q[b,t,h,:]  = q_c[b,t,:] . w_q_b[h*(dn+dr) + (0..dn+dr), :]^T
 *   key k is visible to query t of row b  iff  left_pad[b] <= k <= (keys - tokens) + t
 *   ctx[b,t,h*dv + v] = sum_k softmax_k(score) * V[b,k,h,v]
 *
 * q_c [batch, tokens, q_lora_rank], w_q_b [heads*(qk_nope+qk_rope), q_lora_rank],
 * latent [batch, keys, kv_lora_rank], rope [batch, keys, qk_rope] (already
 * rotated, e.g. by mla_rope_partial_interleaved), w_kv_b as above; all
 * `dtype`, contiguous.  q_offsets [host] int64[batch] >= 0.  left_pad [host]
 * int32[batch] in [0, keys] or NULL (no padding).  keys >= tokens.  A query
 * that sees no key (inside the pad) gets ctx = 0.  ctx fp32 [batch, tokens,
 * heads*v_head].
 *
 * Workspace: with workspace == NULL the call stores in *workspace_bytes a
 * size that suffices for these shapes whatever the data pointers (the other
 * pointers may be NULL then) and returns MLA_OK without enqueuing anything.
 * Otherwise *workspace_bytes must be at least the size the call's path needs
 * (never more than the queried size; MLA_ERR_WORKSPACE) and the device
 * buffer must be 256-byte aligned; its contents are scratch.
 * Limits (MLA_ERR_UNSUPPORTED): qk_nope + qk_rope <= 256, v_head <= 256,
 * qk_rope <= 512.
 */
int mla_prefill_reconstructed(int32_t dtype, int32_t batch, int32_t tokens, int32_t keys, int32_t heads,
                              int32_t q_lora_rank, int32_t kv_lora_rank,
                              int32_t qk_nope, int32_t qk_rope, int32_t v_head,
                              const void* q_c, const void* w_q_b,
                              const void* latent, const void* rope, const void* w_kv_b,
                              const int64_t* q_offsets, double theta, const int32_t* left_pad,
                              float softmax_scale,
                              void* workspace, size_t* workspace_bytes,
                              float* ctx, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
