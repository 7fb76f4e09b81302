// C ABI of libmla.so: argument checks (mirroring the checks the pages make
// before computing), row tables, launch setup.  No allocation, no
// synchronisation: every entry point enqueues work on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>

#include "../../include/mla.h"
#include "launch.hpp"

namespace mla {

void rope_inverse_frequencies(int32_t rotary, double theta, float* out) {
  // Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx:
  // exponent = f32(-2p / R) with the quotient taken in double, inverse
  // frequency = f32(pow(f32(theta), exponent)) with the power in double.
  const double theta32 = static_cast<double>(static_cast<float>(theta));
  for (int p = 0; p < rotary / 2; ++p) {
    const float exponent = static_cast<float>(static_cast<double>(-2 * p) / static_cast<double>(rotary));
    out[p] = static_cast<float>(pow(theta32, static_cast<double>(exponent)));
  }
}

hipError_t launch_decode_generic(int32_t dtype, const DecodeParams& p, hipStream_t stream);
bool decode_mfma_supported(int32_t dtype, int32_t heads, int32_t r, int32_t dr);
bool decode_mfma_layout_ok(const void* q_lat, const void* latent, int64_t lat_sb, int64_t lat_st, const void* rope,
                           int64_t rope_sb, int64_t rope_st);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
size_t prefill_generic_workspace_bytes(const PrefillParams& p);
hipError_t launch_prefill_generic(const PrefillParams& p, hipStream_t stream);

}  // namespace mla

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return MLA_OK;
}

int device(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MLA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int32_t d) { return d == MLA_DTYPE_F32 || d == MLA_DTYPE_BF16; }
size_t elem_size(int32_t d) { return d == MLA_DTYPE_BF16 ? 2 : 4; }

const void* advance(const void* p, int64_t elems, int32_t dtype) {
  return static_cast<const char*>(p) + elems * static_cast<int64_t>(elem_size(dtype));
}

constexpr double kMaxPosition = 9007199254740992.0;   // 2^53

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_error.c_str(); }

int mla_version(void) { return 100; }

int mla_rope_partial_interleaved(int32_t dtype, const void* x, void* y, int32_t batch, int32_t tokens,
                                 int32_t inner, int32_t feat, int64_t stride_b, int64_t stride_t, int64_t stride_i,
                                 int32_t rotary_dims, double theta, const int64_t* offsets, int32_t n_offsets,
                                 hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "rope: unknown dtype %d", dtype);
  if (batch < 0 || tokens < 0 || inner < 0 || feat < 1)
    return fail(MLA_ERR_ARG, "rope: batch, tokens, inner must be >= 0 and feat >= 1");
  if (!offsets) return fail(MLA_ERR_ARG, "rope: offsets is NULL");
  if (n_offsets != 1 && n_offsets != batch)
    return fail(MLA_ERR_ROPE, "rope: n_offsets=%d, need 1 or batch=%d", n_offsets, batch);
  for (int i = 0; i < n_offsets; ++i) {
    if (offsets[i] < 0) return fail(MLA_ERR_ROPE, "rope: offsets[%d] = %lld < 0", i, static_cast<long long>(offsets[i]));
    if (static_cast<double>(offsets[i]) + tokens > kMaxPosition)
      return fail(MLA_ERR_UNSUPPORTED, "rope: offset + tokens exceeds 2^53");
  }
  if (rotary_dims <= 0 || (rotary_dims & 1) || rotary_dims > feat)
    return fail(MLA_ERR_ROPE, "rope: rotary_dims=%d, need an even count in [2, feat=%d]", rotary_dims, feat);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ROPE, "rope: theta=%g, need finite > 0", theta);
  if (rotary_dims > 2 * mla::kRopeMaxPairs)
    return fail(MLA_ERR_UNSUPPORTED, "rope: rotary_dims %d > %d", rotary_dims, 2 * mla::kRopeMaxPairs);
  if (static_cast<int64_t>(batch) * tokens * inner == 0) return ok();
  if (!x || !y) return fail(MLA_ERR_ARG, "rope: x or y is NULL");
  if (stride_b < 0 || stride_t < 0 || stride_i < 0) return fail(MLA_ERR_ARG, "rope: negative stride");

  mla::RopeParams p{};
  p.tokens = tokens;
  p.inner = inner;
  p.feat = feat;
  p.sb = stride_b;
  p.st = stride_t;
  p.si = stride_i;
  p.rotary = rotary_dims;
  p.per_row = n_offsets == batch && batch > 1 ? 1 : 0;
  p.copy_tail = (x != y) && rotary_dims < feat;
  mla::rope_inverse_frequencies(rotary_dims, theta, p.inv);
  if (!p.per_row) p.off[0] = offsets[0];
  for (int b0 = 0; b0 < batch; b0 += mla::kRopeRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kRopeRowsPerLaunch);
    p.x = advance(x, b0 * stride_b, dtype);
    p.y = const_cast<void*>(advance(y, b0 * stride_b, dtype));
    if (p.per_row)
      for (int i = 0; i < p.rows; ++i) p.off[i] = offsets[b0 + i];
    hipError_t e = mla::launch_rope(dtype, p, stream);
    if (e != hipSuccess) return device(e, "rope launch");
  }
  return ok();
}

int mla_absorb_q(int32_t dtype, const void* q_nope, int64_t q_stride_b, int64_t q_stride_h, const void* w_kv_b,
                 void* q_lat, int32_t batch, int32_t heads, int32_t qk_nope, int32_t v_head, int32_t kv_lora_rank,
                 hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "absorb_q: unknown dtype %d", dtype);
  if (batch < 0 || heads < 1 || qk_nope < 1 || v_head < 1 || kv_lora_rank < 1)
    return fail(MLA_ERR_ARG, "absorb_q: batch >= 0 and positive heads, qk_nope, v_head, kv_lora_rank required");
  if (batch == 0) return ok();
  if (!q_nope || !w_kv_b || !q_lat) return fail(MLA_ERR_ARG, "absorb_q: NULL pointer");
  if (q_stride_b < 0 || q_stride_h < 0) return fail(MLA_ERR_ARG, "absorb_q: negative stride");
  if (batch > 65535 * 8) return fail(MLA_ERR_UNSUPPORTED, "absorb_q: batch too large");
  mla::AbsorbQParams p{q_nope, q_stride_b, q_stride_h, w_kv_b, q_lat, batch, heads, qk_nope, v_head, kv_lora_rank};
  return device(mla::launch_absorb_q(dtype, p, stream), "absorb_q launch");
}

int mla_decode_query(int32_t dtype, const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                     const void* q_rope_in, void* q_rope_out, int64_t qr_stride_b, int64_t qr_stride_h,
                     const void* w_kv_b, void* q_lat, int32_t batch, int32_t heads, int32_t qk_nope,
                     int32_t qk_rope, int32_t v_head, int32_t kv_lora_rank, const int64_t* positions, double theta,
                     hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "decode_query: unknown dtype %d", dtype);
  if (batch < 0 || heads < 1 || qk_nope < 1 || v_head < 1 || kv_lora_rank < 1)
    return fail(MLA_ERR_ARG, "decode_query: batch >= 0 and positive heads, qk_nope, v_head, kv_lora_rank required");
  if (qk_rope <= 0 || (qk_rope & 1)) return fail(MLA_ERR_ROPE, "decode_query: qk_rope=%d, need an even count >= 2", qk_rope);
  if (qk_rope > 2 * mla::kRopeMaxPairs)
    return fail(MLA_ERR_UNSUPPORTED, "decode_query: qk_rope %d > %d", qk_rope, 2 * mla::kRopeMaxPairs);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ROPE, "decode_query: theta=%g, need finite > 0", theta);
  if (batch == 0) return ok();
  if (!q_nope || !q_rope_in || !q_rope_out || !w_kv_b || !q_lat || !positions)
    return fail(MLA_ERR_ARG, "decode_query: NULL pointer");
  if (qn_stride_b < 0 || qn_stride_h < 0 || qr_stride_b < 0 || qr_stride_h < 0)
    return fail(MLA_ERR_ARG, "decode_query: negative stride");
  if (batch > 65535 * 8) return fail(MLA_ERR_UNSUPPORTED, "decode_query: batch too large");
  for (int b = 0; b < batch; ++b) {
    if (positions[b] < 0) return fail(MLA_ERR_ROPE, "decode_query: positions[%d] < 0", b);
    if (positions[b] >= (int64_t{1} << 53)) return fail(MLA_ERR_UNSUPPORTED, "decode_query: position >= 2^53");
  }
  mla::RopeParams rp{};
  rp.tokens = 1;
  rp.inner = heads;
  rp.feat = qk_rope;
  rp.sb = qr_stride_b;
  rp.st = 0;
  rp.si = qr_stride_h;
  rp.rotary = qk_rope;
  rp.per_row = 1;
  rp.copy_tail = 0;   // the whole rope part rotates
  mla::rope_inverse_frequencies(qk_rope, theta, rp.inv);
  mla::AbsorbQParams p{nullptr, qn_stride_b, qn_stride_h, w_kv_b, nullptr, 0, heads, qk_nope, v_head, kv_lora_rank};
  for (int b0 = 0; b0 < batch; b0 += mla::kRopeRowsPerLaunch) {
    const int rows = std::min(batch - b0, mla::kRopeRowsPerLaunch);
    rp.rows = rows;
    rp.x = advance(q_rope_in, b0 * qr_stride_b, dtype);
    rp.y = const_cast<void*>(advance(q_rope_out, b0 * qr_stride_b, dtype));
    for (int i = 0; i < rows; ++i) rp.off[i] = positions[b0 + i];
    p.q = advance(q_nope, b0 * qn_stride_b, dtype);
    p.q_lat = const_cast<void*>(advance(q_lat, static_cast<int64_t>(b0) * heads * kv_lora_rank, dtype));
    p.batch = rows;
    hipError_t e = mla::launch_absorb_q_rope(dtype, p, rp, stream);
    if (e != hipSuccess) return device(e, "decode_query launch");
  }
  return ok();
}

int mla_absorb_v(int32_t dtype, const float* o_lat, const void* w_kv_b, float* ctx, int32_t batch, int32_t heads,
                 int32_t qk_nope, int32_t v_head, int32_t kv_lora_rank, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "absorb_v: unknown dtype %d", dtype);
  if (batch < 0 || heads < 1 || qk_nope < 1 || v_head < 1 || kv_lora_rank < 1)
    return fail(MLA_ERR_ARG, "absorb_v: batch >= 0 and positive heads, qk_nope, v_head, kv_lora_rank required");
  if (batch == 0) return ok();
  if (!o_lat || !w_kv_b || !ctx) return fail(MLA_ERR_ARG, "absorb_v: NULL pointer");
  mla::AbsorbVParams p{o_lat, w_kv_b, ctx, batch, heads, qk_nope, v_head, kv_lora_rank};
  return device(mla::launch_absorb_v(dtype, p, stream), "absorb_v launch");
}

int mla_decode_latent_attn(int32_t dtype, const void* q_lat, const void* q_rope, int64_t qr_stride_b,
                           int64_t qr_stride_h, const void* latent, int64_t latent_stride_b, int64_t latent_stride_t,
                           const void* rope, int64_t rope_stride_b, int64_t rope_stride_t, int32_t batch,
                           int32_t heads, int32_t kv_lora_rank, int32_t rope_dim, int32_t width,
                           const int32_t* kv_len, const int32_t* sel_idx, const int32_t* sel_count,
                           float softmax_scale, int32_t chunk_len, int32_t part_dtype, void* part_o,
                           float* part_lse, int32_t s_max, int32_t* dev_err, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "decode: unknown dtype %d", dtype);
  if (!valid_dtype(part_dtype)) return fail(MLA_ERR_ARG, "decode: unknown part_dtype %d", part_dtype);
  if (batch < 0 || heads < 1 || kv_lora_rank < 1 || rope_dim < 1 || width < 1)
    return fail(MLA_ERR_ARG, "decode: batch >= 0 and positive heads, kv_lora_rank, rope_dim, width required");
  if (chunk_len < 1) return fail(MLA_ERR_ARG, "decode: chunk_len must be >= 1");
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_ARG, "decode: softmax_scale must be finite");
  if (batch == 0) return ok();
  if (!q_lat || !q_rope || !latent || !rope || !kv_len || !part_o || !part_lse)
    return fail(MLA_ERR_ARG, "decode: NULL pointer");
  if (latent_stride_b < 0 || latent_stride_t < 1 || rope_stride_b < 0 || rope_stride_t < 1 || qr_stride_b < 0 ||
      qr_stride_h < 0)
    return fail(MLA_ERR_ARG, "decode: bad stride");
  if (kv_lora_rank > 1024 || rope_dim > 256)
    return fail(MLA_ERR_UNSUPPORTED, "decode: kv_lora_rank <= 1024 and rope_dim <= 256 supported");
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: heads > 65535");
  int64_t sel_total = 0;
  int max_splits = 0;
  bool any_sel = false;
  for (int b = 0; b < batch; ++b) {
    if (kv_len[b] < 1 || kv_len[b] > width)
      return fail(MLA_ERR_SHAPE, "decode: kv_len[%d] = %d outside [1, %d]", b, kv_len[b], width);
    int n = kv_len[b];
    if (sel_count) {
      if (sel_count[b] == 0) return fail(MLA_ERR_SELECTION, "decode: sel_count[%d] = 0 (a selected row attends >= 1 index)", b);
      if (sel_count[b] < -1) return fail(MLA_ERR_SELECTION, "decode: sel_count[%d] = %d", b, sel_count[b]);
      if (sel_count[b] > 0) {
        n = sel_count[b];
        sel_total += n;
        any_sel = true;
      }
    }
    max_splits = std::max(max_splits, (n + chunk_len - 1) / chunk_len);
  }
  if (sel_total > 0x7fffffffLL) return fail(MLA_ERR_UNSUPPORTED, "decode: more than 2^31-1 selected indices");
  if (any_sel && !sel_idx) return fail(MLA_ERR_ARG, "decode: sel_idx is NULL but rows are selected");
  if (s_max < max_splits) return fail(MLA_ERR_SHAPE, "decode: s_max %d < %d splits", s_max, max_splits);

  const bool mfma = mla::decode_mfma_supported(dtype, heads, kv_lora_rank, rope_dim) &&
                    mla::decode_mfma_layout_ok(q_lat, latent, latent_stride_b, latent_stride_t, rope, rope_stride_b,
                                               rope_stride_t) &&
                    (reinterpret_cast<uintptr_t>(part_o) & 15) == 0;
  mla::DecodeParams p{};
  p.qr_sb = qr_stride_b;
  p.qr_sh = qr_stride_h;
  p.lat_sb = latent_stride_b;
  p.lat_st = latent_stride_t;
  p.rope_sb = rope_stride_b;
  p.rope_st = rope_stride_t;
  p.sel = sel_idx;
  p.dev_err = dev_err;
  p.heads = heads;
  p.r = kv_lora_rank;
  p.dr = rope_dim;
  p.width = width;
  p.chunk = chunk_len;
  p.s_max = s_max;
  p.scale = softmax_scale;
  p.part_bf16 = part_dtype == MLA_DTYPE_BF16;
  int32_t sel_off = 0;
  for (int b0 = 0; b0 < batch; b0 += mla::kDecodeRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kDecodeRowsPerLaunch);
    p.s_launch = 0;
    p.tab.split_begin[0] = 0;
    for (int i = 0; i < p.rows; ++i) {
      const int b = b0 + i;
      const bool sel = sel_count && sel_count[b] > 0;
      p.tab.kv_len[i] = kv_len[b];
      p.tab.n_att[i] = sel ? sel_count[b] : kv_len[b];
      p.tab.sel_off[i] = sel ? sel_off : -1;
      if (sel) sel_off += sel_count[b];
      const int splits = (p.tab.n_att[i] + chunk_len - 1) / chunk_len;
      p.s_launch = std::max(p.s_launch, splits);
      p.tab.split_begin[i + 1] = p.tab.split_begin[i] + splits;
    }
    p.s_total = p.tab.split_begin[p.rows];
    p.q_lat = advance(q_lat, static_cast<int64_t>(b0) * heads * kv_lora_rank, dtype);
    p.q_rope = advance(q_rope, b0 * qr_stride_b, dtype);
    p.latent = advance(latent, b0 * latent_stride_b, dtype);
    p.rope = advance(rope, b0 * rope_stride_b, dtype);
    p.part_o = static_cast<char*>(part_o) +
               static_cast<int64_t>(b0) * heads * s_max * kv_lora_rank * static_cast<int64_t>(elem_size(part_dtype));
    p.part_lse = part_lse + static_cast<int64_t>(b0) * heads * s_max;
    hipError_t e = mfma ? mla::launch_decode_mfma(p, stream) : mla::launch_decode_generic(dtype, p, stream);
    if (e != hipSuccess) return device(e, "decode launch");
  }
  return ok();
}

int mla_decode_stream_probe(int32_t dtype, const void* latent, int64_t latent_stride_b, int64_t latent_stride_t,
                            const void* rope, int64_t rope_stride_b, int64_t rope_stride_t, int32_t batch,
                            int32_t kv_lora_rank, int32_t rope_dim, int32_t width, const int32_t* kv_len,
                            int32_t chunk_len, hipStream_t stream) {
  if (batch < 0 || width < 1 || chunk_len < 1) return fail(MLA_ERR_ARG, "stream_probe: bad geometry");
  if (batch == 0) return ok();
  if (!latent || !rope || !kv_len) return fail(MLA_ERR_ARG, "stream_probe: NULL pointer");
  // the packed bf16 layout the attention's copy path streams
  if (dtype != MLA_DTYPE_BF16 || kv_lora_rank != 512 || rope_dim != 64 ||
      static_cast<const char*>(rope) != static_cast<const char*>(latent) + 2 * kv_lora_rank ||
      rope_stride_b != latent_stride_b || rope_stride_t != latent_stride_t || latent_stride_t < 576 ||
      latent_stride_b < 0 || (reinterpret_cast<uintptr_t>(latent) & 15) || latent_stride_b % 8 || latent_stride_t % 8)
    return fail(MLA_ERR_UNSUPPORTED, "stream_probe: needs a packed, 16-byte aligned bf16 [B, W, 576] cache");
  for (int b = 0; b < batch; ++b)
    if (kv_len[b] < 1 || kv_len[b] > width)
      return fail(MLA_ERR_SHAPE, "stream_probe: kv_len[%d] = %d outside [1, %d]", b, kv_len[b], width);
  mla::DecodeParams p{};
  p.lat_sb = p.rope_sb = latent_stride_b;
  p.lat_st = p.rope_st = latent_stride_t;
  p.r = kv_lora_rank;
  p.dr = rope_dim;
  p.width = width;
  p.chunk = chunk_len;
  for (int b0 = 0; b0 < batch; b0 += mla::kDecodeRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kDecodeRowsPerLaunch);
    if ((static_cast<int64_t>(p.rows - 1) * latent_stride_b + static_cast<int64_t>(width - 1) * latent_stride_t) * 2 +
            1152 > 0xffffffffLL)
      return fail(MLA_ERR_UNSUPPORTED, "stream_probe: rows of a launch span more than 4 GiB");
    p.tab.split_begin[0] = 0;
    for (int i = 0; i < p.rows; ++i) {
      p.tab.kv_len[i] = kv_len[b0 + i];
      p.tab.n_att[i] = kv_len[b0 + i];
      p.tab.sel_off[i] = -1;
      p.tab.split_begin[i + 1] = p.tab.split_begin[i] + (kv_len[b0 + i] + chunk_len - 1) / chunk_len;
    }
    p.s_total = p.tab.split_begin[p.rows];
    p.latent = p.rope = advance(latent, b0 * latent_stride_b, dtype);
    hipError_t e = mla::launch_stream_probe(p, stream);
    if (e != hipSuccess) return device(e, "stream_probe launch");
  }
  return ok();
}

namespace {

// o_proj: the MFMA GEMM path (rows > 64) stages the context in bf16 in the
// workspace; its size depends on the shapes only.
bool o_proj_gemm_shape(int32_t dtype, int64_t rows, int32_t in_features, int32_t hidden) {
  return dtype == MLA_DTYPE_BF16 && rows > 64 && in_features % 64 == 0 && in_features % 8 == 0 && hidden % 4 == 0;
}

size_t o_proj_need(int32_t dtype, int64_t rows, int32_t in_features, int32_t hidden) {
  return o_proj_gemm_shape(dtype, rows, in_features, hidden)
             ? (static_cast<size_t>(rows) * in_features * 2 + 255) / 256 * 256
             : 0;
}

}  // namespace

int mla_o_proj_workspace_bytes(int32_t dtype, int64_t rows, int32_t in_features, int32_t hidden, size_t* bytes) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "o_proj: unknown dtype %d", dtype);
  if (rows < 0 || in_features < 1 || hidden < 1) return fail(MLA_ERR_ARG, "o_proj: rows >= 0, positive widths required");
  if (!bytes) return fail(MLA_ERR_ARG, "o_proj: bytes is NULL");
  *bytes = o_proj_need(dtype, rows, in_features, hidden);
  return ok();
}

int mla_o_proj(int32_t dtype, const float* ctx, int64_t rows, int32_t in_features, const void* w_o, int32_t hidden,
               float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "o_proj: unknown dtype %d", dtype);
  if (rows < 0 || in_features < 1 || hidden < 1) return fail(MLA_ERR_ARG, "o_proj: rows >= 0, positive widths required");
  if (rows > 0x7fffffffLL) return fail(MLA_ERR_UNSUPPORTED, "o_proj: rows > 2^31-1");
  if (rows == 0) return ok();
  if (!ctx || !w_o || !out) return fail(MLA_ERR_ARG, "o_proj: NULL pointer");
  const size_t need = o_proj_need(dtype, rows, in_features, hidden);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "o_proj: workspace of %zu bytes required", need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MLA_ERR_WORKSPACE, "o_proj: workspace not 256-byte aligned");
  mla::AbsorbVParams v{ctx, w_o, out, static_cast<int32_t>(rows), 1, 0, hidden, in_features};
  hipError_t e;
  if (need > 0 && (reinterpret_cast<uintptr_t>(ctx) & 15) == 0 &&
      mla::gemm_nt_mfma_ok(workspace, in_features, w_o, in_features, out, hidden, rows, hidden, in_features)) {
    uint16_t* a = static_cast<uint16_t*>(workspace);
    e = mla::launch_f32_to_bf16(ctx, a, rows * in_features, stream);
    if (e == hipSuccess) {
      mla::GemmNT g{};
      g.a = a;
      g.lda = in_features;
      g.b = static_cast<const uint16_t*>(w_o);
      g.ldb = in_features;
      g.c = out;
      g.ldc = hidden;
      g.m = static_cast<int32_t>(rows);
      g.n = hidden;
      g.k = in_features;
      e = mla::launch_gemm_nt_mfma(g, false, true, stream);
    }
  } else {
    // weight-streaming contraction of absorb_v with a single "head" (MFMA for
    // bf16 weights of a suitable shape, generic kernel otherwise)
    e = mla::launch_absorb_v(dtype, v, stream);
  }
  if (e != hipSuccess) return device(e, "o_proj launch");
  return ok();
}

int mla_append_compressed(int32_t dtype, const void* kv_a, int64_t kv_a_stride_b, int64_t kv_a_stride_t,
                          int32_t batch, int32_t tokens, int32_t kv_lora_rank, int32_t rope_dim,
                          const void* norm_weight, float eps, const int64_t* positions, double theta,
                          void* latent, int64_t latent_stride_b, int64_t latent_stride_t, void* rope,
                          int64_t rope_stride_b, int64_t rope_stride_t, int32_t slot, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "append: unknown dtype %d", dtype);
  if (batch < 0 || tokens < 0 || kv_lora_rank < 1 || rope_dim < 1 || slot < 0)
    return fail(MLA_ERR_ARG, "append: batch, tokens, slot >= 0 and positive kv_lora_rank, rope_dim required");
  if (!isfinite(eps) || eps < 0.f) return fail(MLA_ERR_ARG, "append: eps=%g, need finite >= 0", static_cast<double>(eps));
  if (rope_dim & 1) return fail(MLA_ERR_ROPE, "append: rope_dim=%d, need an even count", rope_dim);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ROPE, "append: theta=%g, need finite > 0", theta);
  if (rope_dim > 2 * mla::kRopeMaxPairs || kv_lora_rank > 65536)
    return fail(MLA_ERR_UNSUPPORTED, "append: rope_dim <= %d and kv_lora_rank <= 65536 supported", 2 * mla::kRopeMaxPairs);
  if (batch == 0 || tokens == 0) return ok();
  if (!kv_a || !norm_weight || !positions || !latent || !rope) return fail(MLA_ERR_ARG, "append: NULL pointer");
  if (kv_a_stride_b < 0 || kv_a_stride_t < 0 || latent_stride_b < 0 || latent_stride_t < 1 || rope_stride_b < 0 ||
      rope_stride_t < 1)
    return fail(MLA_ERR_ARG, "append: bad stride");
  for (int b = 0; b < batch; ++b) {
    if (positions[b] < 0) return fail(MLA_ERR_ROPE, "append: positions[%d] < 0", b);
    if (static_cast<double>(positions[b]) + tokens > kMaxPosition)
      return fail(MLA_ERR_UNSUPPORTED, "append: position + tokens exceeds 2^53");
  }
  mla::AppendParams p{};
  p.kb = kv_a_stride_b;
  p.kt = kv_a_stride_t;
  p.w = norm_weight;
  p.lb = latent_stride_b;
  p.lt = latent_stride_t;
  p.rb = rope_stride_b;
  p.rt = rope_stride_t;
  p.tokens = tokens;
  p.r = kv_lora_rank;
  p.dr = rope_dim;
  p.slot = slot;
  p.eps = eps;
  mla::rope_inverse_frequencies(rope_dim, theta, p.inv);
  for (int b0 = 0; b0 < batch; b0 += mla::kRopeRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kRopeRowsPerLaunch);
    p.kv_a = advance(kv_a, b0 * kv_a_stride_b, dtype);
    p.latent = const_cast<void*>(advance(latent, b0 * latent_stride_b, dtype));
    p.rope = const_cast<void*>(advance(rope, b0 * rope_stride_b, dtype));
    for (int i = 0; i < p.rows; ++i) p.off[i] = positions[b0 + i];
    hipError_t e = mla::launch_append(dtype, p, stream);
    if (e != hipSuccess) return device(e, "append launch");
  }
  return ok();
}

}  // extern "C"

namespace {

// Host checks of a top-k call; counts the selected indices and the rows that
// take the two-stage form.
int topk_check(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len, int32_t top_k,
               const int32_t* sel_count, int64_t* total, int64_t* two_stage) {
  if (batch < 0) return fail(MLA_ERR_ARG, "dsa_topk: batch must be >= 0");
  if (top_k < 1) return fail(MLA_ERR_ARG, "dsa_topk: top_k must be >= 1");
  *total = *two_stage = 0;
  if (batch == 0) return ok();
  if (!scores || !row_len || !sel_count) return fail(MLA_ERR_ARG, "dsa_topk: NULL pointer");
  for (int b = 0; b < batch; ++b) {
    if (row_len[b] < 1 || row_len[b] > (1 << 30))
      return fail(MLA_ERR_SHAPE, "dsa_topk: row_len[%d] = %d outside [1, 2^30]", b, row_len[b]);
    if (batch > 1 && row_len[b] > score_stride)
      return fail(MLA_ERR_SHAPE, "dsa_topk: row_len[%d] = %d exceeds the score row stride %lld", b, row_len[b],
                  static_cast<long long>(score_stride));
    if (row_len[b] > top_k) *total += top_k;
    if (mla::dsa_topk_two_stage(row_len[b], top_k)) ++*two_stage;
  }
  if (*total > 0x7fffffffLL) return fail(MLA_ERR_UNSUPPORTED, "dsa_topk: more than 2^31-1 selected indices");
  return ok();
}

// Writes sel_count and launches the selection; ws == NULL runs every row on
// one workgroup, otherwise the two-stage rows use ws (kTopkRowWsBytes each).
int topk_launch(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len, int32_t top_k,
                int32_t* sel_idx, int32_t* sel_count, char* ws, hipStream_t stream) {
  for (int b = 0; b < batch; ++b) sel_count[b] = row_len[b] > top_k ? top_k : -1;
  mla::TopkParams one{}, two{};
  one.scores = two.scores = scores;
  one.stride = two.stride = score_stride;
  one.sel_idx = two.sel_idx = sel_idx;
  one.top_k = two.top_k = top_k;
  two.ws = ws;
  int64_t off = 0;
  for (int b = 0; b < batch; ++b) {
    if (row_len[b] <= top_k) continue;
    mla::TopkParams& p = ws && mla::dsa_topk_two_stage(row_len[b], top_k) ? two : one;
    p.row[p.rows] = b;
    p.len[p.rows] = row_len[b];
    p.out_off[p.rows] = static_cast<int32_t>(off);
    off += top_k;
    if (++p.rows == mla::kTopkRowsPerLaunch) {
      hipError_t e = &p == &two ? mla::launch_dsa_topk_two_stage(p, stream) : mla::launch_dsa_topk(p, stream);
      if (e != hipSuccess) return device(e, "dsa_topk launch");
      if (&p == &two) two.ws += static_cast<size_t>(mla::kTopkRowsPerLaunch) * mla::kTopkRowWsBytes;
      p.rows = 0;
    }
  }
  hipError_t e = mla::launch_dsa_topk(one, stream);
  if (e != hipSuccess) return device(e, "dsa_topk launch");
  e = mla::launch_dsa_topk_two_stage(two, stream);
  if (e != hipSuccess) return device(e, "dsa_topk launch");
  return ok();
}

}  // namespace

extern "C" {

int mla_dsa_topk_select(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len,
                        int32_t top_k, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                        size_t* workspace_bytes, hipStream_t stream) {
  int64_t total = 0, two_stage = 0;
  int rc = topk_check(scores, score_stride, batch, row_len, top_k, sel_count, &total, &two_stage);
  if (rc != MLA_OK) return rc;
  if (batch == 0) {
    if (workspace_bytes && !workspace) *workspace_bytes = 0;
    return ok();
  }
  // without a workspace every row runs on one workgroup
  const bool use_ws = workspace_bytes != nullptr;
  const size_t need = use_ws ? static_cast<size_t>(two_stage) * mla::kTopkRowWsBytes : 0;
  if (use_ws && !workspace) {
    *workspace_bytes = need;
    return ok();
  }
  if (use_ws && *workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "dsa_topk: workspace %zu bytes < %zu required", *workspace_bytes, need);
  if (use_ws && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MLA_ERR_WORKSPACE, "dsa_topk: workspace not 256-byte aligned");
  if (total > 0 && !sel_idx) return fail(MLA_ERR_ARG, "dsa_topk: sel_idx is NULL but rows are selected");
  return topk_launch(scores, score_stride, batch, row_len, top_k, sel_idx, sel_count,
                     use_ws ? static_cast<char*>(workspace) : nullptr, stream);
}

int mla_dsa_topk_select_noalloc(const float* scores, int64_t score_stride, int32_t batch, const int32_t* row_len,
                                int32_t top_k, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream) {
  int64_t total = 0, two_stage = 0;
  int rc = topk_check(scores, score_stride, batch, row_len, top_k, sel_count, &total, &two_stage);
  if (rc != MLA_OK) return rc;
  if (two_stage > mla::kTopkNoAllocRows)
    return fail(MLA_ERR_WORKSPACE,
                "dsa_topk_noalloc: %lld rows take the two-stage form; the fixed scratch holds %d (split the batch)",
                static_cast<long long>(two_stage), mla::kTopkNoAllocRows);
  if (batch == 0) return ok();
  if (total > 0 && !sel_idx) return fail(MLA_ERR_ARG, "dsa_topk: sel_idx is NULL but rows are selected");
  char* ws = nullptr;
  if (two_stage > 0) {
    hipError_t e = mla::dsa_topk_scratch(&ws);
    if (e != hipSuccess) return device(e, "dsa_topk_noalloc scratch");
  }
  // rows that need no scratch run on one workgroup as in mla_dsa_topk_select;
  // with ws == NULL (no two-stage row) that is every row
  return topk_launch(scores, score_stride, batch, row_len, top_k, sel_idx, sel_count, ws, stream);
}

int mla_decode_combine(int32_t part_dtype, const void* part_o, const float* part_lse, int32_t batch, int32_t heads,
                       int32_t kv_lora_rank, int32_t s_max, const int32_t* n_splits, float* o_lat, float* lse,
                       hipStream_t stream) {
  if (!valid_dtype(part_dtype)) return fail(MLA_ERR_ARG, "combine: unknown part_dtype %d", part_dtype);
  if (batch < 0 || heads < 1 || kv_lora_rank < 1 || s_max < 1)
    return fail(MLA_ERR_ARG, "combine: batch >= 0 and positive heads, kv_lora_rank, s_max required");
  if (batch == 0) return ok();
  if (!part_o || !part_lse || !n_splits || !o_lat) return fail(MLA_ERR_ARG, "combine: NULL pointer");
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "combine: heads > 65535");
  for (int b = 0; b < batch; ++b)
    if (n_splits[b] < 1 || n_splits[b] > s_max)
      return fail(MLA_ERR_SHAPE, "combine: n_splits[%d] = %d outside [1, %d]", b, n_splits[b], s_max);
  mla::CombineParams p{};
  p.heads = heads;
  p.r = kv_lora_rank;
  p.s_max = s_max;
  p.part_bf16 = part_dtype == MLA_DTYPE_BF16;
  for (int b0 = 0; b0 < batch; b0 += mla::kCombineRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kCombineRowsPerLaunch);
    for (int i = 0; i < p.rows; ++i) p.n_splits[i] = n_splits[b0 + i];
    const int64_t bh = static_cast<int64_t>(b0) * heads;
    p.part_o = advance(part_o, bh * s_max * kv_lora_rank, part_dtype);
    p.part_lse = part_lse + bh * s_max;
    p.o_lat = o_lat + bh * kv_lora_rank;
    p.lse = lse ? lse + bh : nullptr;
    hipError_t e = mla::launch_combine(p, stream);
    if (e != hipSuccess) return device(e, "combine launch");
  }
  return ok();
}

int mla_decode_combine_v(int32_t dtype, int32_t part_dtype, const void* part_o, const float* part_lse, int32_t batch,
                         int32_t heads,
                         int32_t kv_lora_rank, int32_t s_max, const int32_t* n_splits, const void* w_kv_b,
                         int32_t qk_nope, int32_t v_head, float* ctx, float* o_lat, float* lse, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "combine_v: unknown dtype %d", dtype);
  if (!valid_dtype(part_dtype)) return fail(MLA_ERR_ARG, "combine_v: unknown part_dtype %d", part_dtype);
  if (batch < 0 || heads < 1 || kv_lora_rank < 1 || s_max < 1 || qk_nope < 1 || v_head < 1)
    return fail(MLA_ERR_ARG,
                "combine_v: batch >= 0 and positive heads, kv_lora_rank, s_max, qk_nope, v_head required");
  if (kv_lora_rank > 1024) return fail(MLA_ERR_UNSUPPORTED, "combine_v: kv_lora_rank <= 1024 supported");
  if (batch == 0) return ok();
  if (!part_o || !part_lse || !n_splits || !w_kv_b || !ctx) return fail(MLA_ERR_ARG, "combine_v: NULL pointer");
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "combine_v: heads > 65535");
  for (int b = 0; b < batch; ++b)
    if (n_splits[b] < 1 || n_splits[b] > s_max)
      return fail(MLA_ERR_SHAPE, "combine_v: n_splits[%d] = %d outside [1, %d]", b, n_splits[b], s_max);
  mla::CombineParams p{};
  p.heads = heads;
  p.r = kv_lora_rank;
  p.s_max = s_max;
  p.w = w_kv_b;
  p.w_dtype = dtype;
  p.part_bf16 = part_dtype == MLA_DTYPE_BF16;
  p.dn = qk_nope;
  p.dv = v_head;
  for (int b0 = 0; b0 < batch; b0 += mla::kCombineRowsPerLaunch) {
    p.rows = std::min(batch - b0, mla::kCombineRowsPerLaunch);
    for (int i = 0; i < p.rows; ++i) p.n_splits[i] = n_splits[b0 + i];
    const int64_t bh = static_cast<int64_t>(b0) * heads;
    p.part_o = advance(part_o, bh * s_max * kv_lora_rank, part_dtype);
    p.part_lse = part_lse + bh * s_max;
    p.o_lat = o_lat ? o_lat + bh * kv_lora_rank : nullptr;
    p.lse = lse ? lse + bh : nullptr;
    p.ctx = ctx + bh * v_head;
    hipError_t e = mla::launch_combine(p, stream);
    if (e != hipSuccess) return device(e, "combine_v launch");
  }
  return ok();
}

int mla_prefill_reconstructed(int32_t dtype, int32_t batch, int32_t tokens, int32_t keys, int32_t heads,
                              int32_t q_lora_rank, int32_t kv_lora_rank, int32_t qk_nope, int32_t qk_rope,
                              int32_t v_head, const void* q_c, const void* w_q_b, const void* latent,
                              const void* rope, const void* w_kv_b, const int64_t* q_offsets, double theta,
                              const int32_t* left_pad, float softmax_scale, void* workspace, size_t* workspace_bytes,
                              float* ctx, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(MLA_ERR_ARG, "prefill: unknown dtype %d", dtype);
  if (batch < 0 || tokens < 1 || keys < 1 || heads < 1 || q_lora_rank < 1 || kv_lora_rank < 1 || qk_nope < 1 ||
      qk_rope < 1 || v_head < 1)
    return fail(MLA_ERR_ARG, "prefill: batch >= 0 and positive geometry required");
  if (keys < tokens) return fail(MLA_ERR_SHAPE, "prefill: keys=%d < tokens=%d (the keys include the query block)", keys, tokens);
  if (qk_rope & 1) return fail(MLA_ERR_ROPE, "prefill: qk_rope=%d, need an even count", qk_rope);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ROPE, "prefill: theta=%g, need finite > 0", theta);
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_ARG, "prefill: softmax_scale must be finite");
  if (qk_nope + qk_rope > 256 || v_head > 256 || qk_rope > 2 * mla::kRopeMaxPairs)
    return fail(MLA_ERR_UNSUPPORTED, "prefill: qk_nope + qk_rope <= 256 and v_head <= 256 supported");
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "prefill: heads > 65535");
  if (!workspace_bytes) return fail(MLA_ERR_ARG, "prefill: workspace_bytes is NULL");
  mla::PrefillParams p{};
  p.dtype = dtype;
  p.batch = batch;
  p.tokens = tokens;
  p.keys = keys;
  p.heads = heads;
  p.ql = q_lora_rank;
  p.r = kv_lora_rank;
  p.dn = qk_nope;
  p.dr = qk_rope;
  p.dv = v_head;
  p.q_c = q_c;
  p.w_qb = w_q_b;
  p.latent = latent;
  p.rope = rope;
  p.w_kvb = w_kv_b;
  p.q_offsets = q_offsets;
  p.left_pad = left_pad;
  p.theta = theta;
  p.scale = softmax_scale;
  p.ctx = ctx;
  if (!workspace) {
    *workspace_bytes = mla::prefill_workspace_bytes_any_path(p);
    return ok();
  }
  const size_t need = mla::prefill_workspace_bytes(p);
  if (*workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "prefill: workspace %zu bytes < %zu required", *workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(MLA_ERR_WORKSPACE, "prefill: workspace not 256-byte aligned");
  if (batch == 0) return ok();
  if (!q_c || !w_q_b || !latent || !rope || !w_kv_b || !q_offsets || !ctx)
    return fail(MLA_ERR_ARG, "prefill: NULL pointer");
  for (int b = 0; b < batch; ++b) {
    if (q_offsets[b] < 0) return fail(MLA_ERR_ROPE, "prefill: q_offsets[%d] < 0", b);
    if (static_cast<double>(q_offsets[b]) + tokens > kMaxPosition)
      return fail(MLA_ERR_UNSUPPORTED, "prefill: offset + tokens exceeds 2^53");
    if (left_pad && (left_pad[b] < 0 || left_pad[b] > keys))
      return fail(MLA_ERR_SHAPE, "prefill: left_pad[%d] = %d outside [0, %d]", b, left_pad[b], keys);
  }
  p.workspace = workspace;
  return device(mla::launch_prefill(p, stream), "prefill launch");
}

}  // extern "C"
