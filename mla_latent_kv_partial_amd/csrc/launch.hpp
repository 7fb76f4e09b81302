// Internal launch interface between the C ABI layer (mla_abi.cpp) and the
// kernel translation units.  Arguments here are already validated; every
// launcher only enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Per-launch row tables travel in the kernel argument block, so a launch
// covers at most this many rows; the host splits larger batches.
constexpr int kRopeRowsPerLaunch = 128;
constexpr int kRopeMaxPairs = 256;           // rotary_dims <= 512
constexpr int kDecodeRowsPerLaunch = 128;
constexpr int kCombineRowsPerLaunch = 256;

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

// ------------------------------------------------------------------ RoPE
struct RopeParams {
  const void* x;
  void* y;
  int32_t rows;          // batch rows in this launch
  int32_t tokens, inner, feat;
  int64_t sb, st, si;    // element strides (x and y)
  int32_t rotary;        // rotary dims R
  int32_t per_row;       // 1: off[b] per row, 0: off[0] for all rows
  int32_t copy_tail;     // y != x
  int64_t off[kRopeRowsPerLaunch];
  float inv[kRopeMaxPairs];
};
hipError_t launch_rope(int32_t dtype, const RopeParams& p, hipStream_t stream);

// ------------------------------------------------------------------ absorb
struct AbsorbQParams {
  const void* q;          // [B,H,dn] strided
  int64_t q_sb, q_sh;
  const void* w;          // [H*(dn+dv), r]
  void* q_lat;            // [B,H,r] of the dtype
  int32_t batch, heads, dn, dv, r;
};
hipError_t launch_absorb_q(int32_t dtype, const AbsorbQParams& p, hipStream_t stream);
// absorb_q of p and the RoPE of rp (rows of rp = rows of p) in one launch where
// the MFMA absorb applies, else the two launches in order.
hipError_t launch_absorb_q_rope(int32_t dtype, const AbsorbQParams& p, const RopeParams& rp, hipStream_t stream);

struct AbsorbVParams {
  const float* o_lat;     // [B,H,r]
  const void* w;          // [H*(dn+dv), r]
  float* ctx;             // [B,H*dv]
  int32_t batch, heads, dn, dv, r;
};
hipError_t launch_absorb_v(int32_t dtype, const AbsorbVParams& p, hipStream_t stream);

// ------------------------------------------------------------------ decode
struct DecodeRows {
  int32_t kv_len[kDecodeRowsPerLaunch];
  int32_t n_att[kDecodeRowsPerLaunch];   // attended count
  int32_t sel_off[kDecodeRowsPerLaunch]; // -1: dense row, else offset into sel
  int32_t split_begin[kDecodeRowsPerLaunch + 1];   // prefix sum of the rows' split counts
};

struct DecodeParams {
  const void* q_lat;      // [rows,H,r] of the dtype (already offset to the first row of the launch)
  const void* q_rope;     // strided
  int64_t qr_sb, qr_sh;
  const void* latent;     // strided, first row of the launch
  int64_t lat_sb, lat_st;
  const void* rope;
  int64_t rope_sb, rope_st;
  const int32_t* sel;     // selection base (may be null)
  void* part_o;           // [rows,H,s_max,r] fp32, or bf16 when part_bf16
  float* part_lse;        // [rows,H,s_max]
  int32_t* dev_err;
  int32_t rows, heads, r, dr, width;
  int32_t chunk, s_max, s_launch;        // s_launch = max splits over the launch rows
  int32_t s_total;                       // splits of all launch rows (= split_begin[rows])
  int32_t q_copy;                        // queries may be copied HBM -> LDS (16-byte aligned q_rope rows)
  int32_t part_bf16;                     // partials stored as bf16 (round to nearest even)
  float scale;
  DecodeRows tab;
};
hipError_t launch_decode(int32_t dtype, const DecodeParams& p, hipStream_t stream);
// Streaming probe of the attention's copy path (packed bf16 cache, dense rows).
hipError_t launch_stream_probe(const DecodeParams& p, hipStream_t stream);

// ------------------------------------------------------------------ combine
struct CombineParams {
  const void* part_o;     // fp32, or bf16 when part_bf16
  const float* part_lse;
  float* o_lat;           // may be null when ctx is set
  float* lse;             // may be null
  int32_t rows, heads, r, s_max;
  int32_t part_bf16;
  // value projection after the merge (ctx = o_lat . W_UV^T), when ctx is set
  const void* w;          // [H*(dn+dv), r] of w_dtype
  float* ctx;             // [rows, H*dv]
  int32_t w_dtype, dn, dv;
  int32_t n_splits[kCombineRowsPerLaunch];
};
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

// ------------------------------------------------------------------ cache append
struct AppendParams {
  const void* kv_a;       // [rows, T, r + dr] strided (element strides kb, kt)
  int64_t kb, kt;
  const void* w;          // [r] RMSNorm weight
  void* latent;           // cache, element strides lb, lt
  int64_t lb, lt;
  void* rope;
  int64_t rb, rt;
  int32_t rows, tokens, r, dr, slot;
  float eps;
  int64_t off[kRopeRowsPerLaunch];   // RoPE position of token 0, per row
  float inv[kRopeMaxPairs];
};
hipError_t launch_append(int32_t dtype, const AppendParams& p, hipStream_t stream);

// ------------------------------------------------------------------ DSA top-k
constexpr int kTopkRowsPerLaunch = 128;

struct TopkParams {
  const float* scores;    // row b at scores + b * stride
  int64_t stride;
  int32_t* sel_idx;       // concatenated output
  int32_t rows;           // selected rows in this launch
  int32_t top_k;
  int32_t row[kTopkRowsPerLaunch];
  int32_t len[kTopkRowsPerLaunch];
  int32_t out_off[kTopkRowsPerLaunch];
  // two-stage rows: survivor area of launch row i at ws + i * kTopkRowWsBytes
  char* ws;
};
// Rows of at most kTopkSeg scores, or longer than kTopkSeg * kTopkMaxSegs, or
// with top_k above kTopkMaxCand / (their kTopkSeg segments), run on one
// workgroup (launch_dsa_topk); the others ("two-stage" rows) in three
// launches over 8192-score segments (launch_dsa_topk_two_stage), with
// kTopkRowWsBytes of workspace each.
constexpr int kTopkSeg = 16384;
constexpr int kTopkMaxSegs = 8;
constexpr int kTopkMaxCand = 16384;
constexpr size_t kTopkRowWsBytes = static_cast<size_t>(kTopkMaxCand) * 8 + 256;
bool dsa_topk_two_stage(int64_t n, int32_t top_k);
hipError_t launch_dsa_topk(const TopkParams& p, hipStream_t stream);
hipError_t launch_dsa_topk_two_stage(const TopkParams& p, hipStream_t stream);
// Fixed device scratch of mla_dsa_topk_select_noalloc: kTopkNoAllocRows
// two-stage rows.  *ptr = its address on the current device (looked up once
// per device).
constexpr int kTopkNoAllocRows = 32;
hipError_t dsa_topk_scratch(char** ptr);

// ------------------------------------------------------------------ GEMM (MFMA, bf16 operands)
constexpr int kGemmRowsPerLaunch = 128;

// C[m, n] = sum_k A[m, k] B[n, k], both operands bf16 and K-contiguous.
struct GemmNT {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  void* c;                // bf16 or fp32, row stride ldc
  int64_t ldc;
  int32_t m, n, k;
  int32_t m_tiles, n_tiles;   // filled by the launcher
  // RoPE epilogue (q projection, heads of 128 no-PE + 64 rope columns): row m
  // is token m % tokens of batch row m / tokens, rotated at off[row] + token.
  int32_t tokens;
  int64_t off[kGemmRowsPerLaunch];
  float inv[32];
  // RoPE epilogue: {cos, sin} of the angle of GEMM row m and pair q at
  // cs[32 m + q], written by launch_rope_table for the same rows
  const float2* cs;
};
// cs[32 m + q] for m < p.m, q < 32 (the 64-wide rope part): cos and sin of
// the f32 angle (position of row m) * inv[q], taken in double and rounded to
// f32.
hipError_t launch_rope_table(const GemmNT& p, float2* cs, hipStream_t stream);
bool gemm_nt_mfma_ok(const void* a, int64_t lda, const void* b, int64_t ldb, const void* c, int64_t ldc, int64_t m,
                     int64_t n, int64_t k);
hipError_t launch_gemm_nt_mfma(const GemmNT& p, bool rope, bool out_f32, hipStream_t stream);
// x (fp32, 16-byte aligned) -> y (bf16), round to nearest even.
hipError_t launch_f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream);

// ------------------------------------------------------------------ prefill
struct PrefillParams {
  int32_t dtype;
  int32_t batch, tokens, keys, heads, ql, r, dn, dr, dv;
  const void* q_c;
  const void* w_qb;
  const void* latent;
  const void* rope;
  const void* w_kvb;
  const int64_t* q_offsets;   // host
  const int32_t* left_pad;    // host (nullable)
  double theta;
  float scale;
  void* workspace;
  float* ctx;
};
size_t prefill_workspace_bytes(const PrefillParams& p);            // of the path these buffers take
size_t prefill_workspace_bytes_any_path(const PrefillParams& p);   // enough for either path
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Inverse-frequency table of partial interleaved RoPE, built on the host in
// double exactly as the page builds it (see mla_abi.cpp).
void rope_inverse_frequencies(int32_t rotary, double theta, float* out);

}  // namespace mla
