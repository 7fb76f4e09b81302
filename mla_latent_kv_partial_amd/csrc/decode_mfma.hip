// MFMA latent decode attention for the bf16 GLM geometry: kv_lora_rank 512,
// rope 64, heads a multiple of 16.  Computes the split-T partials of the
// page's absorbed decode (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// Glm52Mla.attendAbsorbed: scores = scale * (q_lat . latent + q_rope . rope),
// softmax over the attended tokens, latent context = P . latent), including
// its DSA gather and the ragged right-aligned rows of Glm52Mla.forward.
//
// One workgroup serves one (row, split) for up to 64 heads, so the cache is
// read once for all heads.  The workgroup has two kinds of waves, two per SIMD:
//   * score waves (w < NW, heads 16w..16w+15) hold Q in registers, compute
//     S^T[token, head] = K . Q^T on v_mfma_f32_16x16x32_bf16 from K fragments
//     read by ds_read_b128, run the online softmax in fp32 / exp2 (each lane
//     owns one head) and hand P (bf16, already in MFMA operand layout) and the
//     rescale factors to the context waves through LDS;
//   * context waves (w >= NW) hold the fp32 context accumulators and, one tile
//     behind, compute O^T[dim, head] += V^T . P^T with V^T fragments read from
//     the token-major tile by ds_read_b64_tr_b16.  Context wave c owns the
//     latent dims [512c/NW, 512(c+1)/NW) for all heads of the workgroup, so
//     each V^T fragment is read from LDS once and feeds NW MFMAs (LDS read
//     bandwidth, not HBM, is the per-CU limit of this loop).
// Splitting the two halves keeps each wave under 256 registers, so two waves
// share each SIMD and hide each other's LDS and MFMA latencies.
//
// HBM -> LDS: 32-token tiles stream through a 4-stage LDS ring by
// global_load_lds_dwordx4 (each lane moves 16 bytes; non-temporal for dense rows), two tiles ahead of the
// score waves; with 64 heads the context waves issue the copies.  A token occupies one 1184-byte LDS row: latent (1024 B), rope
// (128 B), 32 B of padding.  A gathered row uses the same copies with
// per-token addresses, so a gather and a dense read of the same tokens are
// bit-identical.  The running max of a head only moves when a tile exceeds it
// by more than 2^8, so accumulator rescales are rare.
//
// Bank layout (measured with the LDS bank-conflict counter on gfx950): the
// 16-byte fragment reads of 16 rows are conflict-free when the row stride is
// an odd multiple of 32 bytes (1184 = 37 x 32), and the transposing reads are
// conflict-free when score row m of a 16-token block holds token sigma(m)
// below.  Every LDS read address is a per-lane base plus an immediate.
#include <math.h>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kR = 512;
constexpr int kDR = 64;
constexpr int kNT = 32;                    // tokens per tile
constexpr int kRowChunks = 74;             // 16-byte chunks per token row (64 latent, 8 rope, 2 pad)
constexpr int kRowBytes = kRowChunks * 16;
constexpr int kDmaPerTile = (kNT * kRowChunks + 63) / 64;   // 37 copies of 1 KB
constexpr int kTileBytes = kDmaPerTile * 1024;              // rows + tail of the last copy
constexpr int kStageBytes = kTileBytes + kNT * 4;           // + the tile's selection indices
constexpr int kStages = 4;
constexpr int kQSteps = kR / 32 + kDR / 32;                 // 18 k-steps of the scores
constexpr int kDimBlocks = kR / 16;                         // 32 output blocks of 16 dims
constexpr float kRescaleSlack = 8.f;                        // log2 units
constexpr int kMaxHeadGroups = 4;                           // 16-head groups per workgroup
constexpr int kQOffset = 2 * kStageBytes;                   // queries copied to LDS: stages 2 and 3
constexpr int kQRowBytes = kR * 2 + 32;                     // an odd number of 32-byte units per head row
static_assert(kQOffset + 64 * kQRowBytes + 64 * kDR * 2 <= kStages * kStageBytes,
              "the queries of a 64-head group must fit stages 2 and 3");
static_assert(kStages * kStageBytes >= kMaxHeadGroups * (16 * kMaxHeadGroups) * (kR * 4 / kMaxHeadGroups + 32),
              "the epilogue regions of the context waves must fit in the stage ring");

__shared__ __attribute__((aligned(1024))) char g_stage[kStages * kStageBytes];
__shared__ __attribute__((aligned(16))) char g_p[2][kMaxHeadGroups][kWave * 16];   // P operands, by tile parity
__shared__ float g_alpha[2][kMaxHeadGroups][16];                                     // rescale factor per head
__shared__ int g_moved[2][kMaxHeadGroups];                                           // any rescale in the wave
__shared__ float g_inv[kMaxHeadGroups][16];                                          // 1 / softmax denominator

// Max over lanes i, i ^ 16, i ^ 32 and i ^ 48 by v_permlane16_swap and
// v_permlane32_swap (VALU; a lane shuffle through ds_bpermute waits on LDS).
// With both operands x, the 16-lane-row swap returns rows (0, 0, 2, 2) and
// (1, 1, 3, 3) of x, the 32-lane swap the halves (lo, lo) and (hi, hi).
__device__ __forceinline__ float max_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Token held by score row m of a 16-token block.
__device__ __forceinline__ int sigma(int m) {
  return 2 * (m & 3) + ((m >> 2) & 1) + 8 * ((m >> 3) & 1);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// NW head groups of 16 per workgroup (2 NW waves).  PACKED: rope = latent + 512
// elements with the same strides (one [B, W, 576] cache) and every row offset
// below 2^32: copies use an SGPR base plus a 32-bit lane offset; otherwise
// each lane forms a 64-bit address.
template <int NW, bool GATHER, bool PACKED>
struct Decode {
  static constexpr int kWaves = 2 * NW;
  // Copy-issuing waves.  With 64 heads only the context waves issue the tile
  // copies: a copy instruction holds its wave until the CU's address path
  // takes it (about 16 cycles per 1 KB copy), so issuing a tile stalls the
  // issuing waves for several hundred cycles, and the score waves, whose
  // scores and softmax are the loop's critical path, start their MFMAs right
  // after the barrier instead.  With 16 or 32 heads every wave issues (fewer
  // waves, and a single context wave would hold all 37 copies in registers).
  static constexpr int kIssuers = NW == 4 ? NW : kWaves;
  static constexpr int kFirstIssuer = NW == 4 ? NW : 0;
  // Issuing wave kFirstIssuer + v issues tile copies n = v, v + kIssuers, ...
  // below kDmaPerTile: kMaxDma or kMaxDma - 1 of them; the others none.
  static constexpr int kMaxDma = (kDmaPerTile + kIssuers - 1) / kIssuers;
  // Context waves: dim blocks per wave; reg[db * NW + hb] holds dims
  // 16 (c kCtxBlocks + db) + 4 g + (0..3) of head 16 hb + h.
  static constexpr int kCtxBlocks = kDimBlocks / NW;

  const DecodeParams& p;
  int lane, wave, hw, h, g, head, head0;   // hw: head group (score) / dim slice (context)
  bool scorer;
  int n_tok, nt, len, pad, sel_base, n_dma;
  bool gather_row;              // this row reads its tokens through the selection list
  bool bad_index;               // an out-of-range selection index was seen (flagged at the end)
  const char* lat_base;
  const char* rope_base;
  int64_t lat_st, rope_st;      // bytes
  float scale_log2;
  int dma_src[kMaxDma];         // bpermute address (4 x token row) of this lane's chunk in copy i
  int dma_off[kMaxDma];         // byte offset of the chunk in its latent row, or rope row (sign bit set)
  uint32_t qk_base, tr_base;    // per-lane LDS byte offsets of the fragment reads within a stage
  // Score waves: reg[0..17] hold the Q operands (bf16 bits).  Context waves:
  // the O^T accumulators (see kCtxBlocks).
  f32x4 reg[kDimBlocks];
  float m_run, l_run;
  uint32_t mask0, mask1, mask2;  // validity of tiles i, i+1, i+2 (bit t: token t)

  __device__ __forceinline__ Decode(const DecodeParams& prm) : p(prm) {}

  // Row slot and validity of tile token `lane` (lanes < 32) from its index
  // into the valid slice.  Only the score waves use the validity mask and
  // flag out-of-range indices.
  template <bool SC>
  __device__ __forceinline__ int slot_of(int tile, int idx, uint32_t& m) {
    const bool in = lane < kNT && tile * kNT + lane < n_tok;
    const bool ok = in && idx >= 0 && idx < len;
    if (SC) {
      bad_index |= in && !ok;
      m = static_cast<uint32_t>(__ballot(ok));
    }
    return ok ? pad + idx : p.width - 1;   // masked tokens read a valid row, weighted by zero
  }

  __device__ __forceinline__ static char* stage(int s) { return g_stage + s * kStageBytes; }
  __device__ __forceinline__ static int* idx_area(int s) { return reinterpret_cast<int*>(stage(s) + kTileBytes); }

  // row_v: lane t < 32 holds token t's row, as a byte offset from lat_base
  // (PACKED) or as a row slot.
  __device__ __forceinline__ void copy(int i, int row_v, uint32_t dst) const {
    int src4, off;
    plan(i, src4, off);
    const int v = __builtin_amdgcn_ds_bpermute(src4, row_v);
    if (PACKED) {
      dma16_off(lat_base, static_cast<uint32_t>(v) + static_cast<uint32_t>(off), dst + block(i) * 1024);
    } else {
      const char* src = off >= 0 ? lat_base + v * lat_st + off : rope_base + v * rope_st + (off & 0x7fff);
      dma16(src, dst + block(i) * 1024);
    }
  }

  // LDS block (1 KB) of this wave's copy i within a stage.
  __device__ __forceinline__ int block(int i) const { return wave - kFirstIssuer + kIssuers * i; }

  // Copy plan (the same for every tile): copy i of an issuing wave moves
  // stage chunk k = 64 block(i) + lane, which is chunk c of token row k / 74
  // (c < 64 latent, c < 72 rope, 72 and 73 padding).  src4 = 4 x the token
  // row (a bpermute address); off = the chunk's byte offset in the packed row,
  // or in the latent row, or in the rope row with the sign bit set.  The plan
  // stays in registers, except in the 64-head separate-array form, whose
  // issuing (context) waves also hold 64-bit addresses: it recomputes the plan,
  // which keeps them unspilled.
  __device__ __forceinline__ void plan_of(int i, int& src4, int& off) const {
    const int k = 64 * block(i) + lane;
    int row = k / kRowChunks;
    const int c = k - row * kRowChunks;
    row = min(row, kNT - 1);   // the tail of the last copy lands past the rows; it reads a valid token
    src4 = 4 * row;
    if (PACKED)
      off = c < 72 ? c * 16 : 0;   // rope follows the latent in the packed row
    else
      off = c < 64 ? c * 16 : (c < 72 ? static_cast<int>(0x80000000u | static_cast<uint32_t>((c - 64) * 16)) : 0);
  }
  static constexpr bool kPlanInRegs = PACKED || NW < 4;
  __device__ __forceinline__ void plan(int i, int& src4, int& off) const {
    if (kPlanInRegs) {
      src4 = dma_src[i];
      off = dma_off[i];
    } else {
      plan_of(i, src4, off);
    }
  }

  // Dense rows: row r of tile `tile` is slot pad + sel_base + 32 tile + r while
  // inside the split; past its end the copy reads the valid slot width - 1
  // (those tokens are masked).  No lane exchange needed.  These copies carry
  // the non-temporal hint (the row streams once per pass; per ragged layer
  // 37.6 -> 34.9 us); gathered rows keep the default policy, with which they
  // measured faster (stacked 64-selection launch 45.5 against 51 us).
  __device__ __forceinline__ void issue_tile_dense(int s, int tile) const {
    if (n_dma == 0) return;   // not an issuing wave (wave-uniform)
    const uint32_t dst = lds_addr(stage(s));
    const int first = tile * kNT;
    const int base = pad + sel_base + first;
#pragma unroll
    for (int i = 0; i < kMaxDma; ++i) {
      if (i == kMaxDma - 1 && n_dma != kMaxDma) break;
      int src4, off;
      plan(i, src4, off);
      const int r = src4 >> 2;
      const int slot = first + r < n_tok ? base + r : p.width - 1;
      if (PACKED) {
        dma16_off_nt(lat_base, static_cast<uint32_t>(slot) * static_cast<uint32_t>(lat_st) + static_cast<uint32_t>(off),
                  dst + block(i) * 1024);
      } else {
        const char* src = off >= 0 ? lat_base + slot * lat_st + off : rope_base + slot * rope_st + (off & 0x7fff);
        dma16_nt(src, dst + block(i) * 1024);
      }
    }
  }

  // Validity of the tokens of tile `tile` of a dense row (bit t: token t).
  __device__ __forceinline__ uint32_t dense_mask(int tile) const {
    const int cnt = n_tok - tile * kNT;
    return cnt >= kNT ? 0xffffffffu : (cnt <= 0 ? 0u : (1u << cnt) - 1u);
  }

  // Copy one tile into stage s.  slot_v: lane t < 32 holds token t's row slot.
  __device__ __forceinline__ void issue_tile(int s, int slot_v) const {
    if (n_dma == 0) return;   // not an issuing wave (wave-uniform)
    const uint32_t dst = lds_addr(stage(s));
    const int row_v = PACKED ? static_cast<int>(static_cast<uint32_t>(slot_v) * static_cast<uint32_t>(lat_st)) : slot_v;
#pragma unroll
    for (int i = 0; i < kMaxDma - 1; ++i) copy(i, row_v, dst);   // every issuing wave has these
    if (n_dma == kMaxDma) copy(kMaxDma - 1, row_v, dst);
  }

  // Gathered rows: copy the 32 selection indices of a tile (clamped inside the
  // row's list) into the index area of stage s.  The first issuing wave only
  // (its tile-copy waits cover these copies, see ops_after).
  __device__ __forceinline__ void issue_idx(int s, int tile) const {
    if (gather_row && wave == kFirstIssuer && lane < kNT) {
      const int j = min(tile * kNT + lane, n_tok - 1);
      dma4(p.sel + sel_base + j, lds_addr(idx_area(s)));
    }
  }

  // Vector-memory operations this wave issued after the copies of tile i, in
  // the issue order of pipeline() (prologue: C0 C1, then step j issues
  // C(j+2); C = the n_dma copies of a tile).  Index copies of gathered rows
  // are not counted, which only makes a wait stronger.
  __device__ __forceinline__ int ops_after(int i) const { return i == 0 || i + 1 < nt ? n_dma : 0; }

  // Score wave, tile i in stage s: scores, softmax, P and rescale factors out.
  __device__ __forceinline__ void score(int s, int parity, uint32_t valid) {
    const char* st = stage(s);
    // two 16-token blocks, each over two accumulators (even / odd k-steps)
    f32x4 acc[4] = {};
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const int off = ks < kR / 32 ? ks * 64 : kR * 2 + (ks - kR / 32) * 64;
      const bf16x8 q = __builtin_bit_cast(bf16x8, reg[ks]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + qk_base + tb * 16 * kRowBytes + off);
        acc[2 * tb + (ks & 1)] = mfma(a, q, acc[2 * tb + (ks & 1)]);
      }
    }
    // lane owns head h and score rows 4g+i of both blocks: tokens 16tb + sigma(4g+i)
    float x[8];
    if (__builtin_amdgcn_readfirstlane(valid) == 0xffffffffu) {
      // a whole tile (wave-uniform branch): no mask
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * tb + i] = (acc[2 * tb][i] + acc[2 * tb + 1][i]) * scale_log2;
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tb + sigma(4 * g + i);
          const float sc = acc[2 * tb][i] + acc[2 * tb + 1][i];
          x[4 * tb + i] = ((valid >> t) & 1u) ? sc * scale_log2 : -INFINITY;
        }
    }
    float mt = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mt = fmaxf(mt, x[k]);
    mt = max_lanes_xor16_32(mt);
    // Move the reference max only when this tile exceeds it by the slack (the
    // first valid tile always moves it from -inf).
    const bool move = mt > m_run + kRescaleSlack;
    const bool any_move = __any(move);
    float alpha = 1.f;
    if (move) {
      alpha = __builtin_amdgcn_exp2f(m_run - mt);
      m_run = mt;
    }
    l_run *= alpha;
    // m_run still -inf: every x of the head is -inf, and exp2(-inf - 0) = 0
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pb;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float pr = __builtin_amdgcn_exp2f(x[k] - m_use);
      l_run += pr;
      pb[k] = static_cast<__bf16>(pr);
    }
    *reinterpret_cast<bf16x8*>(&g_p[parity][hw][lane * 16]) = pb;
    if (any_move) {
      if (g == 0) g_alpha[parity][hw][h] = alpha;
    }
    if (lane == 0) g_moved[parity][hw] = any_move ? 1 : 0;
  }

  // Context wave, tile i-1 in stage s: rescale if asked, then O^T += V^T . P^T.
  __device__ __forceinline__ void context(int s, int parity) {
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      if (g_moved[parity][hb]) {
        const float alpha = g_alpha[parity][hb][h];
#pragma unroll
        for (int db = 0; db < kCtxBlocks; ++db) reg[db * NW + hb] *= alpha;
      }
    }
    bf16x8 pb[NW];
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) pb[hb] = *reinterpret_cast<const bf16x8*>(&g_p[parity][hb][lane * 16]);
    const char* st = stage(s);
#pragma unroll
    for (int db = 0; db < kCtxBlocks; ++db) {
      lds_s16x4* a1 = (lds_s16x4*)(st + tr_base + db * 32);
      lds_s16x4* a2 = (lds_s16x4*)(st + tr_base + 16 * kRowBytes + db * 32);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a1);
      const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a2);
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) reg[db * NW + hb] = mfma(v, pb[hb], reg[db * NW + hb]);
    }
  }

  // Score waves: the queries (bf16) as MFMA operands in reg[0..17].
  __device__ __forceinline__ void convert_queries(const f32x4* qraw, const short (*qrraw)[8]) {
#pragma unroll
    for (int ks = 0; ks < kR / 32; ++ks) reg[ks] = qraw[ks];
#pragma unroll
    for (int ks = 0; ks < kDR / 32; ++ks) {
      s16x8 q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = qrraw[ks][e];
      reg[kR / 32 + ks] = __builtin_bit_cast(f32x4, q);
    }
  }

  __device__ __forceinline__ void run(int b, int s) {
    // ---- the copy plan (see plan_of)
    const int v = wave - kFirstIssuer;
    n_dma = v < 0 ? 0 : (kDmaPerTile - v + kIssuers - 1) / kIssuers;
    if (kPlanInRegs) {
#pragma unroll
      for (int i = 0; i < kMaxDma; ++i) plan_of(i, dma_src[i], dma_off[i]);
    }
    // ---- per-lane LDS fragment bases
    qk_base = sigma(h) * kRowBytes + g * 16;
    tr_base = sigma(4 * g + (h >> 2)) * kRowBytes + ((h & 3) >> 1) * 16 + (h & 1) * 8 + hw * kCtxBlocks * 32;
    // The two roles run separate copies of the pipeline, so each is register
    // allocated on its own (the score waves never hold the accumulators).
    if (scorer)
      pipeline<true>(b, s);
    else
      pipeline<false>(b, s);
    if (GATHER && bad_index && p.dev_err) atomicOr(p.dev_err, 1);
  }

  template <bool SC>
  __device__ __forceinline__ void pipeline(int b, int s) {
    // ---- prologue.  Issue order for a dense row: the copies of tile 0, the
    // query loads (score waves), the copies of tile 1; converting the queries
    // then waits once for all of them, so the latencies overlap, and the HBM
    // requests of tile 0 leave ahead of the (cache-resident) queries.  A row
    // read through a selection first needs the indices of tiles 0 and 1 to
    // address its copies: it loads the queries first and converts them as
    // soon as those indices are in, which costs no extra latency.
    f32x4 qraw[kR / 32];   // 8 bf16 each
    short qrraw[kDR / 32][8];
    const bool dense_row = !(GATHER && gather_row);
    if (dense_row) issue_tile_dense(0, 0);
    // A launch of dense rows over 64-head groups copies the group's queries
    // HBM -> LDS with the tile copies (coalesced 1 KB rows, counted by the
    // same waits) into stages 2 and 3, which stay free until step 0; the
    // score waves read their fragments there after the first barrier.
    const bool q_copy = !GATHER && NW == 4 && p.q_copy;
    if (q_copy) {
      const uint32_t qdst = lds_addr(g_stage) + kQOffset;
      const char* qsrc = static_cast<const char*>(p.q_lat) + (static_cast<int64_t>(b) * p.heads + head0) * kR * 2;
      for (int j = wave; j < 16 * NW; j += kWaves)
        dma16(qsrc + static_cast<int64_t>(j) * kR * 2 + lane * 16, qdst + j * kQRowBytes);
      const int hr = 8 * wave + (lane >> 3);   // 8 heads' rope parts (128 B each) per copy
      dma16(static_cast<const char*>(p.q_rope) +
                (static_cast<int64_t>(b) * p.qr_sb + static_cast<int64_t>(head0 + hr) * p.qr_sh) * 2 + (lane & 7) * 16,
            qdst + 16 * NW * kQRowBytes + wave * 1024);
    }
    if (SC && !q_copy) {
      const uint16_t* ql = static_cast<const uint16_t*>(p.q_lat) + (static_cast<int64_t>(b) * p.heads + head) * kR;
#pragma unroll
      for (int ks = 0; ks < kR / 32; ++ks) qraw[ks] = *reinterpret_cast<const f32x4*>(ql + 8 * g + 32 * ks);
      const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qr_sb + head * p.qr_sh;
#pragma unroll
      for (int ks = 0; ks < kDR / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qrraw[ks][e] = static_cast<short>(qr[8 * g + 32 * ks + e]);
    }
    // Tile 1 is copied even for single-tile splits (all of its tokens are
    // then masked and read a valid row), which keeps the wait counts fixed.
    if (GATHER && gather_row) {
      const int idx0v = lane < kNT ? p.sel[sel_base + min(lane, n_tok - 1)] : 0;
      const int idx1v = lane < kNT ? p.sel[sel_base + min(kNT + lane, n_tok - 1)] : 0;
      if (SC) convert_queries(qraw, qrraw);
      const int slot0 = slot_of<SC>(0, idx0v, mask0);
      issue_tile(0, slot0);
      if (nt > 2) issue_idx(2, 2);
      const int slot1 = slot_of<SC>(1, idx1v, mask1);
      issue_tile(1, slot1);
    } else {
      issue_tile_dense(1, 1);
      if (SC) {
        mask0 = dense_mask(0);
        mask1 = dense_mask(1);
        if (GATHER) convert_queries(qraw, qrraw);
      }
    }
    if (SC && !GATHER && !q_copy) convert_queries(qraw, qrraw);
    if (!SC) {
#pragma unroll
      for (int db = 0; db < kDimBlocks; ++db) reg[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Materialise the registers ahead of the pipeline's first copy issue
    // (volatile asm statements keep their relative order).
    constexpr int kLive = SC ? kQSteps : kDimBlocks;
#pragma unroll
    for (int k = 0; k < kLive; ++k) asm volatile("" : "+v"(reg[k]));
    m_run = -INFINITY;
    l_run = 0.f;

    // ---- pipeline: step i scores tile i and accumulates the context of tile
    // i - 1; tile i + 2 is requested at its start.
    for (int i = 0; i <= nt; ++i) {
      if (i < nt) wait_vm_upto<kMaxDma>(ops_after(i));
      lds_barrier();
      if (q_copy && i == 0) {
        // the queries landed with tile 0 (issued between tiles 0 and 1); read
        // them before tile 2 reuses their LDS
        if (SC) {
          const char* qb = g_stage + kQOffset + (16 * hw + h) * kQRowBytes + 16 * g;
#pragma unroll
          for (int ks = 0; ks < kR / 32; ++ks) reg[ks] = *reinterpret_cast<const f32x4*>(qb + 64 * ks);
          const char* rb = g_stage + kQOffset + 16 * NW * kQRowBytes + (16 * hw + h) * (kDR * 2) + 16 * g;
#pragma unroll
          for (int ks = 0; ks < kDR / 32; ++ks) reg[kR / 32 + ks] = *reinterpret_cast<const f32x4*>(rb + 64 * ks);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        lds_barrier();
      }
      if (i + 2 < nt) {
        if (GATHER && gather_row) {
          const int idx = lane < kNT ? idx_area((i + 2) % kStages)[lane] : 0;
          if (i + 3 < nt) issue_idx((i + 3) % kStages, i + 3);
          const int slot = slot_of<SC>(i + 2, idx, mask2);
          issue_tile((i + 2) % kStages, slot);
        } else {
          issue_tile_dense((i + 2) % kStages, i + 2);
          if (SC) mask2 = dense_mask(i + 2);
        }
      }
      if (SC) {
        if (i < nt) score(i % kStages, i & 1, mask0);
        mask0 = mask1;
        mask1 = mask2;
      } else if (i >= 1) {
        context((i - 1) % kStages, (i - 1) & 1);
      }
    }

    // ---- normalise and store the split's partials
    if (SC) {
      float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
      l_tot += __shfl_xor(l_tot, 32, kWave);
      if (g == 0) {
        const int64_t ps = (static_cast<int64_t>(b) * p.heads + head) * p.s_max + s;
        g_inv[hw][h] = l_tot > 0.f ? 1.f / l_tot : 0.f;
        p.part_lse[ps] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      }
    }
    // A split of one tile still copied tile 1 (the fixed wait counts above),
    // and gathered rows copy index tiles that no count covers: wait for all of
    // this wave's copies before the barrier, so that no copy can land in the
    // stages while the context waves stage O^T there.
    wait_vm<0>();
    lds_barrier();   // every wave's copies have landed: the stages are free
    if (!SC) {
      // O^T leaves through LDS so that every store instruction writes whole
      // partial rows: the wave's region holds its dims of every head, one row
      // per head padded to an odd number of 32-byte units, and each lane
      // stores 8 consecutive dims (one 16-byte store of bf16, two of fp32).
      // The per-head reciprocal comes from the score waves, the row addresses
      // advance by a fixed stride, and bf16 rounding is the hardware's
      // round-to-nearest-even conversion.  The stores are
      // non-temporal: the burst at the end of the launch does not wait on the
      // caches (3-4 us less per 169 MB launch, measured).
      constexpr int kEpiDims = kR / NW;
      constexpr int kLanesPerRow = kEpiDims / 8;
      constexpr int kRowsPerIter = kWave / kLanesPerRow;
      const int r0 = lane / kLanesPerRow, c8 = lane % kLanesPerRow;
      const int64_t row_step = static_cast<int64_t>(kRowsPerIter) * p.s_max * kR;   // elements
      int64_t e = ((static_cast<int64_t>(b) * p.heads + head0 + r0) * p.s_max + s) * kR + kEpiDims * hw + 8 * c8;
      if (p.part_bf16) {
        // bf16 partials: normalise and round in registers, so the LDS round
        // trip carries half the bytes
        constexpr int kEpiRow = kEpiDims * 2 + 32;
        char* region = g_stage + hw * (16 * NW * kEpiRow);
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) {
          const float inv = g_inv[hb][h];
#pragma unroll
          for (int db = 0; db < kCtxBlocks; ++db) {
            const f32x4 v = reg[db * NW + hb] * inv;
            bf16x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(v[j]);
            *reinterpret_cast<bf16x4*>(region + (16 * hb + h) * kEpiRow + (16 * db + 4 * g) * 2) = o;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave reads back its own writes
#pragma unroll 4
        for (int k = 0; k < 16 * NW / kRowsPerIter; ++k, e += row_step) {
          const int row = k * kRowsPerIter + r0;
          const f32x4 v = *reinterpret_cast<const f32x4*>(region + row * kEpiRow + c8 * 16);
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<uint16_t*>(p.part_o) + e));
        }
      } else {
        constexpr int kEpiRow = kEpiDims * 4 + 32;
        char* region = g_stage + hw * (16 * NW * kEpiRow);
#pragma unroll
        for (int hb = 0; hb < NW; ++hb)
#pragma unroll
          for (int db = 0; db < kCtxBlocks; ++db)
            *reinterpret_cast<f32x4*>(region + (16 * hb + h) * kEpiRow + (16 * db + 4 * g) * 4) = reg[db * NW + hb];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave reads back its own writes
#pragma unroll 4
        for (int k = 0; k < 16 * NW / kRowsPerIter; ++k, e += row_step) {
          const int row = k * kRowsPerIter + r0;
          const float inv = g_inv[row >> 4][row & 15];
          const char* src = region + row * kEpiRow + c8 * 32;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(src) * inv;
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 16) * inv;
          __builtin_nontemporal_store(v0, reinterpret_cast<f32x4*>(static_cast<float*>(p.part_o) + e));
          __builtin_nontemporal_store(v1, reinterpret_cast<f32x4*>(static_cast<float*>(p.part_o) + e + 4));
        }
      }
    }
  }
};

template <int NW, bool GATHER, bool PACKED>
__global__ __launch_bounds__(2 * NW * kWave) void decode_mfma_kernel(DecodeParams p) {
  // blockIdx.x enumerates the (row, split) pairs of the launch row by row;
  // find the row by bisection of the split prefix table (uniform, scalar).
  const int wg = blockIdx.x;
  int b = 0, hi = p.rows;
  while (hi - b > 1) {
    const int mid = (b + hi) >> 1;
    if (p.tab.split_begin[mid] <= wg) b = mid; else hi = mid;
  }
  const int s = wg - p.tab.split_begin[b];
  const int n_att = p.tab.n_att[b];
  const int j0 = s * p.chunk;
  Decode<NW, GATHER, PACKED> d(p);
  d.lane = threadIdx.x & (kWave - 1);
  d.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  d.scorer = d.wave < NW;
  d.hw = d.scorer ? d.wave : d.wave - NW;
  d.h = d.lane & 15;
  d.g = d.lane >> 4;
  d.head0 = blockIdx.z * (16 * NW);
  d.head = d.head0 + d.hw * 16 + d.h;
  d.n_tok = min(p.chunk, n_att - j0);
  d.nt = (d.n_tok + kNT - 1) / kNT;
  d.len = p.tab.kv_len[b];
  d.pad = p.width - d.len;
  d.gather_row = GATHER && p.tab.sel_off[b] >= 0;
  d.bad_index = false;
  d.sel_base = d.gather_row ? p.tab.sel_off[b] + j0 : j0;
  d.lat_base = static_cast<const char*>(p.latent) + static_cast<int64_t>(b) * p.lat_sb * 2;
  d.rope_base = static_cast<const char*>(p.rope) + static_cast<int64_t>(b) * p.rope_sb * 2;
  d.lat_st = p.lat_st * 2;
  d.rope_st = p.rope_st * 2;
  d.scale_log2 = p.scale * 1.4426950408889634f;
  d.run(b, s);
}

template <int NW, bool GATHER>
hipError_t launch_nw(const DecodeParams& p, bool packed, int groups, hipStream_t stream) {
  // One workgroup per (row, split) and head group, in a compact 1-D order:
  // with at most one workgroup per CU in flight, consecutive ids land on the
  // XCDs in turn, so a launch of S <= #CU splits never queues a second round
  // on one XCD.
  dim3 grid(p.s_total, 1, groups);
  if (packed)
    hipLaunchKernelGGL((decode_mfma_kernel<NW, GATHER, true>), grid, dim3(2 * NW * kWave), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<NW, GATHER, false>), grid, dim3(2 * NW * kWave), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Head counts of the instantiated groupings: one workgroup of 16 or 32 heads,
// or groups of 64 heads.  Other multiples of 16 (48, 80, ...) would need a
// grouping the kernel does not have; they take the generic kernel.
bool decode_mfma_supported(int32_t dtype, int32_t heads, int32_t r, int32_t dr) {
  return dtype == kBF16 && r == kR && dr == kDR && heads > 0 && (heads == 16 || heads == 32 || heads % 64 == 0);
}

// Layout requirements of the copy path: 16-byte aligned rows.
bool decode_mfma_layout_ok(const void* q_lat, const void* latent, int64_t lat_sb, int64_t lat_st, const void* rope,
                           int64_t rope_sb, int64_t rope_st) {
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  return al(q_lat) && al(latent) && al(rope) && lat_sb % 8 == 0 && lat_st % 8 == 0 && rope_sb % 8 == 0 &&
         rope_st % 8 == 0;
}

hipError_t launch_decode_mfma(const DecodeParams& p0, hipStream_t stream) {
  if (p0.rows == 0 || p0.s_total == 0) return hipSuccess;
  DecodeParams p = p0;
  // the query copy needs 16-byte aligned q_rope rows (q_lat rows are 1 KB)
  p.q_copy = (reinterpret_cast<uintptr_t>(p.q_rope) & 15) == 0 && p.qr_sb % 8 == 0 && p.qr_sh % 8 == 0;
  bool gather = false;
  for (int i = 0; i < p.rows; ++i) gather |= p.tab.sel_off[i] >= 0;
  const int nw = p.heads % 64 == 0 ? 4 : p.heads / 16;   // 1, 2 or 4 (decode_mfma_supported)
  const int groups = p.heads / (16 * nw);
  // Packed cache: rope right after the latent, same strides, and every byte
  // offset of a row start (plus its 1152 bytes) below 2^32.
  const bool packed = static_cast<const char*>(p.rope) == static_cast<const char*>(p.latent) + 2 * kR &&
                      p.rope_sb == p.lat_sb && p.rope_st == p.lat_st &&
                      (static_cast<int64_t>(p.rows - 1) * p.lat_sb + static_cast<int64_t>(p.width - 1) * p.lat_st) * 2 +
                              2 * (kR + kDR) <= 0xffffffffLL;
  switch (nw) {
    case 1: return gather ? launch_nw<1, true>(p, packed, groups, stream) : launch_nw<1, false>(p, packed, groups, stream);
    case 2: return gather ? launch_nw<2, true>(p, packed, groups, stream) : launch_nw<2, false>(p, packed, groups, stream);
    case 4: return gather ? launch_nw<4, true>(p, packed, groups, stream) : launch_nw<4, false>(p, packed, groups, stream);
    default: return hipErrorInvalidValue;   // unreachable behind decode_mfma_supported
  }
}

}  // namespace mla
