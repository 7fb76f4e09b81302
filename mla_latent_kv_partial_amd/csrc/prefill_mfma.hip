// MFMA reconstructed causal prefill for the bf16 GLM geometry (qk_nope 128,
// qk_rope 64, v_head 128).  Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts:
// Glm52Mla.project (q = q_b_proj(c_q), split into q_nope and q_rope, RoPE of
// q_rope at offset + t) and Glm52Mla.attendReconstructed (kv_b_proj expansion
// of the latent into per-head k_nope and v, scores over [q_nope|q_rope] .
// [k_nope|rope], causal mask, softmax, P.V); page "mlx-bun 0.2.0 -> 0.4.0",
// glm52-mla.ts: keys before the row's left pad are masked.
//
// Three kernels over a bf16 workspace:
//   NT GEMM with RoPE epilogue  Q  [rows*T, H*192] = c_q . w_q_b^T, the RoPE of
//                               each head's last 64 columns applied to the
//                               fp32 accumulators before rounding;
//   NT GEMM                     KV [rows*K, H*256] = latent . w_kv_b^T (per head
//                               k_nope then v);
//   flash_attn_kernel           one workgroup per (head, 128 queries): causal
//                               online-softmax attention, K/V tiles of 32 keys
//                               streamed through LDS, fp32 context out.
// The GEMMs live in gemm_mfma.hip.  The attention runs on
// v_mfma_f32_16x16x32_bf16; K/V tiles move HBM -> LDS with
// global_load_lds_dwordx4 into rows padded to an odd number of 32-byte units,
// which makes the 16-byte fragment reads of 16 consecutive rows free of bank
// conflicts (measured with the LDS bank-conflict counter).
#include <math.h>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {

bool prefill_mfma_shape_ok(const PrefillParams& p);
bool prefill_mfma_supported(const PrefillParams& p);
size_t prefill_mfma_workspace_bytes(const PrefillParams& p);
hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t stream);

namespace {

constexpr int kDn = 128, kDr = 64, kDv = 128;
constexpr int kQk = kDn + kDr;          // 192
constexpr int kKvw = kDn + kDv;         // 256
constexpr int kBatchPerLaunch = kGemmRowsPerLaunch;   // per-row tables travel in the kernel arguments

// ------------------------------------------------------------------ attention
// Workgroup = (head, 128 consecutive queries, batch row); wave w owns queries
// 32w .. 32w + 31 as two 16-query blocks.  Per 32-key tile each wave computes
// S^T[key, query] = K . Q^T (Q in registers, K fragments from LDS), the online
// softmax in exp2 with a lazily moved reference max, and O^T[dim, query] +=
// V^T . P^T (V^T fragments by ds_read_b64_tr_b16, each shared by the two
// query blocks).  The layout tricks are those of the latent decode kernel: key
// row m of a 16-key block holds key sigma(m), and rows are odd numbers of
// 32-byte units.  A stage holds the tile's KV rows (k_nope 16 chunks, v 16,
// pad 2: 544 B) and then its rope rows (8 chunks, pad 2: 160 B).  Each 1 KB
// copy then reads either KV rows or rope rows only, from a wave-uniform base
// (SGPRs) that moves by 32 keys per tile plus a per-lane offset that stays
// fixed, so a tile's copies cost no vector arithmetic.
constexpr int kAWaves = 4;                                   // waves per workgroup, 32 queries each
constexpr int kAQ = 32 * kAWaves;
constexpr int kAK = 32;
constexpr int kAKvChunks = 34;
constexpr int kAKvRowBytes = kAKvChunks * 16;                // 544
constexpr int kARopeChunks = 10;
constexpr int kARopeRowBytes = kARopeChunks * 16;            // 160
constexpr int kAKvDma = kAK * kAKvChunks / 64;               // 17 copies of 1 KB
constexpr int kARopeDma = kAK * kARopeChunks / 64;           // 5
constexpr int kARopeOffset = kAKvDma * 1024;                 // rope rows after the KV rows
constexpr int kATileDma = kAKvDma + kARopeDma;               // 22
constexpr int kAStageBytes = kATileDma * 1024;
static_assert(kAK * kAKvChunks % 64 == 0 && kAK * kARopeChunks % 64 == 0, "whole copies per region");
// Two ring stages (44 KB of LDS) and at most 168 VGPRs let three workgroups
// share a CU; at 4096 tokens that ran faster than a third stage at two
// workgroups per CU (483 against 582 us).  With two stages each tile's copies
// are waited for in full before the next tile is issued.
constexpr int kAStages = 2;
constexpr int kAWavesPerEu = 3;
constexpr int kAMaxDma = (kATileDma + kAWaves - 1) / kAWaves;   // copies per wave (the first waves take one more)
constexpr float kSlack = 8.f;

__shared__ __attribute__((aligned(1024))) char g_attn[kAStages * kAStageBytes];

struct AttnMfma {
  const uint16_t* q;      // [rows*T, H*192]
  const uint16_t* kv;     // [rows*K, H*256]
  const uint16_t* rope;   // [rows*K, 64]
  float* ctx;             // [rows*T, H*128]
  int32_t tokens, keys, heads, q_tiles;
  float scale_log2;
  int32_t pad[kBatchPerLaunch];
};

// Maxima of values that are never NaN (finite scores or -inf), as single
// v_max3_f32 / v_max_f32: fmaxf would first quiet every operand the compiler
// cannot prove canonical (lane swaps, selects), one extra VALU op each.
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over lanes i, i ^ 16, i ^ 32 and i ^ 48 by v_permlane16_swap and
// v_permlane32_swap (VALU; a lane shuffle through ds_bpermute waits on LDS).
// With both operands x, the 16-lane-row swap returns rows (0, 0, 2, 2) and
// (1, 1, 3, 3) of x, the 32-lane swap the halves (lo, lo) and (hi, hi).
__device__ __forceinline__ float max_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ int sigma(int m) {
  return 2 * (m & 3) + ((m >> 2) & 1) + 8 * ((m >> 3) & 1);
}

__global__ __launch_bounds__(64 * kAWaves, kAWavesPerEu) void flash_attn_kernel(AttnMfma p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x;
  const int qt = p.q_tiles - 1 - static_cast<int>(blockIdx.y);   // heaviest tiles first
  const int b = blockIdx.z;
  const int t0 = qt * kAQ;
  const int P = p.keys - p.tokens;
  const int pad = p.pad[b];
  const int m = lane & 15, g = lane >> 4;

  // key tiles: from the left pad (rounded down) through the last key the
  // workgroup's last query may see
  const int k_first = (pad / kAK) * kAK;
  const int k_last = min(p.keys - 1, P + min(t0 + kAQ, p.tokens) - 1);
  const int nt = k_last >= k_first ? (k_last - k_first) / kAK + 1 : 0;

  // ---- copy plan (same for every tile): copy x = wave + kAWaves j of a stage
  // fills LDS bytes [1024 x, +1024).  x < 17: KV slot q = 64 x + lane is chunk
  // q % 34 of KV row q / 34 (chunks 32, 33 pad: re-read chunk 0); otherwise
  // rope slot q = 64 (x - 17) + lane is chunk q % 10 of rope row q / 10
  // (chunks 8, 9 pad).  voff[j] = the lane's byte offset from the tile's
  // first KV (rope) row.
  const int n_dma = (kATileDma - wave + kAWaves - 1) / kAWaves;
  const char* kv_base = reinterpret_cast<const char*>(p.kv + (static_cast<int64_t>(b) * p.keys * p.heads + h) * kKvw);
  const char* rope_base = reinterpret_cast<const char*>(p.rope + static_cast<int64_t>(b) * p.keys * kDr);
  const int64_t kv_stride = static_cast<int64_t>(p.heads) * kKvw * 2;   // a multiple of 512
  uint32_t voff[kAMaxDma];
#pragma unroll
  for (int j = 0; j < kAMaxDma; ++j) {
    const int x = wave + kAWaves * j;
    if (x < kAKvDma) {
      const int q = 64 * x + lane;
      const int row = q / kAKvChunks, c = q - row * kAKvChunks;
      voff[j] = static_cast<uint32_t>(row * kv_stride + (c < 32 ? c * 16 : 0));
    } else {
      const int q = 64 * (x - kAKvDma) + lane;
      const int row = q / kARopeChunks, c = q - row * kARopeChunks;
      voff[j] = static_cast<uint32_t>(row * (kDr * 2) + (c < 8 ? c * 16 : 0));
    }
  }
  // A tile past the last key: its missing rows re-read the tile's first row
  // (same chunk; rows are whole multiples of the 512-byte / 128-byte masks),
  // whose scores are masked and whose probabilities are exactly zero.
  auto issue = [&](int s, int tile) {
    const uint32_t dst = lds_addr(g_attn + s * kAStageBytes);
    const int k0 = k_first + tile * kAK;
    const char* kv_t = kv_base + static_cast<int64_t>(k0) * kv_stride;
    const char* rope_t = rope_base + static_cast<int64_t>(k0) * (kDr * 2);
    const bool part = k0 + kAK > p.keys;
    const int rows = p.keys - k0;
#pragma unroll
    for (int j = 0; j < kAMaxDma; ++j) {
      const int x = wave + kAWaves * j;
      if (j == kAMaxDma - 1 && n_dma < kAMaxDma) break;
      const bool kv = x < kAKvDma;
      uint32_t off = voff[j];
      if (part) {
        const uint32_t lim = static_cast<uint32_t>(rows * (kv ? kv_stride : kDr * 2));
        off = off < lim ? off : off & (kv ? 511u : 127u);
      }
      dma16_off(kv ? kv_t : rope_t, off, dst + x * 1024);
    }
  };

  // ---- queries of this wave: two blocks of 16, B operands of the scores
  f32x4 qreg[2][kQk / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = min(t0 + 32 * wave + 16 * qb + m, p.tokens - 1);
    const uint16_t* qrow = p.q + (static_cast<int64_t>(b) * p.tokens + t) * p.heads * kQk + h * kQk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kQk / 32; ++ks) qreg[qb][ks] = *reinterpret_cast<const f32x4*>(qrow + 32 * ks);
  }
  // Take the queries as landed here: the compiler waits for their loads once,
  // before the loop.  (Otherwise it keeps a wait for them at their first uses
  // inside the loop, where the hardware counter also holds the next tile's
  // copies: every tile's scores would wait for the next tile to land.)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < kQk / 32; ++ks) asm volatile("" : "+v"(qreg[qb][ks]));
  for (int t = 0; t < kAStages - 1 && t < nt; ++t) issue(t, t);
  // Probabilities are exp2(fma(score, cs, -max)) with cs > 0 (the tile max
  // of the raw scores times cs is the max of the scaled scores, rounding
  // being monotonic).  A negative scale flips the sign of the queries instead
  // (exact in bf16); a zero scale becomes the least normal float, whose
  // products stay below 2^-24 in magnitude, so every visible key still gets
  // weight exactly 1 while masked scores stay -inf.
  float cs = p.scale_log2;
  if (cs < 0.f) {
    cs = -cs;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < kQk / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qreg[qb][ks][e] = __uint_as_float(__float_as_uint(qreg[qb][ks][e]) ^ 0x80008000u);
  }
  cs = fmaxf(cs, 1.17549435e-38f);

  const uint32_t k_frag = sigma(m) * kAKvRowBytes + g * 16;
  const uint32_t r_frag = kARopeOffset + sigma(m) * kARopeRowBytes + g * 16;
  const uint32_t v_frag = sigma(4 * g + (m >> 2)) * kAKvRowBytes + kDn * 2 + ((m & 3) >> 1) * 16 + (m & 1) * 8;
  f32x4 o[2][kDv / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const int t_lo = t0 + 32 * wave;           // first query of the wave
  const int t_q[2] = {t_lo + m, t_lo + 16 + m};

  for (int i = 0; i < nt; ++i) {
    // tile i's copies done; those of the later tiles issued so far may fly
    wait_vm_upto<kAMaxDma * (kAStages - 2)>(n_dma * min(nt - 1 - i, kAStages - 2));
    lds_barrier();
    if (i + kAStages - 1 < nt) issue((i + kAStages - 1) % kAStages, i + kAStages - 1);
    const int k0 = k_first + i * kAK;
    // tiles past every query of this wave contribute nothing
    if (k0 > P + t_lo + 31 || k0 + kAK - 1 < pad) continue;
    const char* st = g_attn + (i % kAStages) * kAStageBytes;
    f32x4 s[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) s[qb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kQk / 32; ++ks) {
      // k_nope from the KV rows, then rope from the rope rows
      const uint32_t addr = ks < kDn / 32 ? k_frag + ks * 64 : r_frag + (ks - kDn / 32) * 64;
      const uint32_t row16 = ks < kDn / 32 ? 16 * kAKvRowBytes : 16 * kARopeRowBytes;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(st + addr + tb * row16);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[qb][tb] = mfma16x16x32(kf, __builtin_bit_cast(bf16x8, qreg[qb][ks]), s[qb][tb]);
      }
    }
    // raw scores; masked entries -inf.  One wave-uniform branch per tile
    // for both query blocks: a tile every key of which every query of the
    // wave sees takes no mask arithmetic at all.
    float x[2][8];
    if (k0 + kAK - 1 <= P + t_lo && k0 >= pad) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[qb][4 * tb + e] = s[qb][tb][e];
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 16 * tb + sigma(4 * g + e);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const bool vis = key >= pad && key <= P + t_q[qb];
            x[qb][4 * tb + e] = vis ? s[qb][tb][e] : -INFINITY;
          }
        }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // no score is NaN, so the maxima need no quieting of their operands
      float mt = max3_nn(x[qb][0], x[qb][1], x[qb][2]);
      mt = max3_nn(mt, x[qb][3], x[qb][4]);
      mt = max3_nn(mt, x[qb][5], x[qb][6]);
      mt = max_nn(mt, x[qb][7]);
      mt = max_lanes_xor16_32(mt) * cs;
      const bool move = mt > m_run[qb] + kSlack;
      if (__any(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run[qb] - mt) : 1.f;
        if (move) m_run[qb] = mt;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) o[qb][db] *= alpha;
      }
      // m_run still -inf: every x of the query is -inf, and exp2(-inf - 0) = 0
      const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(x[qb][e], cs, -m_use));
        l_run[qb] += pr;
        pb[qb][e] = static_cast<__bf16>(pr);
      }
    }
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
      const s16x4 v1 = lds_read_tr16(st + v_frag + db * 32);
      const s16x4 v2 = lds_read_tr16(st + v_frag + 16 * kAKvRowBytes + db * 32);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[qb][db] = mfma16x16x32(vf, pb[qb], o[qb][db]);
    }
  }

  // ---- normalise and store: lane (query m, group g) holds dims 16 db + 4 g + (0..3)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb] + __shfl_xor(l_run[qb], 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // lane-derived values recomputed here rather than kept live across the loop
    const int ln = threadIdx.x & 63;
    const int t = t0 + 32 * wave + 16 * qb + (ln & 15);
    if (t >= p.tokens) continue;
    float* out = p.ctx + (static_cast<int64_t>(b) * p.tokens + t) * p.heads * kDv + h * kDv + 4 * (ln >> 4);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
      const f32x4 v = o[qb][db] * inv;
      *reinterpret_cast<float4*>(out + 16 * db) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// The shapes of the MFMA path (64: the K step of the GEMMs) ...
bool prefill_mfma_shape_ok(const PrefillParams& p) {
  return p.dtype == kBF16 && p.dn == kDn && p.dr == kDr && p.dv == kDv && p.ql % 64 == 0 && p.r % 64 == 0 &&
         p.heads <= 65535;
}

// ... and 16-byte aligned buffers.
bool prefill_mfma_supported(const PrefillParams& p) {
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  return prefill_mfma_shape_ok(p) && al(p.q_c) && al(p.w_qb) && al(p.latent) && al(p.rope) && al(p.w_kvb) &&
         al(p.ctx);
}

// q RoPE table of one launch: {cos, sin} (f32) per query row and pair
size_t rope_table_bytes(const PrefillParams& p) {
  return static_cast<size_t>(min(p.batch, kBatchPerLaunch)) * p.tokens * 32 * sizeof(float2);
}

size_t prefill_mfma_workspace_bytes(const PrefillParams& p) {
  const size_t q = static_cast<size_t>(p.batch) * p.tokens * p.heads * kQk * 2;
  const size_t kv = static_cast<size_t>(p.batch) * p.keys * p.heads * kKvw * 2;
  return up256(q) + up256(kv) + up256(rope_table_bytes(p));
}

hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t stream) {
  uint16_t* q = static_cast<uint16_t*>(p.workspace);
  const size_t q_bytes = static_cast<size_t>(p.batch) * p.tokens * p.heads * kQk * 2;
  const size_t kv_bytes = static_cast<size_t>(p.batch) * p.keys * p.heads * kKvw * 2;
  uint16_t* kv = reinterpret_cast<uint16_t*>(static_cast<char*>(p.workspace) + up256(q_bytes));
  float2* cs = reinterpret_cast<float2*>(static_cast<char*>(p.workspace) + up256(q_bytes) + up256(kv_bytes));
  const uint16_t* q_c = static_cast<const uint16_t*>(p.q_c);
  const uint16_t* latent = static_cast<const uint16_t*>(p.latent);
  const uint16_t* rope = static_cast<const uint16_t*>(p.rope);
  float inv[kDr / 2];
  rope_inverse_frequencies(kDr, p.theta, inv);
  for (int b0 = 0; b0 < p.batch; b0 += kBatchPerLaunch) {
    const int rows = min(p.batch - b0, kBatchPerLaunch);
    // Q projection with the RoPE epilogue
    GemmNT gq{};
    gq.a = q_c + static_cast<int64_t>(b0) * p.tokens * p.ql;
    gq.lda = p.ql;
    gq.b = static_cast<const uint16_t*>(p.w_qb);
    gq.ldb = p.ql;
    gq.c = q + static_cast<int64_t>(b0) * p.tokens * p.heads * kQk;
    gq.ldc = static_cast<int64_t>(p.heads) * kQk;
    gq.m = rows * p.tokens;
    gq.n = p.heads * kQk;
    gq.k = p.ql;
    gq.tokens = p.tokens;
    for (int i = 0; i < rows; ++i) gq.off[i] = p.q_offsets[b0 + i];
    for (int i = 0; i < kDr / 2; ++i) gq.inv[i] = inv[i];
    gq.cs = cs;
    hipError_t e = launch_rope_table(gq, cs, stream);
    if (e != hipSuccess) return e;
    e = launch_gemm_nt_mfma(gq, true, false, stream);
    if (e != hipSuccess) return e;
    // KV expansion
    GemmNT gk{};
    gk.a = latent + static_cast<int64_t>(b0) * p.keys * p.r;
    gk.lda = p.r;
    gk.b = static_cast<const uint16_t*>(p.w_kvb);
    gk.ldb = p.r;
    gk.c = kv + static_cast<int64_t>(b0) * p.keys * p.heads * kKvw;
    gk.ldc = static_cast<int64_t>(p.heads) * kKvw;
    gk.m = rows * p.keys;
    gk.n = p.heads * kKvw;
    gk.k = p.r;
    gk.tokens = p.keys;
    e = launch_gemm_nt_mfma(gk, false, false, stream);
    if (e != hipSuccess) return e;
    // attention
    AttnMfma ap{};
    ap.q = static_cast<const uint16_t*>(gq.c);
    ap.kv = static_cast<const uint16_t*>(gk.c);
    ap.rope = rope + static_cast<int64_t>(b0) * p.keys * kDr;
    ap.ctx = p.ctx + static_cast<int64_t>(b0) * p.tokens * p.heads * kDv;
    ap.tokens = p.tokens;
    ap.keys = p.keys;
    ap.heads = p.heads;
    ap.q_tiles = (p.tokens + kAQ - 1) / kAQ;
    ap.scale_log2 = p.scale * 1.4426950408889634f;
    for (int i = 0; i < rows; ++i) ap.pad[i] = p.left_pad ? p.left_pad[b0 + i] : 0;
    hipLaunchKernelGGL(flash_attn_kernel, dim3(p.heads, ap.q_tiles, rows), dim3(64 * kAWaves), 0, stream, ap);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
