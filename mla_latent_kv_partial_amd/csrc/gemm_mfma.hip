// MFMA NT GEMM for bf16 operands (both K-contiguous), fp32 accumulation,
// bf16 or fp32 result.  Serves the prefill projections of page "mlx-bun
// 0.0.11 -> 0.0.13", glm52-mla.ts (q_b_proj with the q RoPE of
// Glm52Mla.project as an epilogue; the kv_b_proj expansion of
// attendReconstructed) and the o_proj linear after the attention.
#include <math.h>
#include <type_traits>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kDn = 128, kDr = 64;      // RoPE epilogue geometry: 128 no-PE + 64 rope columns per head
constexpr int kQk = kDn + kDr;

// ------------------------------------------------------------------ NT GEMM
// C[m, n] = sum_k A[m, k] B[n, k]: both operands K-contiguous, bf16; fp32
// accumulation; bf16 result (round to nearest even) or fp32.  Workgroup tile 128 x 128,
// K step 64, 4 waves of 64 x 64 (4 x 4 MFMA blocks), 2-stage LDS ring filled
// one K step ahead; two workgroups per CU hide each other's waits.
constexpr int kGT = 128;
constexpr int kGK = 64;
constexpr int kGRowChunks = kGK / 8 + 2;            // eight data chunks + two pad
constexpr int kGRowBytes = kGRowChunks * 16;        // 160
constexpr int kGOpChunks = kGT * kGRowChunks;       // 1280 per operand tile
constexpr int kGOpDma = kGOpChunks / 64;            // 20 copies of 1 KB
constexpr int kGOpBytes = kGOpChunks * 16;
constexpr int kGStageBytes = 2 * kGOpBytes;         // A tile then B tile
constexpr int kGStages = 2;   // 80 KB of LDS: two workgroups share a CU (measured faster than 3 or 4 stages)
constexpr int kGMaxDma = (kGOpDma + 3) / 4;         // copies per wave per operand

__shared__ __attribute__((aligned(1024))) char g_gemm[kGStages * kGStageBytes];

// Epilogue of one lane: columns n .. n+3 of row m (n a multiple of 4), bf16
// (round to nearest even) or fp32.
template <bool OUT_F32>
__device__ __forceinline__ void store_cols4(const GemmNT& p, int m, int n, const f32x4& v) {
  if (OUT_F32) {
    float* frow = static_cast<float*>(p.c) + static_cast<int64_t>(m) * p.ldc;
    *reinterpret_cast<float4*>(frow + n) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint16_t* crow = static_cast<uint16_t*>(p.c) + static_cast<int64_t>(m) * p.ldc;
    const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<uint2*>(crow + n) = make_uint2(lo, hi);
  }
}

// One rope pair (a, b) of a q row rotated by the table's (cos, sin) in fp32
// (two products and one fused add each), rounded once to bf16; the 128 x 128
// and the 256 x 256 tiles share it, so both give the same bits.
__device__ __forceinline__ void rope_pair_bf16(float a, float b, float2 cs, uint16_t& re, uint16_t& im) {
  re = f32_to_bf16(fmaf(a, cs.x, -(b * cs.y)));
  im = f32_to_bf16(fmaf(b, cs.x, a * cs.y));
}

// A wave's output blocks: block (bm, bn) lane (i16, g) holds row
// m_base + 16 bm + i16, columns n_base + 16 bn + 4 g .. +3.  n_base is a
// multiple of 64 and the wave spans at most 64 columns, so with ROPE (the q
// projection, 192 columns per head: 128 no-PE, then 64 rope) its columns are
// either all no-PE or all the rope part of one head.  Rope columns are
// rotated at the row's position and written as split halves: columns
// (v0, v1) and (v2, v3) are rope pairs q0 and q0 + 1 of the head, rotated by
// the row's cos and sin from the table (rope_pair_bf16).  A rope wave requests the table entries of four row blocks at a time
// (2 BN float2 per block, in the registers the fragments held) before it
// rotates them, so their latency is paid twice per tile, not once per block.
template <bool ROPE, bool OUT_F32, int BM, int BN>
__device__ __forceinline__ void store_tile(const GemmNT& p, const f32x4 (&acc)[BM][BN], int m_base, int n_base,
                                           int i16, int g) {
  static_assert(16 * BN <= 64, "a wave spans at most 64 columns");
  if (ROPE && n_base % kQk >= kDn) {
    const int head_col = n_base - n_base % kQk;           // first column of the head
    const int q_lane = (n_base % kQk - kDn) / 2 + 2 * g;  // pair of column n_base + 4 g
    constexpr int kChunk = BM < 4 ? BM : 4;   // row blocks whose table entries fly together
#pragma unroll
    for (int b0 = 0; b0 < BM; b0 += kChunk) {
      float2 t[kChunk][BN][2];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int m = min(m_base + 16 * (b0 + u) + i16, p.m - 1);
        const float2* cs = p.cs + static_cast<int64_t>(m) * 32 + q_lane;
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) {
          t[u][bn][0] = cs[8 * bn];
          t[u][bn][1] = cs[8 * bn + 1];
        }
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int m = m_base + 16 * (b0 + u) + i16;
        if (m >= p.m) continue;
        uint16_t* head = static_cast<uint16_t*>(p.c) + static_cast<int64_t>(m) * p.ldc + head_col + kDn;
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) {
          if (n_base + 16 * bn + 4 * g >= p.n) continue;
          const int q0 = q_lane + 8 * bn;
          uint16_t re[2], im[2];
#pragma unroll
          for (int e = 0; e < 2; ++e)
            rope_pair_bf16(acc[b0 + u][bn][2 * e], acc[b0 + u][bn][2 * e + 1], t[u][bn][e], re[e], im[e]);
          *reinterpret_cast<uint32_t*>(head + q0) = re[0] | (static_cast<uint32_t>(re[1]) << 16);
          *reinterpret_cast<uint32_t*>(head + kDr / 2 + q0) = im[0] | (static_cast<uint32_t>(im[1]) << 16);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int bm = 0; bm < BM; ++bm) {
    const int m = m_base + 16 * bm + i16;
    if (m >= p.m) continue;
#pragma unroll
    for (int bn = 0; bn < BN; ++bn) {
      const int n = n_base + 16 * bn + 4 * g;
      if (n < p.n) store_cols4<OUT_F32>(p, m, n, acc[bm][bn]);
    }
  }
}

// Workgroup id -> tile: ids go round-robin over the 8 XCDs; each XCD gets a
// contiguous run of tiles, M fastest, so the workgroups that share an XCD's L2
// also share B tiles (plain order when the tiles do not split evenly).
__device__ __forceinline__ int xcd_tile(int id, int tiles) {
  if (tiles % 8 != 0) return id;
  return (id & 7) * (tiles / 8) + (id >> 3);
}

template <bool ROPE, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_nt_mfma_kernel(GemmNT p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int m0 = (tile % p.m_tiles) * kGT;
  const int n0 = (tile / p.m_tiles) * kGT;

  // copy plan: copy j of this wave moves chunk q = 64 (wave + 4 j) + lane of
  // an operand tile: row q / 10, chunk q % 10 (chunks 8 and 9 are padding and
  // re-read chunk 0); rows past the matrix edge re-read its last row.
  const int n_dma = (kGOpDma - wave + 3) / 4;
  const uint16_t* asrc[kGMaxDma];
  const uint16_t* bsrc[kGMaxDma];
#pragma unroll
  for (int j = 0; j < kGMaxDma; ++j) {
    const int q = 64 * (wave + 4 * j) + lane;
    const int row = q / kGRowChunks;
    int c = q - row * kGRowChunks;
    c = c < 8 ? c : 0;
    asrc[j] = p.a + static_cast<int64_t>(min(m0 + row, p.m - 1)) * p.lda + 8 * c;
    bsrc[j] = p.b + static_cast<int64_t>(min(n0 + row, p.n - 1)) * p.ldb + 8 * c;
  }
  auto issue = [&](int s, int k0) {
    const uint32_t da = lds_addr(g_gemm + s * kGStageBytes);
    const uint32_t db = da + kGOpBytes;
#pragma unroll
    for (int j = 0; j < kGMaxDma - 1; ++j) {
      dma16(asrc[j] + k0, da + (wave + 4 * j) * 1024);
      dma16(bsrc[j] + k0, db + (wave + 4 * j) * 1024);
    }
    if (n_dma == kGMaxDma) {
      dma16(asrc[kGMaxDma - 1] + k0, da + (wave + 4 * (kGMaxDma - 1)) * 1024);
      dma16(bsrc[kGMaxDma - 1] + k0, db + (wave + 4 * (kGMaxDma - 1)) * 1024);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g = lane >> 4;
  const uint32_t a_frag = (64 * wm + i16) * kGRowBytes + g * 16;
  const uint32_t b_frag = kGOpBytes + (64 * wn + i16) * kGRowBytes + g * 16;

  const int nk = p.k / kGK;
  // the ring runs kGStages - 1 K steps ahead
  for (int t = 0; t < kGStages - 1 && t < nk; ++t) issue(t, t * kGK);
  f32x4 acc[4][4];
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < nk; ++i) {
    // tile i's copies done; those of the following tiles issued so far may fly
    const int later = min(nk - 1 - i, kGStages - 2);
    wait_vm_upto<2 * kGMaxDma * (kGStages - 2)>(2 * n_dma * later);
    lds_barrier();
    if (i + kGStages - 1 < nk) issue((i + kGStages - 1) % kGStages, (i + kGStages - 1) * kGK);
    const char* st = g_gemm + (i % kGStages) * kGStageBytes;
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = *reinterpret_cast<const bf16x8*>(st + a_frag + t * 16 * kGRowBytes + ks * 64);
        bfr[t] = *reinterpret_cast<const bf16x8*>(st + b_frag + t * 16 * kGRowBytes + ks * 64);
      }
      // D^T blocks: lane (column m = i16, group g) receives C[m][n + 4g + (0..3)]
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = mfma16x16x32(bfr[bn], af[bm], acc[bm][bn]);
    }
  }

  // ---- epilogue: 4 consecutive columns per lane and block
  store_tile<ROPE, OUT_F32>(p, acc, m0 + 64 * wm, n0 + 64 * wn, i16, g);
}

// ------------------------------------------------------------------ 256 x 256 NT GEMM
// Same contract, workgroup tile 256 x 256 for long GEMMs: 8 waves of 128 x 64
// (8 x 4 MFMA blocks).  The operands stream through LDS in K steps of 64 as
// half stages: the A or the B slice of one step (256 rows of 128 bytes, 32
// KB), in a ring of five slots (160 KB), so that up to three half stages fly
// while a step computes.  A row's 16-byte chunk c sits at position
// c ^ (r & 7) of its 128-byte line: each 1 KB copy instruction fills 8 whole
// rows (every request covers whole 128-byte row segments; measured on the
// copy path alone, 23 % faster than the 64-byte segments of 32-wide K steps),
// and the fragment reads (16 rows, one chunk each) hit 32 distinct banks per
// 8 lanes.
// Per K step a wave runs its MFMAs in two halves of K = 32; the fragments of
// each half are read from LDS while the MFMAs of the half before run, and
// the step's one barrier sits between the halves: after it, step i + 1 has
// landed (every wave waited for its own copies) and every wave has finished
// reading step i, whose two slots then take the copies of the next two half
// stages.
constexpr int kBT = 256;
constexpr int kBK = 64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // operand of the non-temporal store builtin
constexpr int kBRowBytes = kBK * 2;                 // 128
constexpr int kBHalfBytes = kBT * kBRowBytes;       // 32 KB: one operand's slice of a step
constexpr int kBSlots = 5;
constexpr int kBCopies = kBHalfBytes / 1024 / 8;    // 1 KB copies per wave per half stage (4)

__shared__ __attribute__((aligned(1024))) char g_gemm256[kBSlots * kBHalfBytes];

// Epilogue of the 256 x 256 tile through LDS (free once the K loop is done):
// the waves write their accumulators in their fragment layout (bf16 rounded
// to nearest even, or fp32), then the tile leaves in whole rows, every store
// instruction covering full 128-byte lines, where the fragment layout stores
// 32-byte pieces of 16 rows (measured: the epilogue took as long as a third
// of the MFMA work).  fp32 tiles go in two passes of 128 rows.
template <bool ROPE, bool OUT_F32, int BN>
__device__ __forceinline__ void store_tile_staged(const GemmNT& p, const f32x4 (&acc)[8][BN / 64], int m0, int n0,
                                                  int wm, int wn, int i16, int g) {
  static_assert(!(ROPE && OUT_F32), "the q projection writes bf16");
  static_assert(!ROPE || BN == 256, "the RoPE epilogue takes 64-column wave spans");
  constexpr int kNb = BN / 64;                      // 16-column blocks per wave
  constexpr int kEs = OUT_F32 ? 4 : 2;              // bytes per element
  constexpr int kRowB = BN * kEs + 16;              // LDS row stride
  constexpr int kPassRows = OUT_F32 ? 128 : 256;
  constexpr int kChunks = BN * kEs / 16;            // 16-byte chunks per row
  static_assert(kPassRows * kRowB <= kBSlots * kBHalfBytes, "a pass fits the LDS ring");
  const int tid = threadIdx.x;
  const bool al16 = (p.ldc * kEs) % 16 == 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  lds_barrier();   // every wave is past its last fragment reads
#pragma unroll
  for (int pass = 0; pass < 256 / kPassRows; ++pass) {
    const int n_base = n0 + 64 * wn;
    if (ROPE && n_base % kQk >= kDn) {
      // rope columns: rotated here, written as split halves (pair q at column
      // q, its imaginary part at 32 + q of the head's rope part), with the
      // table entries of four row blocks requested at a time
      const int q_lane = (n_base % kQk - kDn) / 2 + 2 * g;   // pair of column n_base + 4 g
      const int rope_col = 64 * wn - (n_base % kQk - kDn);    // tile column of the head's rope part
#pragma unroll
      for (int b0 = 0; b0 < 8; b0 += 4) {
        float2 t[4][kNb][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = min(m0 + 128 * wm + 16 * (b0 + u) + i16, p.m - 1);
          const float2* cs = p.cs + static_cast<int64_t>(m) * 32 + q_lane;
#pragma unroll
          for (int bn = 0; bn < kNb; ++bn) {
            t[u][bn][0] = cs[8 * bn];
            t[u][bn][1] = cs[8 * bn + 1];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int bn = 0; bn < kNb; ++bn) {
            uint16_t re[2], im[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
              rope_pair_bf16(acc[b0 + u][bn][2 * e], acc[b0 + u][bn][2 * e + 1], t[u][bn][e], re[e], im[e]);
            char* d = g_gemm256 + (128 * wm + 16 * (b0 + u) + i16) * kRowB + (rope_col + q_lane + 8 * bn) * kEs;
            *reinterpret_cast<uint32_t*>(d) = re[0] | (static_cast<uint32_t>(re[1]) << 16);
            *reinterpret_cast<uint32_t*>(d + (kDr / 2) * kEs) = im[0] | (static_cast<uint32_t>(im[1]) << 16);
          }
      }
    } else if (!OUT_F32 || wm == pass) {
      const int rbase = OUT_F32 ? 0 : 128 * wm;
#pragma unroll
      for (int bm = 0; bm < 8; ++bm)
#pragma unroll
        for (int bn = 0; bn < kNb; ++bn) {
          char* d = g_gemm256 + (rbase + 16 * bm + i16) * kRowB + (16 * kNb * wn + 16 * bn + 4 * g) * kEs;
          const f32x4& v = acc[bm][bn];
          if (OUT_F32) {
            *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
            const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(d) = make_uint2(lo, hi);
          }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
    for (int e = tid; e < kPassRows * kChunks; e += 512) {
      const int r = e / kChunks, ch = e % kChunks;
      const int m = m0 + pass * kPassRows + r;
      const int n = n0 + ch * (16 / kEs);
      if (m < p.m && n < p.n) {
        const uint4 v = *reinterpret_cast<const uint4*>(g_gemm256 + r * kRowB + ch * 16);
        char* crow = static_cast<char*>(p.c) + (static_cast<int64_t>(m) * p.ldc + n) * kEs;
        if (al16 && n + 16 / kEs <= p.n) {
          if constexpr (ROPE) {
            // q rows are read once, by the attention: stored non-temporally
            // they leave the last-level cache to the operands still being
            // re-read (4096-token prefill: q_b 165 -> 161.5, kv_b 102.9 ->
            // 101.3, flash 387.5 -> 382.1 us; on kv_b's own output the hint
            // cost 10 us)
            u32x4 nv;
            nv.x = v.x; nv.y = v.y; nv.z = v.z; nv.w = v.w;
            __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(crow));
          } else {
            *reinterpret_cast<uint4*>(crow) = v;
          }
        } else {   // 8-byte pieces (the row is 8-byte aligned; n + 4 elements of bf16 or 2 of fp32 may end it)
          *reinterpret_cast<uint2*>(crow) = make_uint2(v.x, v.y);
          if (n + 8 / kEs < p.n) *reinterpret_cast<uint2*>(crow + 8) = make_uint2(v.z, v.w);
        }
      }
    }
    if (pass + 1 < 256 / kPassRows) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();   // the pass's rows are read before the next pass overwrites them
    }
  }
}

// BN = 256, or 192 (waves of 128 x 48, B slices of 192 rows) where that
// tiles the output into whole rounds of the CUs and 256 does not.
template <bool ROPE, bool OUT_F32, int BN>
__global__ __launch_bounds__(512) void gemm256_nt_kernel(GemmNT p) {
  static_assert(BN == 256 || BN == 192, "column tile");
  constexpr int kNb = BN / 64;   // 16-column blocks per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int m0 = (tile % p.m_tiles) * kBT;
  const int n0 = (tile / p.m_tiles) * BN;

  // copy plan: waves 0..3 issue every copy (8 per half stage each), so the
  // waves sharing their SIMDs (4..7) keep issuing MFMAs while a copy holds
  // its wave at the address path (q_b 184 -> 174 us).  Copy j of issuing wave
  // w fills 8-row block q = w + 4 j of a half stage; lane l lands at
  // position l of the block: row l / 8, position l % 8, which holds chunk
  // (l % 8) ^ (l / 8).  Each copy is an SGPR base (the operand at the step's
  // K offset) plus a 32-bit lane offset (the launcher takes this kernel only
  // for operands under 4 GB).  Rows past the matrix edge re-read its last row.
  constexpr int kIss = 2 * kBCopies;     // A copies per issuing wave and half stage (8)
  constexpr int kIssB = BN / 32;         // B copies (8, or 6)
  uint32_t offa[kIss], offb[kIssB];
  const bool issuer = wave < 4;
#pragma unroll
  for (int j = 0; j < kIss; ++j) {
    const int r8 = lane >> 3;
    const int row = 8 * ((wave & 3) + 4 * j) + r8;
    const int c = (lane & 7) ^ r8;
    offa[j] = static_cast<uint32_t>((static_cast<int64_t>(min(m0 + row, p.m - 1)) * p.lda + 8 * c) * 2);
    if (j < kIssB)
      offb[j] = static_cast<uint32_t>((static_cast<int64_t>(min(n0 + row, p.n - 1)) * p.ldb + 8 * c) * 2);
  }
  // half stage h: the A slice (h even) or the B slice (h odd) of step h / 2, in slot h % 5
  const int nh = 2 * (p.k / kBK);
  auto issue = [&](int h) {
    if (h >= nh || !issuer) return;
    const uint32_t dst = lds_addr(g_gemm256 + (h % kBSlots) * kBHalfBytes) + (wave & 3) * 1024;
    const int k0 = (h >> 1) * kBK;
    if (h & 1) {
      const char* base = reinterpret_cast<const char*>(p.b + k0);
#pragma unroll
      for (int j = 0; j < kIssB; ++j) dma16_off(base, offb[j], dst + j * 4096);
    } else {
      const char* base = reinterpret_cast<const char*>(p.a + k0);
#pragma unroll
      for (int j = 0; j < kIss; ++j) dma16_off(base, offa[j], dst + j * 4096);
    }
  };

  // Half of the copies of half stage h (the first for even c, the second for
  // odd; h is the B slice 2 i + 5 for c < 2, the A slice 2 i + 6 for c >= 2), for the issue spread over
  // the MFMAs below.  They fill only the two slots freed at this step's
  // barrier, which no wave reads before a later barrier, so they carry no
  // memory clobber: the compiler may keep this step's fragment reads of the
  // other slots where it schedules them (with the clobber it had to finish
  // all of them first and spilled).  The barriers and waits keep theirs.
  auto issue_part = [&](int h, auto cc) {
    constexpr int c = decltype(cc)::value;   // half stage h is a B slice for c < 2
    constexpr bool is_b = c < 2;
    constexpr int per = is_b ? kIssB / 2 : kIss / 2;   // copies per part
    constexpr int part = c & 1;
    if (h >= nh || !issuer) return;
    const uint32_t dst = lds_addr(g_gemm256 + (h % kBSlots) * kBHalfBytes) + (wave & 3) * 1024 + part * per * 4096;
    const char* base = reinterpret_cast<const char*>(is_b ? p.b + (h >> 1) * kBK : p.a + (h >> 1) * kBK);
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const uint32_t off = is_b ? offb[per * part + j] : offa[per * part + j];
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(sgpr(dst + j * 4096))
                   : "m0");
    }
  };
  const int wm = wave >> 2, wn = wave & 3;   // rows 128 wm .., columns 16 kNb wn ..
  const int i16 = lane & 15, g = lane >> 4;
  // fragment of lane l in half q: row l % 16 of a 16-row block, chunk
  // 4 q + l / 16 at its swizzled position
  const uint32_t a_row = (128 * wm + i16) * kBRowBytes;
  const uint32_t b_row = (16 * kNb * wn + i16) * kBRowBytes;
  const uint32_t pos0 = 16 * (g ^ (i16 & 7)), pos1 = 16 * ((4 + g) ^ (i16 & 7));

  const int nk = nh / 2;
  for (int h = 0; h < kBSlots; ++h) issue(h);
  f32x4 acc[8][kNb];
#pragma unroll
  for (int bm = 0; bm < 8; ++bm)
#pragma unroll
    for (int bn = 0; bn < kNb; ++bn) acc[bm][bn] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto read_half = [&](int step, uint32_t pos, bf16x8 (&a)[8], bf16x8 (&b)[kNb]) {
    const char* sa = g_gemm256 + ((2 * step) % kBSlots) * kBHalfBytes + pos;
    const char* sb = g_gemm256 + ((2 * step + 1) % kBSlots) * kBHalfBytes + pos;
#pragma unroll
    for (int t = 0; t < kNb; ++t) b[t] = *reinterpret_cast<const bf16x8*>(sb + b_row + t * 16 * kBRowBytes);
#pragma unroll
    for (int t = 0; t < 8; ++t) a[t] = *reinterpret_cast<const bf16x8*>(sa + a_row + t * 16 * kBRowBytes);
  };
  // D^T blocks: lane (row m = i16, group g) receives C[m][n + 4g + (0..3)]
  auto mfmas = [&](const bf16x8 (&a)[8], const bf16x8 (&b)[kNb]) {
#pragma unroll
    for (int bm = 0; bm < 8; ++bm)
#pragma unroll
      for (int bn = 0; bn < kNb; ++bn) acc[bm][bn] = mfma16x16x32(b[bn], a[bm], acc[bm][bn]);
  };
  // step 0 landed; half stages 2 .. 4 (A, B, A) may fly
  constexpr int kFly3 = 2 * kIss + kIssB;
  wait_vm_upto<kFly3>(!issuer ? 0 : nh >= 5 ? kFly3 : nh == 4 ? kIss + kIssB : 0);
  lds_barrier();
  bf16x8 a0[8], b0[kNb], a1[8], b1[kNb];
  read_half(0, pos0, a0, b0);
  for (int i = 0; i < nk; ++i) {
    read_half(i, pos1, a1, b1);
    mfmas(a0, b0);
    if (i + 1 < nk) {
      // step i + 1 landed (half stage 2 i + 4 may fly); every wave is past
      // its reads of step i, whose slots take half stages 2 i + 5 and 2 i + 6
      wait_vm_upto<kIss>(issuer && 2 * i + 4 < nh ? kIss : 0);   // half stage 2 i + 4 is an A slice
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();
      read_half(i + 1, pos0, a0, b0);
    }
    // The 16 copies of half stages 2 i + 5 and 2 i + 6 (none past the last
    // step) in four groups, each ahead of 8 of the second half's MFMAs: a
    // copy holds its wave until the CU's address path takes it, and spread
    // this way those stalls overlap the wave's MFMAs in flight (q_b 164 ->
    // 158 us in the kernel trace, bit-identical).
    auto group = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      issue_part(2 * i + 5 + (c >> 1), cc);
#pragma unroll
      for (int bm = 2 * c; bm < 2 * c + 2; ++bm)
#pragma unroll
        for (int bn = 0; bn < kNb; ++bn) acc[bm][bn] = mfma16x16x32(b1[bn], a1[bm], acc[bm][bn]);
    };
    group(std::integral_constant<int, 0>{});
    group(std::integral_constant<int, 1>{});
    group(std::integral_constant<int, 2>{});
    group(std::integral_constant<int, 3>{});
  }

  store_tile_staged<ROPE, OUT_F32, BN>(p, acc, m0, n0, wm, wn, i16, g);
}

// cos / sin of the q RoPE angles, one thread per (row, pair): the angle is
// the f32 product of the position and the pair's inverse frequency, its
// cos and sin are taken in double (the accurate device routine: positions
// reach 2^17 and beyond, where a hardware approximation loses the angle) and
// rounded to f32.
__global__ __launch_bounds__(256) void rope_table_kernel(GemmNT p, float2* __restrict__ cs) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(p.m) * 32) return;
  const int m = static_cast<int>(i >> 5), q = static_cast<int>(i & 31);
  if (q >= kDr / 2) return;
  const double pos = static_cast<double>(p.off[m / p.tokens] + m % p.tokens);
  const float ang = static_cast<float>(pos * static_cast<double>(p.inv[q]));
  double sn, c;
  sincos(static_cast<double>(ang), &sn, &c);
  cs[i] = make_float2(static_cast<float>(c), static_cast<float>(sn));
}

}  // namespace

hipError_t launch_rope_table(const GemmNT& p, float2* cs, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(p.m) * 32;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, p, cs);
  return hipGetLastError();
}

bool gemm_nt_mfma_ok(const void* a, int64_t lda, const void* b, int64_t ldb, const void* c, int64_t ldc, int64_t m,
                     int64_t n, int64_t k) {
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  return al(a) && al(b) && al(c) && k % kGK == 0 && k > 0 && lda % 8 == 0 && ldb % 8 == 0 && ldc % 4 == 0 &&
         n % 4 == 0 && m > 0 && n > 0 && (m + kGT - 1) / kGT * ((n + kGT - 1) / kGT) < 0x7fffffffLL;
}

hipError_t launch_gemm_nt_mfma(const GemmNT& p0, bool rope, bool out_f32, hipStream_t stream) {
  GemmNT p = p0;
  // 256 x 256 tiles (one workgroup per CU) when they fill every CU and need
  // no more rounds, in 128 x 128 tile units per CU, than 128 x 128 tiles at
  // two workgroups per CU; the latter otherwise (e.g. 384 big tiles = 1.5
  // rounds).
  const int64_t big = ((p.m + kBT - 1) / kBT) * static_cast<int64_t>((p.n + kBT - 1) / kBT);
  const int64_t small = ((p.m + kGT - 1) / kGT) * static_cast<int64_t>((p.n + kGT - 1) / kGT);
  const int64_t cost_big = (big + 255) / 256 * 4, cost_small = (small + 511) / 512 * 2;
  // the 256 x 256 kernel addresses its copies with 32-bit offsets
  const bool spans32 = static_cast<int64_t>(p.m) * p.lda * 2 < (int64_t{1} << 32) &&
                       static_cast<int64_t>(p.n) * p.ldb * 2 < (int64_t{1} << 32);
  // 256 x 192 tiles (3 units) for the fp32 product (o_proj) where they need
  // fewer rounds than 256 x 256 and no more than 128 x 128 (o_proj at
  // 4096 x 6144: 512 tiles, two whole rounds, against 1.5 rounds of
  // 256 x 256).
  const int64_t mid = ((p.m + kBT - 1) / kBT) * static_cast<int64_t>((p.n + 191) / 192);
  const int64_t cost_mid = (mid + 255) / 256 * 3;
  const bool use_mid = out_f32 && !rope && mid >= 256 && cost_mid < cost_big && cost_mid <= cost_small;
  if (p.k % kBK == 0 && spans32 && use_mid) {
    p.m_tiles = (p.m + kBT - 1) / kBT;
    p.n_tiles = (p.n + 191) / 192;
    hipLaunchKernelGGL((gemm256_nt_kernel<false, true, 192>), dim3(p.m_tiles * p.n_tiles), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  if (p.k % kBK == 0 && big >= 256 && cost_big <= cost_small && spans32) {
    p.m_tiles = (p.m + kBT - 1) / kBT;
    p.n_tiles = (p.n + kBT - 1) / kBT;
    const dim3 grid(p.m_tiles * p.n_tiles);
    if (rope)
      hipLaunchKernelGGL((gemm256_nt_kernel<true, false, 256>), grid, dim3(512), 0, stream, p);
    else if (out_f32)
      hipLaunchKernelGGL((gemm256_nt_kernel<false, true, 256>), grid, dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm256_nt_kernel<false, false, 256>), grid, dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  p.m_tiles = (p.m + kGT - 1) / kGT;
  p.n_tiles = (p.n + kGT - 1) / kGT;
  const dim3 grid(p.m_tiles * p.n_tiles);
  if (rope)
    hipLaunchKernelGGL((gemm_nt_mfma_kernel<true, false>), grid, dim3(256), 0, stream, p);
  else if (out_f32)
    hipLaunchKernelGGL((gemm_nt_mfma_kernel<false, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_nt_mfma_kernel<false, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla

namespace mla {
namespace {

// fp32 -> bf16 (round to nearest even), 4 elements per thread per step.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y,
                                                          int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      const float4 v = *reinterpret_cast<const float4*>(x + i);
      const uint32_t lo = f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
      const uint32_t hi = f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
      *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
    } else {
      for (int64_t j = i; j < n; ++j) y[j] = f32_to_bf16(x[j]);
    }
  }
}

}  // namespace

hipError_t launch_f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 1023) / 1024, 4096);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

}  // namespace mla
