// MFMA NT GEMM for bf16 operands (both K-contiguous), fp32 accumulation,
// bf16 or fp32 result.  Serves the prefill projections of page "mlx-bun
// 0.0.11 -> 0.0.13", glm52-mla.ts (q_b_proj with the q RoPE of
// Glm52Mla.project as an epilogue; the kv_b_proj expansion of
// attendReconstructed) and the o_proj linear after the attention.
#include <math.h>

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

// A wave's output blocks: block (bm, bn) lane (i16, g) holds row
// m_base + 16 bm + i16, columns n_base + 16 bn + 4 g .. +3.  n_base is a
// multiple of 64 and the wave spans at most 64 columns, so with ROPE (the q
// projection, 192 columns per head: 128 no-PE, then 64 rope) its columns are
// either all no-PE or all the rope part of one head.  Rope columns are
// rotated at the row's position and written as split halves: columns
// (v0, v1) and (v2, v3) are rope pairs q0 and q0 + 1 of the head, cos and sin
// come from the row's table in double.  The table entries of row block bm + 1
// are requested before block bm is rotated, so their latency overlaps.
template <bool ROPE, bool OUT_F32, int BM, int BN>
__device__ __forceinline__ void store_tile(const GemmNT& p, const f32x4 (&acc)[BM][BN], int m_base, int n_base,
                                           int i16, int g) {
  static_assert(16 * BN <= 64, "a wave spans at most 64 columns");
  if (ROPE && n_base % kQk >= kDn) {
    const int head_col = n_base - n_base % kQk;           // first column of the head
    const int q_lane = (n_base % kQk - kDn) / 2 + 2 * g;  // pair of column n_base + 4 g
    double2 cur[BN][2], nxt[BN][2];
    auto load = [&](double2 (&t)[BN][2], int bm) {
      const int m = min(m_base + 16 * bm + i16, p.m - 1);
      const double2* cs = p.cs + static_cast<int64_t>(m) * 32 + q_lane;
#pragma unroll
      for (int bn = 0; bn < BN; ++bn) {
        t[bn][0] = cs[8 * bn];
        t[bn][1] = cs[8 * bn + 1];
      }
    };
    load(cur, 0);
#pragma unroll
    for (int bm = 0; bm < BM; ++bm) {
      if (bm + 1 < BM) load(nxt, bm + 1);
      const int m = m_base + 16 * bm + i16;
      if (m < p.m) {
        uint16_t* head = static_cast<uint16_t*>(p.c) + static_cast<int64_t>(m) * p.ldc + head_col + kDn;
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) {
          if (n_base + 16 * bn + 4 * g >= p.n) continue;
          const int q0 = q_lane + 8 * bn;
          uint16_t re[2], im[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const double2 t = cur[bn][e];
            const double a = acc[bm][bn][2 * e], b = acc[bm][bn][2 * e + 1];
            re[e] = f64_to_bf16(a * t.x - b * t.y);
            im[e] = f64_to_bf16(b * t.x + a * t.y);
          }
          *reinterpret_cast<uint32_t*>(head + q0) = re[0] | (static_cast<uint32_t>(re[1]) << 16);
          *reinterpret_cast<uint32_t*>(head + kDr / 2 + q0) = im[0] | (static_cast<uint32_t>(im[1]) << 16);
        }
      }
      if (bm + 1 < BM) {
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) {
          cur[bn][0] = nxt[bn][0];
          cur[bn][1] = nxt[bn][1];
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
// (8 x 4 MFMA blocks), K step 32 through a 4-stage LDS ring, three steps in
// flight.  A 16-row block of an operand tile is 1 KB: row r (64 bytes, four
// 16-byte chunks) at 64 r, chunk c stored at position c ^ ((r >> 2) & 3).
// Each copy instruction fills one block with four lanes per row, so the
// global reads coalesce into whole 64-byte row segments; the XOR spreads the
// fragment reads (16 rows, one chunk each) over the banks.  Relative to the
// 128 x 128 tile this halves the operand bytes per FLOP that reach the CU.
// (Measured: chunk-major blocks read by single lanes per row, which need no
// swizzle, were 12 % slower from the uncoalesced copies; a deeper 5-stage
// ring and register-staged copies were no faster.)
constexpr int kBT = 256;
constexpr int kBK = 32;
constexpr int kBOpBytes = kBT * kBK * 2;            // 16 KB per operand tile
constexpr int kBStageBytes = 2 * kBOpBytes;         // A tile then B tile
constexpr int kBStages = 4;
constexpr int kBCopies = kBStageBytes / 1024 / 8;   // 1 KB copies per wave per stage (4)

__shared__ __attribute__((aligned(1024))) char g_gemm256[kBStages * kBStageBytes];

// chunk swizzle of row r of a 16-row block
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

template <bool ROPE, bool OUT_F32>
__global__ __launch_bounds__(512) void gemm256_nt_kernel(GemmNT p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int m0 = (tile % p.m_tiles) * kBT;
  const int n0 = (tile / p.m_tiles) * kBT;

  // copy plan: copy j of this wave fills 16-row block q = wave + 8 j of the
  // stage (blocks 0..15 of A, 16..31 of B); lane l lands at position l of the
  // block: row l / 4, chunk (l % 4) ^ swz(l / 4).  Rows past the matrix edge
  // re-read its last row.
  const uint16_t* src[kBCopies];
#pragma unroll
  for (int j = 0; j < kBCopies; ++j) {
    const int q = wave + 8 * j;
    const int r16 = lane >> 2;
    const int row = 16 * (q & 15) + r16;
    const int c = (lane & 3) ^ swz(r16);
    src[j] = q < 16 ? p.a + static_cast<int64_t>(min(m0 + row, p.m - 1)) * p.lda + 8 * c
                    : p.b + static_cast<int64_t>(min(n0 + row, p.n - 1)) * p.ldb + 8 * c;
  }
  auto issue = [&](int s, int k0) {
    const uint32_t dst = lds_addr(g_gemm256 + s * kBStageBytes);
#pragma unroll
    for (int j = 0; j < kBCopies; ++j) dma16(src[j] + k0, dst + (wave + 8 * j) * 1024);
  };

  const int wm = wave >> 2, wn = wave & 3;   // rows 128 wm .., columns 64 wn ..
  const int i16 = lane & 15, g = lane >> 4;
  // fragment of lane l: row l % 16, chunk l / 16 of a block
  const uint32_t lpos = 64 * i16 + 16 * (g ^ swz(i16));
  const uint32_t a_frag = (8 * wm) * 1024 + lpos;
  const uint32_t b_frag = kBOpBytes + (4 * wn) * 1024 + lpos;

  const int nk = p.k / kBK;
  for (int t = 0; t < kBStages - 1 && t < nk; ++t) issue(t, t * kBK);
  f32x4 acc[8][4];
#pragma unroll
  for (int bm = 0; bm < 8; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < nk; ++i) {
    // step i's copies done; those of the (up to two) following steps may fly
    const int later = min(nk - 1 - i, kBStages - 2);
    wait_vm_upto<kBCopies * (kBStages - 2)>(kBCopies * later);
    lds_barrier();
    if (i + kBStages - 1 < nk) issue((i + kBStages - 1) % kBStages, (i + kBStages - 1) * kBK);
    const char* st = g_gemm256 + (i % kBStages) * kBStageBytes;
    bf16x8 af[8], bfr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bfr[t] = *reinterpret_cast<const bf16x8*>(st + b_frag + t * 1024);
#pragma unroll
    for (int t = 0; t < 8; ++t) af[t] = *reinterpret_cast<const bf16x8*>(st + a_frag + t * 1024);
    // D^T blocks: lane (row m = i16, group g) receives C[m][n + 4g + (0..3)]
#pragma unroll
    for (int bm = 0; bm < 8; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = mfma16x16x32(bfr[bn], af[bm], acc[bm][bn]);
  }

  store_tile<ROPE, OUT_F32>(p, acc, m0 + 128 * wm, n0 + 64 * wn, i16, g);
}

// cos / sin of the q RoPE angles, one thread per (row, pair): the angle is
// the f32 product of the position and the pair's inverse frequency, its
// cos and sin are taken in double (the accurate device routine: positions
// reach 2^17 and beyond, where a hardware approximation loses the angle).
__global__ __launch_bounds__(256) void rope_table_kernel(GemmNT p, double2* __restrict__ cs) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(p.m) * 32) return;
  const int m = static_cast<int>(i >> 5), q = static_cast<int>(i & 31);
  if (q >= kDr / 2) return;
  const double pos = static_cast<double>(p.off[m / p.tokens] + m % p.tokens);
  const float ang = static_cast<float>(pos * static_cast<double>(p.inv[q]));
  double sn, c;
  sincos(static_cast<double>(ang), &sn, &c);
  cs[i] = make_double2(c, sn);
}

}  // namespace

hipError_t launch_rope_table(const GemmNT& p, double2* cs, hipStream_t stream) {
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
  if (p.k % kBK == 0 && big >= 256 && cost_big <= cost_small) {
    p.m_tiles = (p.m + kBT - 1) / kBT;
    p.n_tiles = (p.n + kBT - 1) / kBT;
    const dim3 grid(p.m_tiles * p.n_tiles);
    if (rope)
      hipLaunchKernelGGL((gemm256_nt_kernel<true, false>), grid, dim3(512), 0, stream, p);
    else if (out_f32)
      hipLaunchKernelGGL((gemm256_nt_kernel<false, true>), grid, dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm256_nt_kernel<false, false>), grid, dim3(512), 0, stream, p);
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
