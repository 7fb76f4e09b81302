// MFMA weight absorption for bf16 weights (page "mlx-bun 0.0.11 -> 0.0.13",
// glm52-mla.ts, Glm52Mla.attendAbsorbed: W_UK[h] = kv_b rows [h(dn+dv),
// h(dn+dv)+dn), W_UV[h] = the next dv rows; q_lat = q_nope . W_UK,
// ctx = o_lat . W_UV^T).  Both are weight-streaming contractions at decode
// batch sizes: every weight byte is read once and reused for all batch rows.
//
// absorb_q: workgroup = (128-column block of r, head).  W_UK[h][:, block] is
//   [dn x 128] with the output columns contiguous and the contraction (d)
//   strided, so the tile is staged in LDS by global_load_lds_dwordx4 and the
//   d-packed MFMA operand is read with ds_read_b64_tr_b16.  Chunks of a tile
//   row are XOR-swizzled (f(d) below) so those reads are bank-conflict free.
//   q_nope rows (bf16) are the other operand, straight from global memory;
//   q_lat is stored in bf16 (round to nearest even).  A variant also applies
//   the query's RoPE in the same launch (the decode query in one kernel).
// absorb_v: workgroup = (32-column block of dv, head).  The contraction runs
//   along the contiguous latent axis of both o_lat and W_UV, so both operands
//   load directly; the latent axis is split over the 4 waves and the partial
//   sums are added in LDS.  o_lat (fp32) enters as a bf16 high part plus a
//   bf16 residual (two MFMAs), which keeps about 16 bits of its mantissa.
#include <algorithm>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "rope_dev.hpp"

namespace mla {
namespace {

constexpr int kQCols = 128;     // absorb_q output columns per workgroup
constexpr int kVCols = 32;      // absorb_v output columns per workgroup
constexpr int kAvBatch = 8;     // absorb_v K steps whose loads are issued together

__device__ __forceinline__ int swz(int d) { return ((d & 3) << 1) ^ (((d >> 3) & 1) << 3); }

__shared__ __attribute__((aligned(1024))) char g_wtile[256 * kQCols * 2];   // up to dn = 256 rows
__shared__ float g_vsum[8][16][kVCols + 1];   // per wave, up to 8 waves

// ROPE: two waves of each workgroup rotate the query's rope part while the
// other two issue the weight-tile copies, so the rotation hides under the copy
// latency.
template <bool ROPE>
__global__ __launch_bounds__(256) void absorb_q_mfma_kernel(AbsorbQParams p, RopeParams rp) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = blockIdx.x * kQCols;
  const int h = blockIdx.y;
  const int dn = p.dn;
  const uint16_t* w = static_cast<const uint16_t*>(p.w) + (static_cast<int64_t>(h) * (dn + p.dv)) * p.r + c0;
  // Waves 0 and 1 issue the weight-tile copies; with ROPE, waves 2 and 3
  // rotate the query's rope part meanwhile (one wave per (row, head) vector).
  // The rotating waves have no copies in flight, so their wait before the
  // rotated stores (which may alias the loads) covers only their own loads.
  constexpr int kMaxKs = 256 / 32;
  const int m = lane & 15, g = lane >> 4;
  const int nks = dn / 32;
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  bf16x8 qa[kMaxKs];
  // q rows of a 16-row batch block, lane (row m, group g)
  auto load_q = [&](int b0) {
    const int b = b0 + m;
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks)
      if (ks < nks)
        qa[ks] = b < p.batch ? *reinterpret_cast<const bf16x8*>(q + b * p.q_sb + h * p.q_sh + 32 * ks + 8 * g)
                             : bf16x8{};
  };
  if (wave < 2) {
    // ---- stage W_UK[h][0..dn)[c0 .. c0+128): position k = 16 d + s holds chunk s ^ swz(d)
    const int copies = dn * 16 / 64;   // 1 KB each
    const uint32_t dst = lds_addr(g_wtile);
    for (int n = wave; n < copies; n += 2) {
      const int k = 64 * n + lane;
      const int d = k >> 4, s = k & 15;
      dma16(w + static_cast<int64_t>(d) * p.r + 8 * (s ^ swz(d)), dst + n * 1024);
    }
  }
  load_q(0);
  if (ROPE && wave >= 2) {
    const int64_t vecs = static_cast<int64_t>(rp.rows) * rp.tokens * rp.inner;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * gridDim.y * 2;
    for (int64_t v = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * 2 + (wave - 2); v < vecs; v += waves)
      rope_vector<uint16_t>(rp, v, lane);
  }
  wait_vm<0>();
  lds_barrier();
  // ---- wave: output columns c0 + 32 wave + (0..31), two 16-column blocks
  for (int b0 = 0; b0 < p.batch; b0 += 16) {
    if (b0 > 0) load_q(b0);
    f32x4 acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) {
      if (ks >= nks) break;
      const bf16x8 a = qa[ks];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int cc = (32 * wave + 16 * nb) / 8 + ((m & 3) >> 1);
        const int r1 = 32 * ks + 8 * g + (m >> 2);
        const int r2 = r1 + 4;
        const char* t = g_wtile;
        const s16x4 v1 = lds_read_tr16(t + r1 * 256 + ((cc ^ swz(r1)) << 4) + (m & 1) * 8);
        const s16x4 v2 = lds_read_tr16(t + r2 * 256 + ((cc ^ swz(r2)) << 4) + (m & 1) * 8);
        const s16x8 bv = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = mfma16x16x32(a, __builtin_bit_cast(bf16x8, bv), acc[nb]);
      }
    }
    // acc[nb] lane (column m, group g): rows b0 + 4g + i
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bb = b0 + 4 * g + i;
        if (bb < p.batch)
          static_cast<uint16_t*>(p.q_lat)[(static_cast<int64_t>(bb) * p.heads + h) * p.r + c0 + 32 * wave + 16 * nb + m] =
              f32_to_bf16(acc[nb][i]);
      }
  }
}

// NB 16-column blocks per workgroup, of which the first `cols` columns are
// the workgroup's (cols <= 16 NB); NWV waves splitting the latent axis.
template <int NB, int NWV>
__global__ __launch_bounds__(NWV * 64) void absorb_v_mfma_kernel(AbsorbVParams p, int cols) {
  constexpr int kCols = 16 * NB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int v0 = blockIdx.x * cols;
  const int ncol = min(cols, p.dv - v0);   // columns of this workgroup that exist
  const int h = blockIdx.y;
  const int m = lane & 15, g = lane >> 4;
  const int kq = p.r / NWV;                 // latent range of this wave (a multiple of 32)
  const uint16_t* w = static_cast<const uint16_t*>(p.w) +
                      (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + v0) * p.r + wave * kq;
  for (int b0 = 0; b0 < p.batch; b0 += 16) {
    // rows past the batch re-read its last row: their sums are never stored,
    // and the loads need no branch (the compiler then waits for each step's
    // own loads rather than for the whole batch)
    const int bl = min(b0 + m, p.batch - 1);
    const float* o = p.o_lat + (static_cast<int64_t>(bl) * p.heads + h) * p.r + wave * kq;
    f32x4 acc[NB] = {};
    auto step = [&](const float4& uu, const float4& vv, const bf16x8 (&bwu)[NB]) {
      const bf16x8 hi = to_bf16x8(uu, vv);
      const float4 ru = make_float4(uu.x - static_cast<float>(hi[0]), uu.y - static_cast<float>(hi[1]),
                                    uu.z - static_cast<float>(hi[2]), uu.w - static_cast<float>(hi[3]));
      const float4 rv = make_float4(vv.x - static_cast<float>(hi[4]), vv.y - static_cast<float>(hi[5]),
                                    vv.z - static_cast<float>(hi[6]), vv.w - static_cast<float>(hi[7]));
      const bf16x8 lo = to_bf16x8(ru, rv);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb] = mfma16x16x32(hi, bwu[nb], acc[nb]);
        acc[nb] = mfma16x16x32(lo, bwu[nb], acc[nb]);
      }
    };
    // B[k = latent 32ks + 8g .. +8][n = value column 16nb + m]
    auto wload = [&](int ks, int nb) {
      // columns past the workgroup's re-read its last one (never stored)
      const int col = min(16 * nb + m, ncol - 1);
      return *reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(col) * p.r + 32 * ks + 8 * g);
    };
    // kAvBatch K steps per batch: their weight and o_lat loads are all issued
    // before the first MFMA, so each wave keeps up to kAvBatch NB KB of
    // weights in flight
    const int nks = kq / 32;
    const int nfull = nks / kAvBatch * kAvBatch;
    for (int ks0 = 0; ks0 < nfull; ks0 += kAvBatch) {
      bf16x8 bw[kAvBatch][NB];
      float4 ou[kAvBatch], ov[kAvBatch];
#pragma unroll
      for (int u = 0; u < kAvBatch; ++u) {
        ou[u] = *reinterpret_cast<const float4*>(o + 32 * (ks0 + u) + 8 * g);
        ov[u] = *reinterpret_cast<const float4*>(o + 32 * (ks0 + u) + 8 * g + 4);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bw[u][nb] = wload(ks0 + u, nb);
      }
#pragma unroll
      for (int u = 0; u < kAvBatch; ++u) step(ou[u], ov[u], bw[u]);
    }
    for (int ks = nfull; ks < nks; ++ks) {
      bf16x8 bw[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bw[nb] = wload(ks, nb);
      step(*reinterpret_cast<const float4*>(o + 32 * ks + 8 * g), *reinterpret_cast<const float4*>(o + 32 * ks + 8 * g + 4),
           bw);
    }
    // partial sums of this wave: lane (column m, group g) holds rows 4g + i
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) g_vsum[wave][4 * g + i][16 * nb + m] = acc[nb][i];
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * kCols; e += NWV * 64) {
      const int row = e / kCols, col = e % kCols;
      const int bb = b0 + row;
      if (bb < p.batch && col < ncol) {
        float sum = 0.f;
#pragma unroll
        for (int wv = 0; wv < NWV; ++wv) sum += g_vsum[wv][row][col];
        p.ctx[static_cast<int64_t>(bb) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv + v0 + col] = sum;
      }
    }
    __syncthreads();
  }
}

}  // namespace

bool absorb_q_mfma_ok(const AbsorbQParams& p) {
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  return p.dn % 32 == 0 && p.dn <= 256 && p.r % kQCols == 0 && p.q_sb % 8 == 0 && p.q_sh % 8 == 0 && al(p.q) &&
         al(p.w) && p.heads <= 65535;
}

bool absorb_v_mfma_ok(const AbsorbVParams& p) {
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  return p.dv % kVCols == 0 && p.r % 128 == 0 && p.dn % 8 == 0 && al(p.o_lat) && al(p.w) && p.heads <= 65535;
}

hipError_t launch_absorb_q_mfma(const AbsorbQParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_mfma_kernel<false>, dim3(p.r / kQCols, p.heads), dim3(256), 0, stream, p,
                     RopeParams{});
  return hipGetLastError();
}

hipError_t launch_absorb_q_rope_mfma(const AbsorbQParams& p, const RopeParams& rp, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_mfma_kernel<true>, dim3(p.r / kQCols, p.heads), dim3(256), 0, stream, p, rp);
  return hipGetLastError();
}

hipError_t launch_absorb_v_mfma(const AbsorbVParams& p, hipStream_t stream) {
  // 32 columns and 4 waves per workgroup while that fills the CUs; otherwise
  // 8 waves (a long latent axis over few heads, as in o_proj) and 16 to 32
  // columns per workgroup, as many as make the workgroups about one per CU
  // (o_proj to 6144 columns: 384 blocks of 16 left half the CUs with two,
  // 256 blocks of 24 give every CU the same bytes).
  if (static_cast<int64_t>(p.dv / kVCols) * p.heads >= 256 || p.r % (8 * 32) != 0) {
    hipLaunchKernelGGL((absorb_v_mfma_kernel<2, 4>), dim3(p.dv / kVCols, p.heads), dim3(256), 0, stream, p, kVCols);
    return hipGetLastError();
  }
  const int64_t per_cu = (static_cast<int64_t>(p.dv) * p.heads + 255) / 256;
  const int cols = static_cast<int>(std::min<int64_t>(32, std::max<int64_t>(16, (per_cu + 7) / 8 * 8)));
  const dim3 grid(static_cast<uint32_t>((p.dv + cols - 1) / cols), p.heads);
  if (cols <= 16)
    hipLaunchKernelGGL((absorb_v_mfma_kernel<1, 8>), grid, dim3(512), 0, stream, p, cols);
  else
    hipLaunchKernelGGL((absorb_v_mfma_kernel<2, 8>), grid, dim3(512), 0, stream, p, cols);
  return hipGetLastError();
}

}  // namespace mla
