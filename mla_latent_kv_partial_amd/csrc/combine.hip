// Merge of split-T decode partials: the exact log-sum-exp decomposition of
// the page's per-head softmax (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// attendAbsorbed).  For row b, head h over its n_b splits:
//   LSE = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) o_s.
// One workgroup of 512 threads per (head, row).  The partials of one
// (row, head) are contiguous [n_b, r] fp32.  Four groups of 128 threads split
// the splits (group j takes s = j mod 4); a thread owns four consecutive
// latent features (one 16-byte load per split) and loads 16 splits at a
// time.  The first 16 loads of every thread are issued before the split
// weights are known, so their latency overlaps the log-sum-exp reduction,
// which runs as one (max, sum) pair per thread, wave shuffles and a single
// LDS exchange; the split weights are then formed once each, in LDS.  The
// four group sums meet in LDS.
//
// With a value projection (mla_decode_combine_v) the merged latent context of
// the (head, row) stays in LDS and the same workgroup projects it through the
// head's value block ([P1] attendAbsorbed: ctx_h = o_lat_h . W_UV[h]^T).  For
// bf16 weights with r a multiple of 64 up to 512 and dv <= 128, eight threads
// share one output column: each reads 16-byte pieces of the column's weight
// row (the eight together read 128 contiguous bytes per load), and the eight
// partial dot products meet by lane shuffles.  Workgroup ids run head
// fastest, so with a head count divisible by 8 every row of one head lands on
// the same XCD and its weight block is fetched from HBM once.
#include <math.h>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kGroups = 4;
constexpr int kGroupThreads = kThreads / kGroups;
constexpr int kUnroll = 16;
constexpr int kMaxSplitsLds = 4096;
constexpr int kMaxRankLds = 1024;    // latent context kept in LDS for the projection

// Value projection after the merge: none, any weight dtype (one thread per
// output column), or the bf16 fast path (eight threads per column).
enum VMode : int { kVNone = 0, kVGeneric = 1, kVFastBf16 = 2 };
constexpr int kFastCols = kThreads / 8;   // output columns per pass of the fast path
constexpr int kFastPasses = 2;            // dv <= 128
constexpr int kFastLoads = 8;             // r / 64 <= 8

// (m, l) with l = sum exp(v - m) over the values seen; m = -inf means none.
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;
  l = (m == -INFINITY ? 0.f : l * expf(m - mx)) + (m2 == -INFINITY ? 0.f : l2 * expf(m2 - mx));
  m = mx;
}

__device__ __forceinline__ float split_weight(float v, float m) {
  return (m == -INFINITY || v == -INFINITY) ? 0.f : expf(v - m);
}

// Four consecutive partial features as fp32: one 16-byte load of fp32
// partials, or one 8-byte load of bf16 partials (widened exactly).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// a split with no valid token (weight 0) adds nothing, whatever its partial holds
__device__ __forceinline__ void fma4(float4& acc, float w, const float4& v) {
  if (w == 0.f) return;
  acc.x = fmaf(w, v.x, acc.x);
  acc.y = fmaf(w, v.y, acc.y);
  acc.z = fmaf(w, v.z, acc.z);
  acc.w = fmaf(w, v.w, acc.w);
}

// Two workgroups per CU (at most 128 VGPRs): the (head, row) grid of a decode
// step then runs in one round.
// PT: the partials' storage type (float, or uint16_t for bf16 bits).
template <typename PT, bool VEC, int VM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void combine_kernel(CombineParams p) {
  constexpr int kU = kUnroll;   // batch of partial loads per thread
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const PT* po = static_cast<const PT*>(p.part_o) + bh * p.s_max * p.r;
  __shared__ float red_m[kWaves], red_l[kWaves];
  __shared__ float ws[kMaxSplitsLds];   // split lse, then split weights
  __shared__ float4 grp_s[kGroups - 1][kGroupThreads];
  __shared__ __attribute__((aligned(16))) float o_sh[VM != kVNone ? kMaxRankLds : 1];   // merged o_lat

  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);
  const int gt = tid % kGroupThreads;

  // Fast projection: this thread's weight pieces.  Thread (jj, q) of column
  // j = jj + 64 pass reads elements 8 (8u + q) .. +8 of the column's weight
  // row; columns past dv read the last column (never stored).  They are
  // requested after the merge (the weight block of a head is shared by the
  // rows' workgroups on one XCD, mostly from L2), so the merge keeps its
  // registers for partial loads.
  f32x4 wv[kFastPasses][kFastLoads];
  const int fq = tid & 7, fjj = tid >> 3;
  auto load_weights = [&]() {
    const uint16_t* w = static_cast<const uint16_t*>(p.w);
    const int nu = p.r / 64;
#pragma unroll
    for (int ps = 0; ps < kFastPasses; ++ps) {
      const int j = min(fjj + kFastCols * ps, p.dv - 1);
      const uint16_t* row = w + (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + j) * p.r;
#pragma unroll
      for (int u = 0; u < kFastLoads; ++u)
        if (u < nu) wv[ps][u] = *reinterpret_cast<const f32x4*>(row + 8 * (8 * u + fq));
    }
  };

  // The thread's first split lse is requested first, then the first batch of
  // partials of the first feature block: the lse reduction waits only for the
  // former, the partial loads stay in flight through it.
  const float lse0_raw = lse_in[min(tid, n - 1)];
  asm volatile("" ::: "memory");
  float4 v0[kU];
  if (VEC) {
    // clamped to a valid split and feature (n >= 1): a value past either end
    // is loaded but never used, which keeps the loads free of branches
    const int c = min(4 * gt, p.r - 4);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = min(grp + kGroups * u, n - 1);
      v0[u] = load4(po + static_cast<int64_t>(s) * p.r + c);
    }
  }

  // ---- LSE over the splits: per-thread (max, sum) pairs, then waves, then
  // LDS; the split lse values are kept in LDS for the weights
  const float lse0 = tid < n ? lse0_raw : -INFINITY;
  float m = lse0, l = lse0 == -INFINITY ? 0.f : 1.f;
  if (tid < n && tid < kMaxSplitsLds) ws[tid] = lse0;
  for (int s = tid + kThreads; s < n; s += kThreads) {
    const float x = lse_in[s];
    if (s < kMaxSplitsLds) ws[s] = x;
    lse_merge(m, l, x, 1.f);
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave), l2 = __shfl_xor(l, off, kWave);
    lse_merge(m, l, m2, l2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_l[wave] = l;
  }
  __syncthreads();
  m = red_m[0];
  l = red_l[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) lse_merge(m, l, red_m[w], red_l[w]);
  // each thread turns the lse values it stored into weights; beyond the LDS
  // copy the weights are formed where they are used
  if (tid < n && tid < kMaxSplitsLds) ws[tid] = split_weight(lse0, m);
  for (int s = tid + kThreads; s < min(n, kMaxSplitsLds); s += kThreads) ws[s] = split_weight(ws[s], m);
  __syncthreads();
  auto weight = [&](int s) { return s < kMaxSplitsLds ? ws[s] : split_weight(lse_in[s], m); };
  const float inv = l > 0.f ? 1.f / l : 0.f;

  if (VEC) {
    for (int c0 = 0; c0 < p.r; c0 += 4 * kGroupThreads) {
      const bool own = c0 + 4 * gt < p.r;
      const int c = min(c0 + 4 * gt, p.r - 4);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      // whole batches of kU splits per thread, loads clamped as above;
      // the first batch of the first feature block is already in flight
      for (int s = grp; s < n; s += kGroups * kU) {
        if (c0 > 0 || s > grp) {
#pragma unroll
          for (int u = 0; u < kU; ++u)
            v0[u] = load4(po + static_cast<int64_t>(min(s + kGroups * u, n - 1)) * p.r + c);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (s + kGroups * u < n) fma4(acc, weight(s + kGroups * u), v0[u]);
      }
      if (grp > 0) grp_s[grp - 1][gt] = acc;
      __syncthreads();
      if (grp == 0 && own) {
#pragma unroll
        for (int j = 0; j < kGroups - 1; ++j) {
          const float4 o = grp_s[j][gt];
          acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
        }
        const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        if (p.o_lat) *reinterpret_cast<float4*>(p.o_lat + bh * p.r + c) = o;
        if constexpr (VM != kVNone) *reinterpret_cast<float4*>(o_sh + c) = o;
      }
      __syncthreads();
    }
  } else {
    for (int c = tid; c < p.r; c += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < n; ++s) {
        const float w = weight(s);
        if (w != 0.f) acc = fmaf(w, ld(po + static_cast<int64_t>(s) * p.r + c), acc);
      }
      if (p.o_lat) p.o_lat[bh * p.r + c] = acc * inv;
      if constexpr (VM != kVNone) o_sh[c] = acc * inv;
    }
  }
  if (p.lse && tid == 0) p.lse[bh] = l > 0.f ? m + logf(l) : -INFINITY;
  if constexpr (VM == kVNone) return;
  __syncthreads();   // o_sh complete

  // ---- value projection: ctx[b, h dv + j] = sum_c o_lat[c] W_UV[h][j][c]
  float* ctx = p.ctx + static_cast<int64_t>(b) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv;
  if constexpr (VM == kVFastBf16) {
    load_weights();
    const int nu = p.r / 64;
#pragma unroll
    for (int ps = 0; ps < kFastPasses; ++ps) {
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < kFastLoads; ++u) {
        if (u < nu) {
          const float4* o4 = reinterpret_cast<const float4*>(o_sh + 8 * (8 * u + fq));
          const float4 o0 = o4[0], o1 = o4[1];
          const f32x4 wb = wv[ps][u];   // 8 bf16: element 2i in the low half of word i
          const uint32_t w0 = __float_as_uint(wb[0]), w1 = __float_as_uint(wb[1]);
          const uint32_t w2 = __float_as_uint(wb[2]), w3 = __float_as_uint(wb[3]);
          acc = fmaf(o0.x, __uint_as_float(w0 << 16), acc);
          acc = fmaf(o0.y, __uint_as_float(w0 & 0xffff0000u), acc);
          acc = fmaf(o0.z, __uint_as_float(w1 << 16), acc);
          acc = fmaf(o0.w, __uint_as_float(w1 & 0xffff0000u), acc);
          acc = fmaf(o1.x, __uint_as_float(w2 << 16), acc);
          acc = fmaf(o1.y, __uint_as_float(w2 & 0xffff0000u), acc);
          acc = fmaf(o1.z, __uint_as_float(w3 << 16), acc);
          acc = fmaf(o1.w, __uint_as_float(w3 & 0xffff0000u), acc);
        }
      }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      acc += __shfl_xor(acc, 4, kWave);
      const int j = fjj + kFastCols * ps;
      if (fq == 0 && j < p.dv) ctx[j] = acc;
    }
  } else {
    for (int j = tid; j < p.dv; j += kThreads) {
      const int64_t row = (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + j) * p.r;
      float acc = 0.f;
      if (p.w_dtype == kBF16) {
        const uint16_t* w = static_cast<const uint16_t*>(p.w) + row;
        for (int c = 0; c < p.r; ++c) acc = fmaf(o_sh[c], bf16_to_f32(w[c]), acc);
      } else {
        const float* w = static_cast<const float*>(p.w) + row;
        for (int c = 0; c < p.r; ++c) acc = fmaf(o_sh[c], w[c], acc);
      }
      ctx[j] = acc;
    }
  }
}

template <typename PT>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  // whole 4-feature partial groups from aligned bases (16 bytes fp32, 8 bf16)
  const uintptr_t pa = reinterpret_cast<uintptr_t>(p.part_o) & (4 * sizeof(PT) - 1);
  const bool vec = p.r >= 4 && (p.r & 3) == 0 && pa == 0 && (reinterpret_cast<uintptr_t>(p.o_lat) & 15) == 0;
  const dim3 grid(p.heads, p.rows), block(kThreads);
  if (!p.ctx) {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<PT, true, kVNone>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((combine_kernel<PT, false, kVNone>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  const bool fast = vec && p.w_dtype == kBF16 && p.r % 64 == 0 && p.r / 64 <= kFastLoads &&
                    p.dv <= kFastCols * kFastPasses && (reinterpret_cast<uintptr_t>(p.w) & 15) == 0;
  if (fast)
    hipLaunchKernelGGL((combine_kernel<PT, true, kVFastBf16>), grid, block, 0, stream, p);
  else if (vec)
    hipLaunchKernelGGL((combine_kernel<PT, true, kVGeneric>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((combine_kernel<PT, false, kVGeneric>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  return p.part_bf16 ? launch_combine_t<uint16_t>(p, stream) : launch_combine_t<float>(p, stream);
}

}  // namespace mla
