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
#include <math.h>

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

// a split with no valid token (weight 0) adds nothing, whatever its partial holds
__device__ __forceinline__ void fma4(float4& acc, float w, const float4& v) {
  if (w == 0.f) return;
  acc.x = fmaf(w, v.x, acc.x);
  acc.y = fmaf(w, v.y, acc.y);
  acc.z = fmaf(w, v.z, acc.z);
  acc.w = fmaf(w, v.w, acc.w);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const float* po = p.part_o + bh * p.s_max * p.r;
  __shared__ float red_m[kWaves], red_l[kWaves];
  __shared__ float ws[kMaxSplitsLds];   // split lse, then split weights
  __shared__ float4 grp_s[kGroups - 1][kGroupThreads];

  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);
  const int gt = tid % kGroupThreads;

  // The thread's first split lse is requested first, then the first batch of
  // partials of the first feature block: the lse reduction waits only for the
  // former, the partial loads stay in flight through it.
  const float lse0_raw = lse_in[min(tid, n - 1)];
  asm volatile("" ::: "memory");
  float4 v0[kUnroll];
  if (VEC) {
    // clamped to a valid split and feature (n >= 1): a value past either end
    // is loaded but never used, which keeps the loads free of branches
    const int c = min(4 * gt, p.r - 4);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = min(grp + kGroups * u, n - 1);
      v0[u] = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s) * p.r + c);
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
      // whole batches of kUnroll splits per thread, loads clamped as above;
      // the first batch of the first feature block is already in flight
      for (int s = grp; s < n; s += kGroups * kUnroll) {
        if (c0 > 0 || s > grp) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            v0[u] = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(min(s + kGroups * u, n - 1)) * p.r + c);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
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
        *reinterpret_cast<float4*>(p.o_lat + bh * p.r + c) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      }
      __syncthreads();
    }
  } else {
    for (int c = tid; c < p.r; c += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < n; ++s) {
        const float w = weight(s);
        if (w != 0.f) acc = fmaf(w, po[static_cast<int64_t>(s) * p.r + c], acc);
      }
      p.o_lat[bh * p.r + c] = acc * inv;
    }
  }
  if (p.lse && tid == 0) p.lse[bh] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  // 16-byte partial rows: r a multiple of 4 from 16-byte aligned bases
  const bool vec = p.r >= 4 && (p.r & 3) == 0 && (reinterpret_cast<uintptr_t>(p.part_o) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.o_lat) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(p.heads, p.rows), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(p.heads, p.rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
