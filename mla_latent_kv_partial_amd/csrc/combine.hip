// Merge of split-T decode partials: the exact log-sum-exp decomposition of
// the page's per-head softmax (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// attendAbsorbed).  For row b, head h over its n_b splits:
//   LSE = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) o_s.
// One workgroup per (head, row): the split weights are formed once in LDS.
// The partials of one (row, head) are contiguous [n_b, r] fp32; the workgroup
// is two groups of 128 threads, group j summing the splits s = j (mod 2) for
// four consecutive latent features per thread (one 16-byte load per split),
// eight splits in flight per thread; the two sums meet in LDS.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = 2;
constexpr int kGroupThreads = kThreads / kGroups;
constexpr int kMaxSplitsLds = 4096;
constexpr int kUnroll = 8;

__device__ __forceinline__ float split_weight(float v, float m) {
  return (m == -INFINITY || v == -INFINITY) ? 0.f : expf(v - m);
}

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const float* po = p.part_o + bh * p.s_max * p.r;
  __shared__ float w_s[kMaxSplitsLds];
  __shared__ float red[kThreads / kWave];
  __shared__ float4 half_s[kGroupThreads];

  float m = -INFINITY;
  for (int s = tid; s < n; s += kThreads) m = fmaxf(m, lse_in[s]);
  m = block_reduce(m, MaxOp(), red);
  float part = 0.f;
  for (int s = tid; s < n; s += kThreads) {
    const float w = split_weight(lse_in[s], m);
    if (s < kMaxSplitsLds) w_s[s] = w;
    part += w;
  }
  const float tot = block_reduce(part, SumOp(), red);   // publishes w_s
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const bool vec = (p.r & 3) == 0 && (reinterpret_cast<uintptr_t>(po) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.o_lat + bh * p.r) & 15) == 0 && n <= kMaxSplitsLds;
  if (vec) {
    const int grp = tid / kGroupThreads, gt = tid % kGroupThreads;
    for (int c0 = 0; c0 < p.r; c0 += 4 * kGroupThreads) {
      const int c = c0 + 4 * gt;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < p.r) {
        int s = grp;
        for (; s + kGroups * (kUnroll - 1) < n; s += kGroups * kUnroll) {
          float4 v[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            v[u] = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s + kGroups * u) * p.r + c);
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const float w = w_s[s + kGroups * u];
            if (w != 0.f) {   // a split with no valid token holds o = 0, lse = -inf
              acc.x = fmaf(w, v[u].x, acc.x); acc.y = fmaf(w, v[u].y, acc.y);
              acc.z = fmaf(w, v[u].z, acc.z); acc.w = fmaf(w, v[u].w, acc.w);
            }
          }
        }
        for (; s < n; s += kGroups) {
          const float w = w_s[s];
          if (w != 0.f) {
            const float4 v = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s) * p.r + c);
            acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
            acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
          }
        }
      }
      if (grp == 1) half_s[gt] = acc;
      __syncthreads();
      if (grp == 0 && c < p.r) {
        const float4 o = half_s[gt];
        *reinterpret_cast<float4*>(p.o_lat + bh * p.r + c) =
            make_float4((acc.x + o.x) * inv, (acc.y + o.y) * inv, (acc.z + o.z) * inv, (acc.w + o.w) * inv);
      }
      __syncthreads();
    }
  } else {
    for (int c = tid; c < p.r; c += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < n; ++s) {
        const float w = s < kMaxSplitsLds ? w_s[s] : split_weight(lse_in[s], m);
        if (w != 0.f) acc = fmaf(w, po[static_cast<int64_t>(s) * p.r + c], acc);
      }
      p.o_lat[bh * p.r + c] = acc * inv;
    }
  }
  if (p.lse && tid == 0) p.lse[bh] = tot > 0.f ? m + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(p.heads, p.rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
