// Merge of split-T decode partials: the exact log-sum-exp decomposition of
// the page's per-head softmax (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// attendAbsorbed).  For row b, head h over its n_b splits:
//   LSE = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) o_s.
// One workgroup per (head, row): the split weights are formed once in LDS,
// then each thread owns latent features and streams the partials, which are
// contiguous per (b, h).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplitsLds = 2048;

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const float* po = p.part_o + bh * p.s_max * p.r;
  __shared__ float w_s[kMaxSplitsLds];
  __shared__ float red[kThreads / kWave];

  float m = -INFINITY;
  for (int s = tid; s < n; s += kThreads) m = fmaxf(m, lse_in[s]);
  m = block_reduce(m, MaxOp(), red);
  float part = 0.f;
  for (int s = tid; s < n; s += kThreads) {
    const float v = lse_in[s];
    const float w = (m == -INFINITY || v == -INFINITY) ? 0.f : expf(v - m);
    if (s < kMaxSplitsLds) w_s[s] = w;
    part += w;
  }
  const float tot = block_reduce(part, SumOp(), red);   // publishes w_s
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  for (int c = tid; c < p.r; c += kThreads) {
    float acc = 0.f;
    for (int s = 0; s < n; ++s) {
      float w;
      if (s < kMaxSplitsLds) {
        w = w_s[s];
      } else {
        const float v = lse_in[s];
        w = (m == -INFINITY || v == -INFINITY) ? 0.f : expf(v - m);
      }
      if (w != 0.f) acc = fmaf(w, po[static_cast<int64_t>(s) * p.r + c], acc);
    }
    p.o_lat[bh * p.r + c] = acc * inv;
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
