// Fused cache append (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts:
// Glm52Mla.project splits the kv_a_proj_with_mqa output into the latent part
// and the rope part; rmsNormF32Mlx normalises the latent with the
// kv_a_layernorm weight; partialInterleavedRopeMlx rotates the rope part at the
// row's position; Glm52Mla.forward appends both to the cache).
//
// One wave per (row, token): the latent's mean square is a wave reduction in
// fp32 (as the page computes it), x * (1 / sqrt(mean + eps)) * w is rounded
// once to the cache type; the rope pairs are rotated exactly as the RoPE entry
// does (f32 angle from the host's inverse-frequency table, cos/sin and the
// rotation in double).  Writes latent[b, slot + t, :] and rope[b, slot + t, :].
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (vec >= static_cast<int64_t>(p.rows) * p.tokens) return;
  const int b = static_cast<int>(vec / p.tokens);
  const int t = static_cast<int>(vec - static_cast<int64_t>(b) * p.tokens);
  const T* x = static_cast<const T*>(p.kv_a) + b * p.kb + t * p.kt;
  const T* w = static_cast<const T*>(p.w);
  T* lat = static_cast<T*>(p.latent) + b * p.lb + static_cast<int64_t>(p.slot + t) * p.lt;
  T* rope = static_cast<T*>(p.rope) + b * p.rb + static_cast<int64_t>(p.slot + t) * p.rt;

  float ss = 0.f;
  for (int c = lane; c < p.r; c += kWave) {
    const float v = ld(x + c);
    ss = fmaf(v, v, ss);
  }
  ss = wave_reduce(ss, SumOp());
  const float inv = 1.f / sqrtf(ss / static_cast<float>(p.r) + p.eps);
  for (int c = lane; c < p.r; c += kWave) st(lat + c, static_cast<double>(ld(x + c) * inv * ld(w + c)));

  const int half = p.dr / 2;
  const double pos = static_cast<double>(p.off[b] + t);
  for (int q = lane; q < half; q += kWave) {
    const double a = ld(x + p.r + 2 * q), bb = ld(x + p.r + 2 * q + 1);
    const float ang = static_cast<float>(pos * static_cast<double>(p.inv[q]));
    double s, c;
    sincos(static_cast<double>(ang), &s, &c);
    st(rope + q, a * c - bb * s);
    st(rope + half + q, bb * c + a * s);
  }
}

}  // namespace

hipError_t launch_append(int32_t dtype, const AppendParams& p, hipStream_t stream) {
  const int64_t vecs = static_cast<int64_t>(p.rows) * p.tokens;
  if (vecs == 0) return hipSuccess;
  const int64_t blocks = (vecs + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dtype == kBF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(append_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
