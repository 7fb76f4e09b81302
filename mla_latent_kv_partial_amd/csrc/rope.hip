// Partial interleaved RoPE (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// partialInterleavedRopeMlx), one wave per row vector; the per-vector
// arithmetic is rope_vector.
#include "common.hpp"
#include "launch.hpp"
#include "rope_dev.hpp"

namespace mla {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (vec >= static_cast<int64_t>(p.tokens) * p.inner * p.rows) return;
  rope_vector<T>(p, vec, lane);
}

}  // namespace

hipError_t launch_rope(int32_t dtype, const RopeParams& p, hipStream_t stream) {
  const int64_t vecs = static_cast<int64_t>(p.rows) * p.tokens * p.inner;
  if (vecs == 0) return hipSuccess;
  const int per_block = 256 / kWave;
  const int64_t blocks = (vecs + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dtype == kBF16)
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rope_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
