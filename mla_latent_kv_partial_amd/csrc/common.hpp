// Device helpers shared by the MLA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 storage
// bf16 values travel as raw 16-bit patterns; arithmetic is fp32.

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// double -> bf16 with a single rounding: truncate to fp32 and keep a sticky
// bit when inexact (round-to-odd), then round to nearest even.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  float t = __double2float_rz(d);
  uint32_t u = __float_as_uint(t);
  if (static_cast<double>(t) != d && (u & 0x7fffffffu) < 0x7f800000u) u |= 1u;
  return f32_to_bf16(__uint_as_float(u));
}

// Typed load/store of one element of a storage type (float or bf16 bits).
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st(float* p, double v) { *p = static_cast<float>(v); }
__device__ __forceinline__ void st(uint16_t* p, double v) { *p = f64_to_bf16(v); }

// ---------------------------------------------------------------- reductions
template <typename F>
__device__ __forceinline__ float wave_reduce(float v, F op) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
  return v;
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// Block-wide reduction through LDS; every thread receives the result.
// `scratch` must hold blockDim.x / 64 floats; the call contains barriers.
template <typename F>
__device__ __forceinline__ float block_reduce(float v, F op, float* scratch) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves = blockDim.x / kWave;
  v = wave_reduce(v, op);
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < waves; ++w) r = op(r, scratch[w]);
  return r;
}

}  // namespace mla
