// Partial interleaved RoPE of one row vector by one wave (page "mlx-bun
// 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx): the
// pair-interleaved rotary prefix [a0,b0,a1,b1,...] leaves as split halves
// [real..., imag...]; the tail after the rotary prefix is kept; positions
// advance along the token axis.
//
// All of a vector's pairs are loaded before any is stored, so y may alias x.
// The angle is the f32 rounding of the double product position * inverse
// frequency (table from the host); cos, sin and the rotation are done in
// double and rounded once to the storage type.  The wave waits for all of its
// outstanding memory operations before its first store.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int kRopePairsPerLane = kRopeMaxPairs / kWave;   // 4

// vec enumerates (row, token, inner) row-major over p.rows x p.tokens x p.inner.
template <typename T>
__device__ __forceinline__ void rope_vector(const RopeParams& p, int64_t vec, int lane) {
  const int64_t per_b = static_cast<int64_t>(p.tokens) * p.inner;
  const int b = static_cast<int>(vec / per_b);
  const int64_t rem = vec - b * per_b;
  const int t = static_cast<int>(rem / p.inner);
  const int i = static_cast<int>(rem - static_cast<int64_t>(t) * p.inner);
  const int64_t base = b * p.sb + t * p.st + i * p.si;
  const T* x = static_cast<const T*>(p.x) + base;
  T* y = static_cast<T*>(p.y) + base;
  const int half = p.rotary / 2;
  const double pos = static_cast<double>(p.off[p.per_row ? b : 0] + t);

  float a[kRopePairsPerLane], bb[kRopePairsPerLane];
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    if (q < half) {
      a[k] = ld(x + 2 * q);
      bb[k] = ld(x + 2 * q + 1);
    }
  }
  // In place, another lane's store may target an element this wave still
  // reads: wait until every load of the wave has returned before storing.
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    if (q < half) {
      const float ang = static_cast<float>(pos * static_cast<double>(p.inv[q]));
      double s, c;
      sincos(static_cast<double>(ang), &s, &c);
      const double ad = a[k], bd = bb[k];
      st(y + q, ad * c - bd * s);
      st(y + half + q, bd * c + ad * s);
    }
  }
  // Out of place only (x and y do not overlap): copy the non-rotary tail.
  if (p.copy_tail)
    for (int f = p.rotary + lane; f < p.feat; f += kWave) st(y + f, static_cast<double>(ld(x + f)));
}

}  // namespace mla
