// Partial interleaved RoPE of one row vector by one wave (page "mlx-bun
// 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx): the
// pair-interleaved rotary prefix [a0,b0,a1,b1,...] leaves as split halves
// [real..., imag...]; the tail after the rotary prefix is kept; positions
// advance along the token axis.
//
// All of a vector's pairs are loaded before any is stored, so y may alias x.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int kRopePairsPerLane = kRopeMaxPairs / kWave;   // 4

// One row vector's pairs in registers: loaded by rope_load, rotated and
// stored by rope_store.
struct RopeVec {
  int64_t base;   // element offset of the vector in x and y
  int64_t pos;    // position of the vector's token
  float a[kRopePairsPerLane], b[kRopePairsPerLane];
};

// vec enumerates (row, token, inner) row-major over p.rows x p.tokens x p.inner.
template <typename T>
__device__ __forceinline__ void rope_load(const RopeParams& p, int64_t vec, int lane, RopeVec& v) {
  const int64_t per_b = static_cast<int64_t>(p.tokens) * p.inner;
  const int b = static_cast<int>(vec / per_b);
  const int64_t rem = vec - b * per_b;
  const int t = static_cast<int>(rem / p.inner);
  const int i = static_cast<int>(rem - static_cast<int64_t>(t) * p.inner);
  v.base = b * p.sb + t * p.st + i * p.si;
  v.pos = p.off[p.per_row ? b : 0] + t;
  const T* x = static_cast<const T*>(p.x) + v.base;
  const int half = p.rotary / 2;
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    if (q < half) {
      v.a[k] = ld(x + 2 * q);
      v.b[k] = ld(x + 2 * q + 1);
    }
  }
}

// The caller has waited for every load of the vector (in place, another
// lane's store may target an element this wave still reads).  The angle is
// the f32 rounding of the double product position * inverse frequency (table
// from the host).  fp32 storage: cos, sin and the rotation in double, rounded
// once.  bf16 storage: cos and sin from the accurate fp32 device sincosf (full
// range reduction: positions reach 2^17 and beyond, where the hardware's fast
// sin/cos is off) and the rotation in fp32 (errors near 2^-23, against the
// 2^-9 of the bf16 result), rounded once to bf16.
template <typename T>
__device__ __forceinline__ void rope_store(const RopeParams& p, int lane, const RopeVec& v) {
  T* y = static_cast<T*>(p.y) + v.base;
  const int half = p.rotary / 2;
  const double pos = static_cast<double>(v.pos);
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    if (q < half) {
      const float ang = static_cast<float>(pos * static_cast<double>(p.inv[q]));
      if constexpr (sizeof(T) == 4) {
        double sn, cs;
        sincos(static_cast<double>(ang), &sn, &cs);
        const double ad = v.a[k], bd = v.b[k];
        st(y + q, ad * cs - bd * sn);
        st(y + half + q, bd * cs + ad * sn);
      } else {
        float sn, cs;
        sincosf(ang, &sn, &cs);
        st(y + q, static_cast<double>(v.a[k] * cs - v.b[k] * sn));
        st(y + half + q, static_cast<double>(v.b[k] * cs + v.a[k] * sn));
      }
    }
  }
  // Out of place only (x and y do not overlap): copy the non-rotary tail.
  if (p.copy_tail) {
    const T* x = static_cast<const T*>(p.x) + v.base;
    for (int f = p.rotary + lane; f < p.feat; f += kWave) st(y + f, static_cast<double>(ld(x + f)));
  }
}

// One vector by one wave, loads and stores with nothing else in flight.
template <typename T>
__device__ __forceinline__ void rope_vector(const RopeParams& p, int64_t vec, int lane) {
  RopeVec v;
  rope_load<T>(p, vec, lane, v);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  rope_store<T>(p, lane, v);
}

}  // namespace mla
