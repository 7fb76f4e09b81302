// Partial interleaved RoPE of one row vector by one wave (page "mlx-bun
// 0.0.11 -> 0.0.13", glm52-mla.ts, partialInterleavedRopeMlx): the
// pair-interleaved rotary prefix [a0,b0,a1,b1,...] leaves as split halves
// [real..., imag...]; the tail after the rotary prefix is kept; positions
// advance along the token axis.
//
// All of a vector's pairs are loaded before any is stored, so y may alias x.
#pragma once

#include <type_traits>

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
  float inv[kRopePairsPerLane];   // inverse frequency of the lane's pairs
};

// vec enumerates (row, token, inner) row-major over p.rows x p.tokens x p.inner.
// vec is the same in every lane of the wave; its row, token and position are
// then scalar values (the position a scalar load), and the pairs' inverse
// frequencies are requested with the vector's own loads.
template <typename T>
__device__ __forceinline__ void rope_load(const RopeParams& p, int64_t vec, int lane, RopeVec& v) {
  const int64_t per_b = static_cast<int64_t>(p.tokens) * p.inner;
  const int b = __builtin_amdgcn_readfirstlane(static_cast<int>(vec / per_b));
  const int64_t rem = vec - b * per_b;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(rem / p.inner));
  const int i = __builtin_amdgcn_readfirstlane(static_cast<int>(rem - static_cast<int64_t>(t) * p.inner));
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
      v.inv[k] = p.inv[q];
    }
  }
}

// Sine and cosine of the lane's pairs: the angle is the f32 rounding of the
// double product position * inverse frequency (table from the host).  fp32
// storage: sin and cos in double (rotated in double, rounded once).  bf16
// storage: the accurate fp32 device sincosf (full range reduction: positions
// reach 2^17 and beyond, where the hardware's fast sin/cos is off).  They
// depend on the position only, so they are computed while the vector's loads
// are in flight where the compiler can arrange it.
template <typename T>
using RopeTrig = typename std::conditional<sizeof(T) == 4, double, float>::type;

template <typename T>
__device__ __forceinline__ void rope_trig(const RopeParams& p, int lane, const RopeVec& v,
                                          RopeTrig<T> (&sn)[kRopePairsPerLane], RopeTrig<T> (&cs)[kRopePairsPerLane]) {
  const int half = p.rotary / 2;
  const double dpos = static_cast<double>(v.pos);
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    sn[k] = 0;
    cs[k] = 1;
    if (q < half) {
      const float ang = static_cast<float>(dpos * static_cast<double>(v.inv[k]));
      if constexpr (sizeof(T) == 4)
        sincos(static_cast<double>(ang), &sn[k], &cs[k]);
      else
        sincosf(ang, &sn[k], &cs[k]);
    }
  }
}

// The caller has waited for every load of the vector (in place, another
// lane's store may target an element this wave still reads).  fp32 storage:
// the rotation in double, rounded once; bf16 storage: the rotation in fp32
// (errors near 2^-23, against the 2^-9 of the bf16 result), rounded once to
// bf16.
template <typename T>
__device__ __forceinline__ void rope_store(const RopeParams& p, int lane, const RopeVec& v,
                                           const RopeTrig<T> (&sn)[kRopePairsPerLane],
                                           const RopeTrig<T> (&cs)[kRopePairsPerLane]) {
  T* y = static_cast<T*>(p.y) + v.base;
  const int half = p.rotary / 2;
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int q = lane + k * kWave;
    if (q < half) {
      if constexpr (sizeof(T) == 4) {
        const double ad = v.a[k], bd = v.b[k];
        st(y + q, ad * cs[k] - bd * sn[k]);
        st(y + half + q, bd * cs[k] + ad * sn[k]);
      } else {
        st(y + q, static_cast<double>(v.a[k] * cs[k] - v.b[k] * sn[k]));
        st(y + half + q, static_cast<double>(v.b[k] * cs[k] + v.a[k] * sn[k]));
      }
    }
  }
  // Out of place only (x and y do not overlap): copy the non-rotary tail.
  if (p.copy_tail) {
    const T* x = static_cast<const T*>(p.x) + v.base;
    for (int f = p.rotary + lane; f < p.feat; f += kWave) st(y + f, static_cast<double>(ld(x + f)));
  }
}

// One vector by one wave: the loads issued together, sine and cosine
// computed, then the rotated stores with nothing else in flight.
template <typename T>
__device__ __forceinline__ void rope_vector(const RopeParams& p, int64_t vec, int lane) {
  RopeVec v;
  rope_load<T>(p, vec, lane, v);
  RopeTrig<T> sn[kRopePairsPerLane], cs[kRopePairsPerLane];
  rope_trig<T>(p, lane, v, sn, cs);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  rope_store<T>(p, lane, v, sn, cs);
}

}  // namespace mla
