// DSA top-k position selection (page "mlx-bun 0.4.0 -> 1.0.0", glm52-dsa.ts,
// selectGlm52DsaDevice).  Per row of float32 scores s[0..n), n > top_k:
//   rank key  = ~(order-preserving uint32 of the float bits), so ascending
//               keys are descending scores and equal keys mean equal bits;
//   selection = the top_k smallest keys, equal keys taken in ascending
//               position order (the page's stable sort);
//   threshold = the minimum selected score;
//   output    = selected positions with score > threshold (float compare),
//               ascending, then the other selected positions, ascending.
//
// One workgroup of 1024 threads per selected row, no workspace:
//   1. radix select with digits of 12, 12 and 8 bits from the top, over
//      coalesced chunks of the row: an LDS histogram of the keys that match
//      the prefix found so far locates the digit of the top_k-th smallest key
//      K*; at the end, m = how many of the keys equal to K* are selected (the
//      first m by position);
//   2. wave w owns a contiguous run of positions, swept 64 at a time: a first
//      sweep counts the class-0 positions (key < K* and score > threshold; the
//      threshold is the score with key K*, the minimum selected score), the
//      other positions below K*, and the ties (key == K*); the 16 wave counts
//      give each wave its starting ranks; a second sweep writes: class 0 at
//      its class-0 rank, class 1 after all n0 class-0 positions at (lower
//      class-1 positions before it) + min(ties before it, m), since the
//      selected ties are the first m.  Ranks inside 64 positions come from
//      ballots.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kTT = 1024;
constexpr int kTW = kTT / kWave;   // 16 waves
constexpr int kU = 32;             // scores per thread loaded together in every pass (128 KB in flight per CU)

__device__ __forceinline__ uint32_t rank_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t ascending = (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
  return ~ascending;
}

__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t ascending = ~key;
  return __uint_as_float((ascending & 0x80000000u) ? (ascending ^ 0x80000000u) : ~ascending);
}

__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(ballot), 0u));
}

__global__ __launch_bounds__(kTT) void dsa_topk_kernel(TopkParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int row = p.row[blockIdx.x];
  const int n = p.len[blockIdx.x];
  const float* sc = p.scores + static_cast<int64_t>(row) * p.stride;
  int32_t* out = p.sel_idx + p.out_off[blockIdx.x];
  const uint32_t k = static_cast<uint32_t>(p.top_k);
  // whole 16-byte groups: an aligned row whose length is a multiple of 4
  const bool vec4 = (reinterpret_cast<uintptr_t>(sc) & 15) == 0 && (n & 3) == 0;

  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_prefix, s_rank;
  __shared__ int s_tot[3][kTW];

  // ---- 1. radix select of the k-th smallest key: digits of 12, 12 and 8 bits
  // from the top (12-bit digits spread the sign-and-exponent-heavy top bits
  // of the keys over enough bins that the histogram atomics rarely collide)
  uint32_t prefix = 0, mask = 0, rank = k;   // rank: 1-based, among keys matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass < 2 ? 12 : 8;
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = 1 << bits;
    const uint32_t digit = static_cast<uint32_t>(nb - 1);
    for (int i = tid; i < nb; i += kTT) hist[i] = 0;
    __syncthreads();
    if (vec4) {
      // 16-byte loads: thread t covers positions base + 4 (u kTT + t) .. +3
      for (int base = 0; base < n; base += kTT * kU) {
        float4 v[kU / 4];
#pragma unroll
        for (int u = 0; u < kU / 4; ++u) {
          const int i = base + 4 * (u * kTT + tid);
          v[u] = i < n ? *reinterpret_cast<const float4*>(sc + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kU / 4; ++u) {
          const int i = base + 4 * (u * kTT + tid);
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t key = rank_key(e[q]);
            if (i < n && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & digit], 1u);
          }
        }
      }
    } else {
      for (int base = 0; base < n; base += kTT * kU) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = base + u * kTT + tid;
          v[u] = i < n ? sc[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t key = rank_key(v[u]);
          if (base + u * kTT + tid < n && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & digit], 1u);
        }
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns the per = nb / 64 consecutive bins from l * per
      const int per = nb / kWave;
      uint32_t sum = 0;
      for (int j = 0; j < per; ++j) sum += hist[tid * per + j];
      uint32_t incl = sum;   // inclusive scan of the lane sums
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, kWave);
        if (tid >= off) incl += v;
      }
      const uint32_t before = incl - sum;
      // the lane whose range holds the rank-th key: before < rank <= incl
      if (before < rank && rank <= incl) {
        uint32_t cum = before;
        int bin = tid * per;
        for (int j = 0; j < per; ++j) {
          const uint32_t c = hist[tid * per + j];
          if (cum + c >= rank) {
            bin = tid * per + j;
            break;
          }
          cum += c;
        }
        s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
        s_rank = rank - cum;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    rank = s_rank;
    mask |= digit << shift;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int m = static_cast<int>(rank);   // the first m keys equal to K* are selected
  const float thr = key_score(kstar);

  // ---- 2. wave runs: count, exchange, write
  const int per_wave = ((n + kTW - 1) / kTW + kWave - 1) / kWave * kWave;
  const int w_lo = min(n, wave * per_wave), w_hi = min(n, w_lo + per_wave);
  int c0 = 0, c1 = 0, ct = 0;   // wave-uniform: class 0, other keys below K*, ties
  for (int base = w_lo; base < w_hi; base += kWave * kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kWave + lane;
      v[u] = i < w_hi ? sc[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = base + u * kWave + lane < w_hi;
      const uint32_t key = rank_key(v[u]);
      c0 += __popcll(__ballot(ok && key < kstar && v[u] > thr));
      c1 += __popcll(__ballot(ok && key < kstar && !(v[u] > thr)));
      ct += __popcll(__ballot(ok && key == kstar));
    }
  }
  if (lane == 0) {
    s_tot[0][wave] = c0;
    s_tot[1][wave] = c1;
    s_tot[2][wave] = ct;
  }
  __syncthreads();
  int r0 = 0, r1 = 0, rt = 0, n0 = 0;
  for (int w = 0; w < kTW; ++w) {
    if (w < wave) {
      r0 += s_tot[0][w];
      r1 += s_tot[1][w];
      rt += s_tot[2][w];
    }
    n0 += s_tot[0][w];
  }
  for (int base = w_lo; base < w_hi; base += kWave * kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kWave + lane;
      v[u] = i < w_hi ? sc[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kWave + lane;
      const bool ok = i < w_hi;
      const uint32_t key = rank_key(v[u]);
      const bool f0 = ok && key < kstar && v[u] > thr;
      const bool f1 = ok && key < kstar && !(v[u] > thr);
      const bool ft = ok && key == kstar;
      const uint64_t b0 = __ballot(f0), b1 = __ballot(f1), bt = __ballot(ft);
      const int t_before = rt + lanes_below(bt);
      if (f0) out[r0 + lanes_below(b0)] = i;
      if (f1) out[n0 + r1 + lanes_below(b1) + min(t_before, m)] = i;
      if (ft && t_before < m) out[n0 + r1 + lanes_below(b1) + t_before] = i;
      r0 += __popcll(b0);
      r1 += __popcll(b1);
      rt += __popcll(bt);
    }
  }
}

}  // namespace

hipError_t launch_dsa_topk(const TopkParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_topk_kernel, dim3(p.rows), dim3(kTT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
