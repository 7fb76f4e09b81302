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
//   1. radix select, 8 bits per pass from the top: a 256-bin LDS histogram of
//      the keys that match the prefix found so far locates the byte of the
//      top_k-th smallest key K*; at the end, m = how many of the keys equal
//      to K* are selected (the first m by position);
//   2. one pass counts n0 = selected positions strictly above the threshold
//      (keys below K* whose score is > the score of K*; the threshold is the
//      score with key K*, which is the minimum selected score);
//   3. one ordered pass over the positions in chunks of 1024: block-wide
//      exclusive scans (wave ballots + per-wave totals in LDS) of the tie and
//      class flags give every selected position its output slot.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kTT = 1024;
constexpr int kTW = kTT / kWave;   // 16 waves

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

// Exclusive block scan of three flags; returns the block totals in tot[].
// Contains two barriers; every thread of the block must call it.
__device__ __forceinline__ void block_scan3(const bool f[3], int ex[3], int tot[3], int (*s_tot)[kTW]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint64_t b[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    b[k] = __ballot(f[k]);
    ex[k] = lanes_below(b[k]);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) s_tot[k][wave] = __popcll(b[k]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int below = 0, all = 0;
    for (int w = 0; w < kTW; ++w) {
      const int t = s_tot[k][w];
      below += w < wave ? t : 0;
      all += t;
    }
    ex[k] += below;
    tot[k] = all;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTT) void dsa_topk_kernel(TopkParams p) {
  const int tid = threadIdx.x;
  const int row = p.row[blockIdx.x];
  const int n = p.len[blockIdx.x];
  const float* sc = p.scores + static_cast<int64_t>(row) * p.stride;
  int32_t* out = p.sel_idx + p.out_off[blockIdx.x];
  const uint32_t k = static_cast<uint32_t>(p.top_k);

  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rank;
  __shared__ int s_tot[3][kTW];

  // ---- 1. radix select of the k-th smallest key
  uint32_t prefix = 0, mask = 0, rank = k;   // rank: 1-based, among keys matching the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTT) {
      const uint32_t key = rank_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns bins 4l .. 4l+3
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[4 * tid + j];
        sum += c[j];
      }
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
        int bin = 4 * tid;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= rank) {
            bin = 4 * tid + j;
            break;
          }
          cum += c[j];
        }
        s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
        s_rank = rank - cum;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    rank = s_rank;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int ties_taken = static_cast<int>(rank);   // first `rank` keys equal to K* are selected
  const float thr = key_score(kstar);

  // ---- 2. n0 = selected positions strictly above the threshold
  int cnt = 0;
  for (int i = tid; i < n; i += kTT) {
    const float v = sc[i];
    cnt += (rank_key(v) < kstar && v > thr) ? 1 : 0;
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
  if ((tid & (kWave - 1)) == 0) s_tot[0][tid / kWave] = cnt;
  __syncthreads();
  int n0 = 0;
  for (int w = 0; w < kTW; ++w) n0 += s_tot[0][w];
  __syncthreads();

  // ---- 3. ordered write
  int ties_before = 0, w0 = 0, w1 = 0;
  for (int base = 0; base < n; base += kTT) {
    const int i = base + tid;
    bool lt = false, tie = false;
    float v = 0.f;
    if (i < n) {
      v = sc[i];
      const uint32_t key = rank_key(v);
      lt = key < kstar;
      tie = key == kstar;
    }
    bool f[3] = {tie, false, false};
    int ex[3], tot[3];
    // first scan: tie ranks decide which ties are selected
    block_scan3(f, ex, tot, s_tot);
    const bool sel = lt || (tie && ties_before + ex[0] < ties_taken);
    const bool c0 = sel && v > thr;
    const bool c1 = sel && !c0;
    const int tie_total = tot[0];
    f[0] = c0;
    f[1] = c1;
    block_scan3(f, ex, tot, s_tot);
    if (c0) out[w0 + ex[0]] = i;
    if (c1) out[n0 + w1 + ex[1]] = i;
    ties_before += tie_total;
    w0 += tot[0];
    w1 += tot[1];
    if (w0 + w1 >= static_cast<int>(k)) break;   // uniform: every selected position is written
  }
}

}  // namespace

hipError_t launch_dsa_topk(const TopkParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_topk_kernel, dim3(p.rows), dim3(kTT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
