// DSA top-k position selection (page "mlx-bun 0.2.0 -> 0.4.0", glm52-dsa.ts,
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
//
// Multi-workgroup form for the long rows of a 131072-token context (16385 to
// 131072 scores), in three launches with a caller workspace: per segment of
// 8192 scores a bound on K*, then each segment's keys at or below the
// largest bound (the survivors, in position order), then one workgroup per
// row runs the select and the two sweeps over the survivors (see the
// kernels below).
// Both forms give the same integers.
#include <mutex>

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

// Cross-lane steps on the VALU (DPP and the gfx950 lane swaps) instead of
// lane shuffles through ds_bpermute, which wait on LDS latency at every step.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {   // lanes without a source read 0
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_self(uint32_t v) {   // every lane has a source in these patterns
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf,
                                                           false));
}

// Inclusive prefix sum over the wave's 64 lanes: shifts by 1, 2, 4 and 8 lanes
// inside each row of 16, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then the first half's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp_zero<0x111>(v);
  v += dpp_zero<0x112>(v);
  v += dpp_zero<0x114>(v);
  v += dpp_zero<0x118>(v);
  v += dpp_zero<0x142, 0xa>(v);
  v += dpp_zero<0x143, 0xc>(v);
  return v;
}

// Minimum and maximum over the wave (every lane receives both): lane pairs
// i ^ 1 and i ^ 2 (quad permutes), then the mirrors inside 8 and 16 lanes,
// then the 16- and 32-lane swaps.
__device__ __forceinline__ void wave_min_max(uint32_t& lo, uint32_t& hi) {
  lo = min(lo, dpp_self<0xB1>(lo));
  hi = max(hi, dpp_self<0xB1>(hi));
  lo = min(lo, dpp_self<0x4E>(lo));
  hi = max(hi, dpp_self<0x4E>(hi));
  lo = min(lo, dpp_self<0x141>(lo));
  hi = max(hi, dpp_self<0x141>(hi));
  lo = min(lo, dpp_self<0x140>(lo));
  hi = max(hi, dpp_self<0x140>(hi));
  auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  lo = min(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  a = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  hi = max(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  lo = min(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  a = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  hi = max(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
}

// After a histogram pass over `nb` bins: the bin holding the rank-th key
// (1-based) among those matching the prefix; the thread that finds it writes
// the extended prefix and the rank within the bin.  Whole-block call: thread t
// owns nb / min(nb, kTT) consecutive bins; their sums are scanned by waves,
// then across the waves through `wtot` (kTW entries).
__device__ __forceinline__ void locate_digit(const uint32_t* hist, int nb, uint32_t rank, uint32_t prefix, int shift,
                                             uint32_t* s_prefix, uint32_t* s_rank, uint32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int users = min(nb, kTT);
  const int per = nb / users;
  uint32_t sum = 0;
  if (tid < users)
    for (int j = 0; j < per; ++j) sum += hist[tid * per + j];
  uint32_t incl = wave_inclusive_sum(sum);
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wtot[w];
  const uint32_t before = incl - sum;
  if (tid < users && before < rank && rank <= incl) {
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
    *s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
    *s_rank = rank - cum;
  }
}

// Radix select over keys[0..n) in LDS (digits of 12, 12 and 8 bits): K* = the
// k-th smallest key, m = how many keys equal to K* the selection takes (the
// first m in array order).  Whole-block call (contains barriers).
__device__ __forceinline__ void lds_radix_select(const uint32_t* keys, int n, uint32_t k, uint32_t* hist,
                                                 uint32_t* s_prefix, uint32_t* s_rank, uint32_t* wtot,
                                                 uint32_t& kstar, int& m) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, rank = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass < 2 ? 12 : 8;
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = 1 << bits;
    const uint32_t digit = static_cast<uint32_t>(nb - 1);
    for (int i = tid; i < nb; i += kTT) hist[i] = 0;
    __syncthreads();
#pragma unroll 8
    for (int i = tid; i < n; i += kTT) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & digit], 1u);
    }
    __syncthreads();
    locate_digit(hist, nb, rank, prefix, shift, s_prefix, s_rank, wtot);
    __syncthreads();
    prefix = *s_prefix;
    rank = *s_rank;
    mask |= digit << shift;
    __syncthreads();
  }
  kstar = prefix;
  m = static_cast<int>(rank);
}

// ---- select by score buckets (the two-stage kernels' first try).  Keys
// ascend as scores descend, so the bucket of a score, floor((vmax - score) *
// scale) with scale = kBuckets / (vmax - vmin), is non-decreasing in the key
// (fp32 subtraction, product and truncation are monotone) and equal scores
// share one: every key of a lower bucket is smaller than every key of a
// higher one.  One histogram pass locates the bucket b holding the k-th
// smallest key and its rank r inside b; the few keys of b are gathered, and
// K* is the key of b with fewer than r keys of b below it and at least r at
// or below it, found by direct comparison; m = r - (keys of b below K*).
// Normal-like scores spread evenly over the buckets, so the histogram's
// atomics rarely collide (the radix digits' top bits put a whole octave of
// scores in one bin).  The result is the (K*, m) the radix select finds.
// Rows with a non-finite or zero score range, or more than kSmallCap keys in
// b (long runs of equal scores), take the radix select instead.
constexpr int kBuckets = 4096;
constexpr int kSweep = 8;   // LDS keys read together by each lane in the passes
constexpr int kSmallCap = 1024;

__device__ __forceinline__ int score_bucket(uint32_t key, float vmax, float scale) {
  const float f = (vmax - key_score(key)) * scale;
  return f >= static_cast<float>(kBuckets - 1) ? kBuckets - 1 : (f >= 0.f ? static_cast<int>(f) : 0);
}

// Whole-block minimum and maximum (every thread receives both).
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, uint32_t* s_mm, uint32_t& kmin, uint32_t& kmax) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  wave_min_max(lo, hi);
  if (lane == 0) {
    s_mm[wave] = lo;
    s_mm[kTW + wave] = hi;
  }
  __syncthreads();
  kmin = s_mm[0];
  kmax = s_mm[kTW];
#pragma unroll
  for (int w = 1; w < kTW; ++w) {
    kmin = min(kmin, s_mm[w]);
    kmax = max(kmax, s_mm[kTW + w]);
  }
}

// The one-workgroup selection of a whole row of n scores at sc into out
// (whole-block call).  LDS: hist (4096 bins), two scalars, kTW wave totals and
// three rows of kTW wave counts.
__device__ __forceinline__ void select_row(const float* sc, int n, uint32_t k, int32_t* out, uint32_t* hist,
                                           uint32_t* s_prefix, uint32_t* s_rank, uint32_t* s_wtot,
                                           int (*s_tot)[kTW]) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // whole 16-byte groups: an aligned row whose length is a multiple of 4
  const bool vec4 = (reinterpret_cast<uintptr_t>(sc) & 15) == 0 && (n & 3) == 0;

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
    locate_digit(hist, nb, rank, prefix, shift, s_prefix, s_rank, s_wtot);
    __syncthreads();
    prefix = *s_prefix;
    rank = *s_rank;
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

__global__ __launch_bounds__(kTT) void dsa_topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_prefix, s_rank;
  __shared__ uint32_t s_wtot[kTW];
  __shared__ int s_tot[3][kTW];
  select_row(p.scores + static_cast<int64_t>(p.row[blockIdx.x]) * p.stride, p.len[blockIdx.x],
             static_cast<uint32_t>(p.top_k), p.sel_idx + p.out_off[blockIdx.x], hist, &s_prefix, &s_rank, s_wtot,
             s_tot);
}

// ---- multi-workgroup form, three launches.  Segments of kPrSeg scores.
//   1. bound: segment i of a row of n scores finds t_i, its r_i-th smallest
//      key, r_i = ceil(top_k len_i / n).  Every segment holds r_i keys <= t_i
//      and the r_i add up to at least top_k, so at least top_k keys of the row
//      are <= T = max_i t_i: K* <= T, and no key above T is selected.
//   2. prune: segment i writes its keys <= T (the survivors, typically a few
//      percent of the row) with their positions, in ascending position order,
//      and their count.
//   3. final: one workgroup per row gathers the survivors of its segments
//      (ascending positions) into LDS and runs the select and the two sweeps
//      of the one-workgroup form over them: every key <= K* survives, so K*,
//      m and the output are the row's.  A segment with more survivors than
//      its area holds (long runs of equal scores) sends its row through the
//      one-workgroup form instead, in the same launch.
// Workspace of launch row i (kTopkRowWsBytes): survivor keys [kTopkMaxCand]
// uint32, their positions [kTopkMaxCand] int32 (segment s from s * kPrCap),
// then per segment its survivor count [kPrMaxSegs] int32 and t_s
// [kPrMaxSegs] uint32.
constexpr int kPrSeg = 8192;
constexpr int kPrMaxSegs = 16;
constexpr int kPrCap = kTopkMaxCand / kPrMaxSegs;   // survivors a segment's area holds
static_assert(kPrSeg * kPrMaxSegs >= kTopkSeg * kTopkMaxSegs, "the segments cover the rows of this form");
static_assert(kTopkMaxCand * 8 + 8 * kPrMaxSegs <= static_cast<int>(kTopkRowWsBytes), "workspace of a row");

__device__ __forceinline__ uint32_t* ws_keys(const TopkParams& p, int i) {
  return reinterpret_cast<uint32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes);
}
__device__ __forceinline__ int32_t* ws_pos(const TopkParams& p, int i) {
  return reinterpret_cast<int32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes + kTopkMaxCand * 4);
}
__device__ __forceinline__ int32_t* ws_cnt(const TopkParams& p, int i) {
  return reinterpret_cast<int32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes + kTopkMaxCand * 8);
}
__device__ __forceinline__ uint32_t* ws_bound(const TopkParams& p, int i) {
  return reinterpret_cast<uint32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes + kTopkMaxCand * 8 +
                                     4 * kPrMaxSegs);
}

// The bucket select of the multi-workgroup kernels, fused with the per-wave counts
// of the order-keeping sweep that follows it.  Wave w owns the run
// [w_lo, w_hi) of the n keys.  On success: K* and m, and for every wave the
// number of its keys in buckets below K*'s (their scores exceed the
// threshold) in s_below[wave]; the keys of K*'s bucket are in small[0..c)
// with their index in small_at, for the caller to classify.  Returns false
// (nothing written but the histogram) when the radix select has to run.
__device__ __forceinline__ bool bucket_select_runs(const uint32_t* keys, int n, uint32_t k, uint32_t kmin,
                                                   uint32_t kmax, int w_lo, int w_hi, uint32_t* hist, uint32_t* small,
                                                   uint16_t* small_at, uint32_t* s_prefix, uint32_t* s_rank,
                                                   uint32_t* wtot, uint32_t* s_cnt, int* s_below, uint32_t& kstar,
                                                   int& m, int& c) {
  const float vmax = key_score(kmin), vmin = key_score(kmax);
  const float range = vmax - vmin;
  const float scale = static_cast<float>(kBuckets) / range;
  // uniform: every thread holds the same kmin and kmax
  if (!__builtin_isfinite(vmax) || !__builtin_isfinite(vmin) || !(range > 0.f) || !__builtin_isfinite(range) ||
      !__builtin_isfinite(scale))
    return false;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // a batch of keys read before its atomics (the compiler would otherwise wait
  // for each read behind the previous atomic)
  for (int i0 = tid; i0 < n; i0 += kSweep * kTT) {
    uint32_t kk[kSweep];
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      const int i = i0 + u * kTT;
      kk[u] = i < n ? keys[i] : 0u;
    }
    // past n: no atomic (a short candidate list would otherwise pile its idle
    // lanes' atomics onto one bin), and no work at all once the whole wave is
    // past n (wave-uniform)
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      if (i0 - lane + u * kTT >= n) break;
      if (i0 + u * kTT < n) atomicAdd(&hist[score_bucket(kk[u], vmax, scale)], 1u);
    }
  }
  __syncthreads();
  locate_digit(hist, kBuckets, k, 0u, 0, s_prefix, s_rank, wtot);
  __syncthreads();
  const int b = static_cast<int>(*s_prefix);
  const uint32_t r = *s_rank;
  c = static_cast<int>(hist[b]);
  if (c > kSmallCap) return false;   // uniform
  // the wave's run: keys of lower buckets counted, K*'s bucket gathered
  uint32_t below = 0;
  for (int i0 = w_lo; i0 < w_hi; i0 += kSweep * kWave) {
    uint32_t kk[kSweep];
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      const int i = i0 + u * kWave + lane;
      kk[u] = i < w_hi ? keys[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      if (i0 + u * kWave >= w_hi) break;   // the rest of the batch lies past the run (uniform)
      const int i = i0 + u * kWave + lane;
      const int bk = i < w_hi ? score_bucket(kk[u], vmax, scale) : kBuckets;
      below += __popcll(__ballot(bk < b));
      if (bk == b) {
        const uint32_t at = atomicAdd(s_cnt, 1u);
        small[at] = kk[u];
        small_at[at] = static_cast<uint16_t>(i);
      }
    }
  }
  if (lane == 0) s_below[wave] = static_cast<int>(below);
  __syncthreads();
  for (int t = tid; t < c; t += kTT) {
    const uint32_t kt = small[t];
    uint32_t less = 0, le = 0;
    for (int j = 0; j < c; ++j) {
      const uint32_t kj = small[j];
      less += kj < kt;
      le += kj <= kt;
    }
    if (less < r && r <= le) {   // every thread holding K* writes the same values
      *s_prefix = kt;
      *s_rank = r - less;
    }
  }
  __syncthreads();
  kstar = *s_prefix;
  m = static_cast<int>(*s_rank);
  return true;
}

// The keys of a segment's len scores at sc into keys[] (LDS); klo / khi: this
// thread's minimum and maximum.
__device__ __forceinline__ void load_segment_keys(const float* sc, int len, uint32_t* keys, uint32_t& klo,
                                                  uint32_t& khi) {
  const int tid = threadIdx.x;
  klo = 0xffffffffu;
  khi = 0u;
  if ((reinterpret_cast<uintptr_t>(sc) & 15) == 0 && (len & 3) == 0) {
    float4 v[kPrSeg / (4 * kTT)];
#pragma unroll
    for (int u = 0; u < kPrSeg / (4 * kTT); ++u) {
      const int i = 4 * (u * kTT + tid);
      v[u] = i < len ? *reinterpret_cast<const float4*>(sc + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kPrSeg / (4 * kTT); ++u) {
      const int i = 4 * (u * kTT + tid);
      if (i < len) {
        const uint4 q = make_uint4(rank_key(v[u].x), rank_key(v[u].y), rank_key(v[u].z), rank_key(v[u].w));
        *reinterpret_cast<uint4*>(&keys[i]) = q;
        klo = min(klo, min(min(q.x, q.y), min(q.z, q.w)));
        khi = max(khi, max(max(q.x, q.y), max(q.z, q.w)));
      }
    }
  } else {
    float v[kPrSeg / kTT];
#pragma unroll
    for (int u = 0; u < kPrSeg / kTT; ++u) {
      const int i = u * kTT + tid;
      v[u] = i < len ? sc[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPrSeg / kTT; ++u) {
      const int i = u * kTT + tid;
      if (i < len) {
        const uint32_t key = rank_key(v[u]);
        keys[i] = key;
        klo = min(klo, key);
        khi = max(khi, key);
      }
    }
  }
}

// 1. bound
__global__ __launch_bounds__(kTT) void dsa_topk_bound_kernel(TopkParams p) {
  const int seg = blockIdx.x, i_row = blockIdx.y;
  const int n = p.len[i_row];
  const int lo = seg * kPrSeg;
  if (lo >= n) return;   // the row has fewer segments (uniform)
  const int len = min(kPrSeg, n - lo);
  const int tid = threadIdx.x, wave = tid / kWave;
  const float* sc = p.scores + static_cast<int64_t>(p.row[i_row]) * p.stride + lo;
  // 1 <= r <= len, as top_k < n
  const uint32_t r = static_cast<uint32_t>((static_cast<int64_t>(p.top_k) * len + n - 1) / n);

  __shared__ __attribute__((aligned(16))) uint32_t keys[kPrSeg];
  __shared__ uint32_t hist[kBuckets];
  __shared__ uint32_t small[kSmallCap];
  __shared__ uint16_t small_at[kSmallCap];
  __shared__ uint32_t s_prefix, s_rank, s_cnt;
  __shared__ uint32_t s_wtot[kTW];
  __shared__ uint32_t s_mm[2 * kTW];
  __shared__ int s_below[kTW];
  uint32_t klo, khi;
  load_segment_keys(sc, len, keys, klo, khi);
  for (int i = tid; i < kBuckets; i += kTT) hist[i] = 0;
  if (tid == 0) s_cnt = 0;
  uint32_t kmin, kmax, t = 0;
  int m = 0, c = 0;
  block_minmax(klo, khi, s_mm, kmin, kmax);   // its barrier publishes the keys and the zeroed counters
  const int per_wave = ((len + kTW - 1) / kTW + kWave - 1) / kWave * kWave;
  const int w_lo = min(len, wave * per_wave), w_hi = min(len, w_lo + per_wave);
  if (!bucket_select_runs(keys, len, r, kmin, kmax, w_lo, w_hi, hist, small, small_at, &s_prefix, &s_rank, s_wtot,
                          &s_cnt, s_below, t, m, c))
    lds_radix_select(keys, len, r, hist, &s_prefix, &s_rank, s_wtot, t, m);
  if (tid == 0) ws_bound(p, i_row)[seg] = t;
}

// 2. prune.  Wave w owns positions [512 w, 512 w + 512) of the segment; a
// survivor's slot is the survivors of the lower waves plus those before it
// in its wave.
__global__ __launch_bounds__(kTT) void dsa_topk_prune_kernel(TopkParams p) {
  constexpr int kPer = kPrSeg / kTT;   // 8 scores per lane
  const int seg = blockIdx.x, i_row = blockIdx.y;
  const int n = p.len[i_row];
  const int lo = seg * kPrSeg;
  if (lo >= n) return;   // uniform
  const int len = min(kPrSeg, n - lo);
  const int segs = (n + kPrSeg - 1) / kPrSeg;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float* sc = p.scores + static_cast<int64_t>(p.row[i_row]) * p.stride + lo;
  __shared__ int s_cnt[kTW];
  // all bounds requested at once (a fixed trip count: one batch of loads, not
  // one round trip per segment)
  const uint32_t* bound = ws_bound(p, i_row);
  uint32_t tmax = 0u;
#pragma unroll
  for (int s = 0; s < kPrMaxSegs; ++s) tmax = max(tmax, s < segs ? bound[s] : 0u);
  uint32_t key[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = wave * (kPer * kWave) + u * kWave + lane;
    key[u] = i < len ? rank_key(sc[i]) : 0xffffffffu;
  }
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = wave * (kPer * kWave) + u * kWave + lane;
    cnt += __popcll(__ballot(i < len && key[u] <= tmax));
  }
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  int at = 0, total = 0;
  for (int w = 0; w < kTW; ++w) {
    if (w < wave) at += s_cnt[w];
    total += s_cnt[w];
  }
  uint32_t* out_key = ws_keys(p, i_row) + seg * kPrCap;
  int32_t* out_pos = ws_pos(p, i_row) + seg * kPrCap;
  if (total <= kPrCap) {   // uniform
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = wave * (kPer * kWave) + u * kWave + lane;
      const bool keep = i < len && key[u] <= tmax;
      const uint64_t b = __ballot(keep);
      if (keep) {
        const int d = at + lanes_below(b);
        out_key[d] = key[u];
        out_pos[d] = lo + i;
      }
      at += __popcll(b);
    }
  }
  if (tid == 0) ws_cnt(p, i_row)[seg] = total;
}

// 3. final: the row's selection among the survivors, in the page's order.
__global__ __launch_bounds__(kTT) void dsa_topk_final_kernel(TopkParams p) {
  const int i_row = blockIdx.x;
  const int n = p.len[i_row];
  const int segs = (n + kPrSeg - 1) / kPrSeg;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t k = static_cast<uint32_t>(p.top_k);
  int32_t* out = p.sel_idx + p.out_off[i_row];

  __shared__ uint32_t ckey[kTopkMaxCand];
  __shared__ int32_t cpos[kTopkMaxCand];
  __shared__ uint32_t hist[kBuckets];   // the histogram, then the staged output
  __shared__ uint32_t small[kSmallCap];
  __shared__ uint16_t small_at[kSmallCap];
  __shared__ uint32_t s_prefix, s_rank, s_cnt;
  __shared__ uint32_t s_wtot[kTW];
  __shared__ uint32_t s_mm[2 * kTW];
  __shared__ int s_tot[3][kTW];   // per wave: class 0, other keys below K*, keys equal to K*
  // thread t takes survivor t of every segment (at most kPrCap = kTT each),
  // requested together with the counts: one round trip for both (slots past a
  // segment's count hold stale values and are never used)
  static_assert(kPrCap <= kTT, "one survivor per thread and segment");
  uint32_t kv[kPrMaxSegs];
  int32_t pv[kPrMaxSegs];
  {
    const uint32_t* ks = ws_keys(p, i_row);
    const int32_t* ps = ws_pos(p, i_row);
#pragma unroll
    for (int s = 0; s < kPrMaxSegs; ++s) {
      kv[s] = ks[s * kPrCap + tid];
      pv[s] = ps[s * kPrCap + tid];
    }
  }
  // survivors per segment (uniform: every thread reads the same counts; all
  // requested at once)
  const int32_t* cnt = ws_cnt(p, i_row);
  int cs[kPrMaxSegs];
  int c_total = 0;
  bool overflow = false;
#pragma unroll
  for (int s = 0; s < kPrMaxSegs; ++s) {
    cs[s] = s < segs ? cnt[s] : 0;
    overflow |= cs[s] > kPrCap;
    c_total += cs[s];
  }
  if (overflow) {
    select_row(p.scores + static_cast<int64_t>(p.row[i_row]) * p.stride, n, k, out, hist, &s_prefix, &s_rank, s_wtot,
               s_tot);
    return;
  }
  uint32_t klo = 0xffffffffu, khi = 0u;
  {
    int base = 0;
#pragma unroll
    for (int s = 0; s < kPrMaxSegs; ++s) {
      if (tid < cs[s]) {
        ckey[base + tid] = kv[s];
        cpos[base + tid] = pv[s];
        klo = min(klo, kv[s]);
        khi = max(khi, kv[s]);
      }
      base += cs[s];
    }
  }
  for (int i = tid; i < kBuckets; i += kTT) hist[i] = 0;
  if (tid == 0) s_cnt = 0;
  if (tid < kTW) {
    s_tot[1][tid] = 0;
    s_tot[2][tid] = 0;
  }
  uint32_t kmin, kmax, kstar = 0;
  int m = 0, c = 0;
  block_minmax(klo, khi, s_mm, kmin, kmax);   // its barrier publishes the candidates and the zeroed counters
  const int per_wave = ((c_total + kTW - 1) / kTW + kWave - 1) / kWave * kWave;
  const int w_lo = min(c_total, wave * per_wave), w_hi = min(c_total, w_lo + per_wave);
  float thr;
  if (bucket_select_runs(ckey, c_total, k, kmin, kmax, w_lo, w_hi, hist, small, small_at, &s_prefix, &s_rank, s_wtot,
                         &s_cnt, s_tot[0], kstar, m, c)) {
    // keys of lower buckets score above the threshold (class 0, counted);
    // K*'s bucket is classified key by key
    thr = key_score(kstar);
    for (int t = tid; t < c; t += kTT) {
      const uint32_t kt = small[t];
      const int w = small_at[t] / per_wave;
      if (kt < kstar)
        atomicAdd(&s_tot[key_score(kt) > thr ? 0 : 1][w], 1);
      else if (kt == kstar)
        atomicAdd(&s_tot[2][w], 1);
    }
  } else {
    lds_radix_select(ckey, c_total, k, hist, &s_prefix, &s_rank, s_wtot, kstar, m);
    thr = key_score(kstar);
    int c0 = 0, c1 = 0, ct = 0;
    for (int i0 = w_lo; i0 < w_hi; i0 += kSweep * kWave) {
      uint32_t kk[kSweep];
#pragma unroll
      for (int u = 0; u < kSweep; ++u) {
        const int i = i0 + u * kWave + lane;
        kk[u] = i < w_hi ? ckey[i] : 0xffffffffu;
      }
#pragma unroll
      for (int u = 0; u < kSweep; ++u) {
        if (i0 + u * kWave >= w_hi) break;   // uniform
        const bool ok = i0 + u * kWave + lane < w_hi;
        const uint32_t key = kk[u];
        const float v = key_score(key);
        c0 += __popcll(__ballot(ok && key < kstar && v > thr));
        c1 += __popcll(__ballot(ok && key < kstar && !(v > thr)));
        ct += __popcll(__ballot(ok && key == kstar));
      }
    }
    if (lane == 0) {
      s_tot[0][wave] = c0;
      s_tot[1][wave] = c1;
      s_tot[2][wave] = ct;
    }
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
  // the sweeps of the one-workgroup form over the candidates (ascending
  // positions): class 0 (key < K*, score > threshold), class 1 (other keys
  // below K*) and ties (key == K*, the first m selected); staged in LDS (the
  // histogram's space) when it holds top_k positions
  const bool stage = k <= static_cast<uint32_t>(kBuckets);
  int32_t* st = reinterpret_cast<int32_t*>(hist);
  int32_t* dst_base = stage ? st : out;
  for (int i0 = w_lo; i0 < w_hi; i0 += kSweep * kWave) {
    uint32_t kk[kSweep];
    int32_t pp[kSweep];
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      const int i = i0 + u * kWave + lane;
      kk[u] = i < w_hi ? ckey[i] : 0xffffffffu;
      pp[u] = i < w_hi ? cpos[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kSweep; ++u) {
      if (i0 + u * kWave >= w_hi) break;   // uniform
      const int i = i0 + u * kWave + lane;
      const bool ok = i < w_hi;
      const uint32_t key = kk[u];
      const float v = key_score(key);
      const bool f0 = ok && key < kstar && v > thr;
      const bool f1 = ok && key < kstar && !(v > thr);
      const bool ft = ok && key == kstar;
      const uint64_t b0 = __ballot(f0), b1 = __ballot(f1), bt = __ballot(ft);
      const int t_before = rt + lanes_below(bt);
      int d = -1;
      if (f0) d = r0 + lanes_below(b0);
      if (f1) d = n0 + r1 + lanes_below(b1) + min(t_before, m);
      if (ft && t_before < m) d = n0 + r1 + lanes_below(b1) + t_before;
      if (d >= 0 && d < static_cast<int>(k)) dst_base[d] = pp[u];
      r0 += __popcll(b0);
      r1 += __popcll(b1);
      rt += __popcll(bt);
    }
  }
  if (stage) {
    __syncthreads();
    for (int e = tid; e < static_cast<int>(k); e += kTT) out[e] = st[e];
  }
}

}  // namespace

bool dsa_topk_two_stage(int64_t n, int32_t top_k) {
  const int64_t segs = (n + kTopkSeg - 1) / kTopkSeg;
  return n > top_k && segs >= 2 && segs <= kTopkMaxSegs && segs * top_k <= kTopkMaxCand;
}

hipError_t launch_dsa_topk_two_stage(const TopkParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_topk_bound_kernel, dim3(kPrMaxSegs, p.rows), dim3(kTT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dsa_topk_prune_kernel, dim3(kPrMaxSegs, p.rows), dim3(kTT), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dsa_topk_final_kernel, dim3(p.rows), dim3(kTT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dsa_topk(const TopkParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_topk_kernel, dim3(p.rows), dim3(kTT), 0, stream, p);
  return hipGetLastError();
}

// The candidate areas of mla_dsa_topk_select_noalloc: a fixed array in device
// memory (each device holds its own copy for the life of the process), so that
// entry allocates nothing.  Every call on a device shares it: calls that
// overlap on one device race.  Host code never passes the array's name to a
// kernel (in host code it is a host-side stand-in): the address on the current
// device comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) char scratch[static_cast<size_t>(kTopkNoAllocRows) * kTopkRowWsBytes];

hipError_t dsa_topk_scratch(char** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<char*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace mla
