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
// Two-stage form for rows of 2 to 8 segments of 16384 scores (the 131072-
// score rows of a long context), in two launches with a caller workspace:
//   A. one workgroup per (row, segment): the segment's keys go to LDS, the
//      same radix select finds the segment's top_k under the page's order
//      (key, then position), and an order-keeping compaction writes those
//      top_k (key, position) pairs to the workspace in ascending position
//      order.  A position the whole row selects has fewer than top_k
//      predecessors in the row, so fewer in its segment: the segments'
//      candidates contain the row's selection.
//   B. one workgroup per row: the candidates of the segments (one contiguous
//      run, ascending positions) go to LDS, and the select and the two sweeps of
//      the one-workgroup form run over them (the score of a candidate is its
//      key mapped back, bit for bit).
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
  uint32_t incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
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
  __shared__ uint32_t s_wtot[kTW];
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
    locate_digit(hist, nb, rank, prefix, shift, &s_prefix, &s_rank, s_wtot);
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

// ---- two-stage form.  Workspace of launch row i (kTopkRowWsBytes): keys of
// the candidates [kTopkMaxCand] uint32, their positions [kTopkMaxCand] int32,
// then the candidate count of each segment [kTopkMaxSegs] int32.  Segment s
// writes its candidates from s * top_k.
__device__ __forceinline__ uint32_t* ws_keys(const TopkParams& p, int i) {
  return reinterpret_cast<uint32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes);
}
__device__ __forceinline__ int32_t* ws_pos(const TopkParams& p, int i) {
  return reinterpret_cast<int32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes + kTopkMaxCand * 4);
}
__device__ __forceinline__ int32_t* ws_cnt(const TopkParams& p, int i) {
  return reinterpret_cast<int32_t*>(p.ws + static_cast<size_t>(i) * kTopkRowWsBytes + kTopkMaxCand * 8);
}

// A: the top_k of one segment, written in ascending position order.
__global__ __launch_bounds__(kTT) void dsa_topk_segment_kernel(TopkParams p) {
  const int seg = blockIdx.x, i_row = blockIdx.y;
  const int n = p.len[i_row];
  const int lo = seg * kTopkSeg;
  if (lo >= n) return;   // the row has fewer segments (uniform)
  const int len = min(kTopkSeg, n - lo);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float* sc = p.scores + static_cast<int64_t>(p.row[i_row]) * p.stride + lo;
  const uint32_t k = static_cast<uint32_t>(p.top_k);
  uint32_t* out_key = ws_keys(p, i_row) + static_cast<int64_t>(seg) * p.top_k;
  int32_t* out_pos = ws_pos(p, i_row) + static_cast<int64_t>(seg) * p.top_k;

  __shared__ uint32_t keys[kTopkSeg];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_prefix, s_rank;
  __shared__ uint32_t s_wtot[kTW];
  __shared__ int s_tot[2][kTW];
  {
    // every load of the thread in flight before the first LDS store
    float v[kTopkSeg / kTT];
#pragma unroll
    for (int u = 0; u < kTopkSeg / kTT; ++u) {
      const int i = u * kTT + tid;
      v[u] = i < len ? sc[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kTopkSeg / kTT; ++u) {
      const int i = u * kTT + tid;
      if (i < len) keys[i] = rank_key(v[u]);
    }
  }
  __syncthreads();
  if (static_cast<uint32_t>(len) <= k) {   // the whole segment is a candidate
    for (int i = tid; i < len; i += kTT) {
      out_key[i] = keys[i];
      out_pos[i] = lo + i;
    }
    if (tid == 0) ws_cnt(p, i_row)[seg] = len;
    return;
  }
  uint32_t kstar;
  int m;
  lds_radix_select(keys, len, k, hist, &s_prefix, &s_rank, s_wtot, kstar, m);
  // order-keeping compaction: wave w owns a run of positions; a selected
  // position lands at (keys below K* before it) + min(ties before it, m)
  const int per_wave = ((len + kTW - 1) / kTW + kWave - 1) / kWave * kWave;
  const int w_lo = min(len, wave * per_wave), w_hi = min(len, w_lo + per_wave);
  int cb = 0, ct = 0;
  for (int i0 = w_lo; i0 < w_hi; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t key = i < w_hi ? keys[i] : 0xffffffffu;
    cb += __popcll(__ballot(i < w_hi && key < kstar));
    ct += __popcll(__ballot(i < w_hi && key == kstar));
  }
  if (lane == 0) {
    s_tot[0][wave] = cb;
    s_tot[1][wave] = ct;
  }
  __syncthreads();
  int rb = 0, rt = 0;
  for (int w = 0; w < wave; ++w) {
    rb += s_tot[0][w];
    rt += s_tot[1][w];
  }
  for (int i0 = w_lo; i0 < w_hi; i0 += kWave) {
    const int i = i0 + lane;
    const bool ok = i < w_hi;
    const uint32_t key = ok ? keys[i] : 0xffffffffu;
    const bool fb = ok && key < kstar, ft = ok && key == kstar;
    const uint64_t bb = __ballot(fb), bt = __ballot(ft);
    const int b_before = rb + lanes_below(bb), t_before = rt + lanes_below(bt);
    int dst = -1;
    if (fb) dst = b_before + min(t_before, m);
    if (ft && t_before < m) dst = b_before + t_before;
    if (dst >= 0) {
      out_key[dst] = key;
      out_pos[dst] = lo + i;
    }
    rb += __popcll(bb);
    rt += __popcll(bt);
  }
  if (tid == 0) ws_cnt(p, i_row)[seg] = p.top_k;
}

// B: the row's selection among the segments' candidates, in the page's order.
__global__ __launch_bounds__(kTT) void dsa_topk_merge_kernel(TopkParams p) {
  const int i_row = blockIdx.x;
  const int n = p.len[i_row];
  const int segs = (n + kTopkSeg - 1) / kTopkSeg;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t k = static_cast<uint32_t>(p.top_k);
  int32_t* out = p.sel_idx + p.out_off[i_row];

  __shared__ uint32_t ckey[kTopkMaxCand];
  __shared__ int32_t cpos[kTopkMaxCand];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_prefix, s_rank;
  __shared__ uint32_t s_wtot[kTW];
  __shared__ int s_tot[3][kTW];
  // Every segment but the last is longer than top_k (16384 > 8192 >= top_k)
  // and wrote exactly top_k candidates from s * top_k, so the candidates are
  // one contiguous run of (segs - 1) * top_k + the last segment's count.
  const int c_total = (segs - 1) * p.top_k + ws_cnt(p, i_row)[segs - 1];
  {
    const uint32_t* ks = ws_keys(p, i_row);
    const int32_t* ps = ws_pos(p, i_row);
    uint32_t kv[kTopkMaxCand / kTT];
    int32_t pv[kTopkMaxCand / kTT];
#pragma unroll
    for (int u = 0; u < kTopkMaxCand / kTT; ++u) {
      const int i = u * kTT + tid;
      kv[u] = i < c_total ? ks[i] : 0u;
      pv[u] = i < c_total ? ps[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kTopkMaxCand / kTT; ++u) {
      const int i = u * kTT + tid;
      if (i < c_total) {
        ckey[i] = kv[u];
        cpos[i] = pv[u];
      }
    }
  }
  __syncthreads();
  uint32_t kstar;
  int m;
  lds_radix_select(ckey, c_total, k, hist, &s_prefix, &s_rank, s_wtot, kstar, m);
  const float thr = key_score(kstar);

  // the sweeps of the one-workgroup form over the candidates (ascending
  // positions): class 0 (key < K*, score > threshold), class 1 (other keys
  // below K*) and ties (key == K*, the first m selected)
  const int per_wave = ((c_total + kTW - 1) / kTW + kWave - 1) / kWave * kWave;
  const int w_lo = min(c_total, wave * per_wave), w_hi = min(c_total, w_lo + per_wave);
  int c0 = 0, c1 = 0, ct = 0;
  for (int i0 = w_lo; i0 < w_hi; i0 += kWave) {
    const int i = i0 + lane;
    const bool ok = i < w_hi;
    const uint32_t key = ok ? ckey[i] : 0xffffffffu;
    const float v = key_score(key);
    c0 += __popcll(__ballot(ok && key < kstar && v > thr));
    c1 += __popcll(__ballot(ok && key < kstar && !(v > thr)));
    ct += __popcll(__ballot(ok && key == kstar));
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
  for (int i0 = w_lo; i0 < w_hi; i0 += kWave) {
    const int i = i0 + lane;
    const bool ok = i < w_hi;
    const uint32_t key = ok ? ckey[i] : 0xffffffffu;
    const float v = key_score(key);
    const bool f0 = ok && key < kstar && v > thr;
    const bool f1 = ok && key < kstar && !(v > thr);
    const bool ft = ok && key == kstar;
    const uint64_t b0 = __ballot(f0), b1 = __ballot(f1), bt = __ballot(ft);
    const int t_before = rt + lanes_below(bt);
    const int pos = ok ? cpos[i] : 0;
    if (f0) out[r0 + lanes_below(b0)] = pos;
    if (f1) out[n0 + r1 + lanes_below(b1) + min(t_before, m)] = pos;
    if (ft && t_before < m) out[n0 + r1 + lanes_below(b1) + t_before] = pos;
    r0 += __popcll(b0);
    r1 += __popcll(b1);
    rt += __popcll(bt);
  }
}

}  // namespace

bool dsa_topk_two_stage(int64_t n, int32_t top_k) {
  const int64_t segs = (n + kTopkSeg - 1) / kTopkSeg;
  return n > top_k && segs >= 2 && segs <= kTopkMaxSegs && segs * top_k <= kTopkMaxCand;
}

hipError_t launch_dsa_topk_two_stage(const TopkParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_topk_segment_kernel, dim3(kTopkMaxSegs, p.rows), dim3(kTT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dsa_topk_merge_kernel, dim3(p.rows), dim3(kTT), 0, stream, p);
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
