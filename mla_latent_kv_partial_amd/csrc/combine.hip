// Merge of split-T decode partials: the exact log-sum-exp decomposition of
// the page's per-head softmax (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts,
// attendAbsorbed).  For row b, head h over its n_b splits:
//   LSE = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) o_s.
// One workgroup of 512 threads per (head, row).  The partials of one
// (row, head) are contiguous [n_b, r] (fp32 or bf16).  Four groups of 128
// threads split the splits (group j takes s = j mod 4); a thread owns four
// consecutive latent features and loads 16 splits (their lse and partials)
// at a time, all in flight together.  Every thread of a group reads the same
// lse values, so each keeps the group's running (max, sum of weights) itself
// and weights its partials at once: no block-wide log-sum-exp reduction sits
// between the loads and the accumulation.  The four groups' (max, sum,
// partial sums) then meet in LDS once.
//
// With a value projection (mla_decode_combine_v) the merged latent context of
// the (head, row) stays in LDS and the same workgroup projects it through the
// head's value block ([P1] attendAbsorbed: ctx_h = o_lat_h . W_UV[h]^T).  For
// bf16 weights with r a multiple of 64 up to 512 and dv <= 128, eight threads
// share one output column: each reads 16-byte pieces of the column's weight
// row (the eight together read 128 contiguous bytes per load), and the eight
// partial dot products meet by lane shuffles.  Workgroup ids run head
// fastest, so with a head count divisible by 8 every row of one head lands on
// the same XCD and its weight block is fetched from HBM once.
#include <math.h>

#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kGroups = 4;
constexpr int kGroupThreads = kThreads / kGroups;
constexpr int kUnroll = 16;
constexpr int kMaxSplitsLds = 4096;
constexpr int kMaxRankLds = 1024;    // latent context kept in LDS for the projection

// Value projection after the merge: none, any weight dtype (one thread per
// output column), or the bf16 fast path (eight threads per column).
enum VMode : int { kVNone = 0, kVGeneric = 1, kVFastBf16 = 2 };
constexpr int kFastCols = kThreads / 8;   // output columns per pass of the fast path
constexpr int kFastPasses = 2;            // dv <= 128
constexpr int kFastLoads = 8;             // r / 64 <= 8

// (m, l) with l = sum exp(v - m) over the values seen; m = -inf means none.
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;
  l = (m == -INFINITY ? 0.f : l * expf(m - mx)) + (m2 == -INFINITY ? 0.f : l2 * expf(m2 - mx));
  m = mx;
}

__device__ __forceinline__ float split_weight(float v, float m) {
  return (m == -INFINITY || v == -INFINITY) ? 0.f : expf(v - m);
}

// Four consecutive partial features as fp32: one 16-byte load of fp32
// partials, or one 8-byte load of bf16 partials (widened exactly).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// a split with no valid token (weight 0) adds nothing, whatever its partial holds
__device__ __forceinline__ void fma4(float4& acc, float w, const float4& v) {
  if (w == 0.f) return;
  acc.x = fmaf(w, v.x, acc.x);
  acc.y = fmaf(w, v.y, acc.y);
  acc.z = fmaf(w, v.z, acc.z);
  acc.w = fmaf(w, v.w, acc.w);
}

constexpr float kLog2e = 1.4426950408889634f;

// exp(x - m) for x <= m; 0 for x = -inf
__device__ __forceinline__ float weight_of(float x, float m) {
  return x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// The splits s = grp + 4 k of one (row, head), features c .. c + 3, in
// batches of kUnroll: Mg = their max lse, lg = sum exp(lse_s - Mg) and
// acc = sum exp(lse_s - Mg) o_s (Mg = -inf: no split with a token).  Every
// thread of the group reads the same lse values, so Mg and lg agree across
// the group.  The first batch (lse in ls, partials in v) is loaded by the
// caller; its entries past n hold lse -inf.
template <typename PT>
__device__ __forceinline__ void group_merge(const PT* po, const float* lse_in, int n, int r, int c, int grp,
                                            float (&ls)[kUnroll], float4 (&v)[kUnroll], float& Mg, float& lg,
                                            float4& acc) {
  Mg = -INFINITY;
  lg = 0.f;
  acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = grp; s0 < n; s0 += kGroups * kUnroll) {
    if (s0 > grp) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int sc = min(s0 + kGroups * u, n - 1);
        ls[u] = s0 + kGroups * u < n ? lse_in[sc] : -INFINITY;
        v[u] = load4(po + static_cast<int64_t>(sc) * r + c);
      }
    }
    float bm = ls[0];
#pragma unroll
    for (int u = 1; u < kUnroll; ++u) bm = fmaxf(bm, ls[u]);
    const float mn = fmaxf(Mg, bm);
    if (mn == -INFINITY) continue;   // no token in these splits yet (same in the whole group)
    const float rs = weight_of(Mg, mn);
    acc.x *= rs; acc.y *= rs; acc.z *= rs; acc.w *= rs;
    lg *= rs;
    Mg = mn;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = weight_of(ls[u], Mg);
      lg += w;
      fma4(acc, w, v[u]);
    }
  }
}

// The first batch of group_merge: lse and partials of splits grp + 4 u,
// clamped to a valid split (entries past n get lse -inf; their partials are
// loaded but never used, which keeps the loads free of branches).
template <typename PT>
__device__ __forceinline__ void first_batch(const PT* po, const float* lse_in, int n, int r, int c, int grp,
                                            float (&ls)[kUnroll], float4 (&v)[kUnroll]) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int sc = min(grp + kGroups * u, n - 1);
    ls[u] = lse_in[sc];
    v[u] = load4(po + static_cast<int64_t>(sc) * r + c);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (grp + kGroups * u >= n) ls[u] = -INFINITY;
}

// The four groups' merges meet: group 0 thread gt combines them (gm, gl: the
// groups' max and sum, part: groups 1..3's partial sums) into the merged
// features (o) and the log-sum-exp.
__device__ __forceinline__ void meet_groups(const float* gm, const float* gl, const float4* p1, const float4* p2,
                                            const float4* p3, float4 acc, float4& o, float& lse) {
  float m = gm[0];
#pragma unroll
  for (int g = 1; g < kGroups; ++g) m = fmaxf(m, gm[g]);
  if (m == -INFINITY) {
    o = make_float4(0.f, 0.f, 0.f, 0.f);
    lse = -INFINITY;
    return;
  }
  const float f0 = weight_of(gm[0], m), f1 = weight_of(gm[1], m), f2 = weight_of(gm[2], m), f3 = weight_of(gm[3], m);
  const float4 a1 = *p1, a2 = *p2, a3 = *p3;
  const float l = f0 * gl[0] + f1 * gl[1] + f2 * gl[2] + f3 * gl[3];
  const float inv = 1.f / l;
  o.x = (f0 * acc.x + f1 * a1.x + f2 * a2.x + f3 * a3.x) * inv;
  o.y = (f0 * acc.y + f1 * a1.y + f2 * a2.y + f3 * a3.y) * inv;
  o.z = (f0 * acc.z + f1 * a1.z + f2 * a2.z + f3 * a3.z) * inv;
  o.w = (f0 * acc.w + f1 * a1.w + f2 * a2.w + f3 * a3.w) * inv;
  lse = m + logf(l);
}

// Two workgroups per CU (at most 128 VGPRs): the (head, row) grid of a decode
// step then runs in one round.
// PT: the partials' storage type (float, or uint16_t for bf16 bits).
template <typename PT, bool VEC, int VM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void combine_kernel(CombineParams p) {
  constexpr int kU = kUnroll;   // batch of partial loads per thread
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const PT* po = static_cast<const PT*>(p.part_o) + bh * p.s_max * p.r;
  __shared__ float red_m[kWaves], red_l[kWaves];
  __shared__ float ws[kMaxSplitsLds];   // split lse, then split weights
  __shared__ float4 grp_s[kGroups - 1][kGroupThreads];
  __shared__ __attribute__((aligned(16))) float o_sh[VM != kVNone ? kMaxRankLds : 1];   // merged o_lat

  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);
  const int gt = tid % kGroupThreads;

  // Fast projection: this thread's weight pieces.  Thread (jj, q) of column
  // j = jj + 64 pass reads elements 8 (8u + q) .. +8 of the column's weight
  // row; columns past dv read the last column (never stored).  They are
  // requested after the merge (the weight block of a head is shared by the
  // rows' workgroups on one XCD, mostly from L2), so the merge keeps its
  // registers for partial loads.
  f32x4 wv[kFastPasses][kFastLoads];
  const int fq = tid & 7, fjj = tid >> 3;
  auto load_weights = [&]() {
    const uint16_t* w = static_cast<const uint16_t*>(p.w);
    const int nu = p.r / 64;
#pragma unroll
    for (int ps = 0; ps < kFastPasses; ++ps) {
      const int j = min(fjj + kFastCols * ps, p.dv - 1);
      const uint16_t* row = w + (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + j) * p.r;
#pragma unroll
      for (int u = 0; u < kFastLoads; ++u)
        if (u < nu) wv[ps][u] = *reinterpret_cast<const f32x4*>(row + 8 * (8 * u + fq));
    }
  };

  if constexpr (VEC) {
    __shared__ float gm_s[kGroups], gl_s[kGroups];
    for (int c0 = 0; c0 < p.r; c0 += 4 * kGroupThreads) {
      const bool own = c0 + 4 * gt < p.r;
      const int c = min(c0 + 4 * gt, p.r - 4);
      float ls[kU];
      float4 v[kU];
      first_batch(po, lse_in, n, p.r, c, grp, ls, v);
      float mg, lg;
      float4 acc;
      group_merge(po, lse_in, n, p.r, c, grp, ls, v, mg, lg, acc);
      if (grp > 0) grp_s[grp - 1][gt] = acc;
      if (gt == 0) {
        gm_s[grp] = mg;
        gl_s[grp] = lg;
      }
      __syncthreads();
      if (grp == 0) {
        float4 o;
        float lse;
        meet_groups(gm_s, gl_s, &grp_s[0][gt], &grp_s[1][gt], &grp_s[2][gt], acc, o, lse);
        if (own) {
          if (p.o_lat) *reinterpret_cast<float4*>(p.o_lat + bh * p.r + c) = o;
          if constexpr (VM != kVNone) *reinterpret_cast<float4*>(o_sh + c) = o;
        }
        if (c0 == 0 && gt == 0 && p.lse) p.lse[bh] = lse;
      }
      __syncthreads();
    }
  } else {
    // ---- scalar path: LSE over the splits (per-thread (max, sum) pairs,
    // waves, LDS), split weights in LDS, one thread per feature
    const float lse0 = tid < n ? lse_in[tid] : -INFINITY;
    float m = lse0, l = lse0 == -INFINITY ? 0.f : 1.f;
    if (tid < n && tid < kMaxSplitsLds) ws[tid] = lse0;
    for (int s = tid + kThreads; s < n; s += kThreads) {
      const float x = lse_in[s];
      if (s < kMaxSplitsLds) ws[s] = x;
      lse_merge(m, l, x, 1.f);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off, kWave), l2 = __shfl_xor(l, off, kWave);
      lse_merge(m, l, m2, l2);
    }
    if (lane == 0) {
      red_m[wave] = m;
      red_l[wave] = l;
    }
    __syncthreads();
    m = red_m[0];
    l = red_l[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) lse_merge(m, l, red_m[w], red_l[w]);
    if (tid < n && tid < kMaxSplitsLds) ws[tid] = split_weight(lse0, m);
    for (int s = tid + kThreads; s < min(n, kMaxSplitsLds); s += kThreads) ws[s] = split_weight(ws[s], m);
    __syncthreads();
    auto weight = [&](int s) { return s < kMaxSplitsLds ? ws[s] : split_weight(lse_in[s], m); };
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int c = tid; c < p.r; c += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < n; ++s) {
        const float w = weight(s);
        if (w != 0.f) acc = fmaf(w, ld(po + static_cast<int64_t>(s) * p.r + c), acc);
      }
      if (p.o_lat) p.o_lat[bh * p.r + c] = acc * inv;
      if constexpr (VM != kVNone) o_sh[c] = acc * inv;
    }
    if (p.lse && tid == 0) p.lse[bh] = l > 0.f ? m + logf(l) : -INFINITY;
  }
  if constexpr (VM == kVNone) return;
  __syncthreads();   // o_sh complete

  // ---- value projection: ctx[b, h dv + j] = sum_c o_lat[c] W_UV[h][j][c]
  float* ctx = p.ctx + static_cast<int64_t>(b) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv;
  if constexpr (VM == kVFastBf16) {
    load_weights();
    const int nu = p.r / 64;
#pragma unroll
    for (int ps = 0; ps < kFastPasses; ++ps) {
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < kFastLoads; ++u) {
        if (u < nu) {
          const float4* o4 = reinterpret_cast<const float4*>(o_sh + 8 * (8 * u + fq));
          const float4 o0 = o4[0], o1 = o4[1];
          const f32x4 wb = wv[ps][u];   // 8 bf16: element 2i in the low half of word i
          const uint32_t w0 = __float_as_uint(wb[0]), w1 = __float_as_uint(wb[1]);
          const uint32_t w2 = __float_as_uint(wb[2]), w3 = __float_as_uint(wb[3]);
          acc = fmaf(o0.x, __uint_as_float(w0 << 16), acc);
          acc = fmaf(o0.y, __uint_as_float(w0 & 0xffff0000u), acc);
          acc = fmaf(o0.z, __uint_as_float(w1 << 16), acc);
          acc = fmaf(o0.w, __uint_as_float(w1 & 0xffff0000u), acc);
          acc = fmaf(o1.x, __uint_as_float(w2 << 16), acc);
          acc = fmaf(o1.y, __uint_as_float(w2 & 0xffff0000u), acc);
          acc = fmaf(o1.z, __uint_as_float(w3 << 16), acc);
          acc = fmaf(o1.w, __uint_as_float(w3 & 0xffff0000u), acc);
        }
      }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      acc += __shfl_xor(acc, 4, kWave);
      const int j = fjj + kFastCols * ps;
      if (fq == 0 && j < p.dv) ctx[j] = acc;
    }
  } else {
    for (int j = tid; j < p.dv; j += kThreads) {
      const int64_t row = (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + j) * p.r;
      float acc = 0.f;
      if (p.w_dtype == kBF16) {
        const uint16_t* w = static_cast<const uint16_t*>(p.w) + row;
        for (int c = 0; c < p.r; ++c) acc = fmaf(o_sh[c], bf16_to_f32(w[c]), acc);
      } else {
        const float* w = static_cast<const float*>(p.w) + row;
        for (int c = 0; c < p.r; ++c) acc = fmaf(o_sh[c], w[c], acc);
      }
      ctx[j] = acc;
    }
  }
}

// ---- The fused merge + projection for bf16 weights, kv_lora_rank 512 and
// v_head <= 128 (the decode step's combine_v): one workgroup of 1024 threads
// per (head, pair of rows).  Each half of the workgroup merges one row as
// combine_kernel does, while the head's value block (v_head weight rows of
// 1 KB) streams into LDS by global_load_lds copies issued right behind the
// merge's first loads: wave v < 8 copies rows 16 v .. 16 v + 15 and then
// projects exactly those 16 output columns for both rows on MFMA, as soon as
// its own copies have landed (no wait for the whole block).  Against one
// workgroup per (head, row) this fetches each value block once per row pair
// rather than per row.  Workgroup ids run head fastest: the row pairs of a
// head share an XCD and its L2.
constexpr int kPairThreads = 2 * kThreads;
constexpr int kPairR = 512;
constexpr int kWRowBytes = kPairR * 2 + 32;    // weight row in LDS: an odd number of 32-byte units
constexpr int kPairMaxDv = 128;

__shared__ __attribute__((aligned(1024))) char g_w[kPairMaxDv * kWRowBytes];

template <typename PT>
__global__ __launch_bounds__(kPairThreads) void combine_v_pair_kernel(CombineParams p) {
  constexpr int kU = kUnroll;
  const int h = blockIdx.x;
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x / kThreads);
  const int tid = threadIdx.x % kThreads;   // thread of this half
  const int lane = tid & (kWave - 1);
  const int b_want = 2 * blockIdx.y + half;
  const bool real = b_want < p.rows;
  const int b = real ? b_want : p.rows - 1;   // a missing second row merges the last row again, unstored
  const int n = p.n_splits[b];
  const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
  const float* lse_in = p.part_lse + bh * p.s_max;
  const PT* po = static_cast<const PT*>(p.part_o) + bh * p.s_max * kPairR;
  __shared__ float gm_s[2][kGroups], gl_s[2][kGroups];
  __shared__ float4 grp_all[2][kGroups - 1][kGroupThreads];   // group sums, then the projection's partial sums
  // the merged rows as MFMA operands: bf16 high part and bf16 residual
  __shared__ __attribute__((aligned(16))) __bf16 o_hi[2][kPairR];
  __shared__ __attribute__((aligned(16))) __bf16 o_lo[2][kPairR];

  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);
  const int gt = tid % kGroupThreads;
  const int c = 4 * gt;   // this thread's four latent features (kPairR = 4 x 128)

  // the merge's first batch (lse and partials of 16 splits per thread), then
  // the value block behind it: weight row j (output column j) to
  // g_w + j * kWRowBytes, one 1 KB copy per row; wave v of the workgroup copies
  // rows v, v + 16, ...  (the compiler's waits for the merge's loads count
  // only its own loads, so they also wait for some of the copies issued after
  // them: safe, and nothing the merge waits for lies behind the copies)
  float ls[kU];
  float4 v[kU];
  first_batch(po, lse_in, n, kPairR, c, grp, ls, v);
  const int wgw = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (wgw < kPairMaxDv / 16) {
    // wave v < 8 copies weight rows 16 v .. 16 v + 15 (below dv), which only
    // it reads in the projection
    const uint16_t* wb = static_cast<const uint16_t*>(p.w) + (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn) * kPairR;
    for (int i = 0; i < 16; ++i) {
      const int j = 16 * wgw + i;
      if (j >= p.dv) break;
      dma16(wb + static_cast<int64_t>(j) * kPairR + 8 * lane, lds_addr(g_w) + j * kWRowBytes);
    }
  }
  float mg, lg;
  float4 acc;
  group_merge(po, lse_in, n, kPairR, c, grp, ls, v, mg, lg, acc);
  if (grp > 0) grp_all[half][grp - 1][gt] = acc;
  if (gt == 0) {
    gm_s[half][grp] = mg;
    gl_s[half][grp] = lg;
  }
  __syncthreads();
  if (grp == 0) {
    float4 o;
    float lse;
    meet_groups(gm_s[half], gl_s[half], &grp_all[half][0][gt], &grp_all[half][1][gt], &grp_all[half][2][gt], acc, o,
                lse);
    if (p.o_lat && real) *reinterpret_cast<float4*>(p.o_lat + bh * kPairR + c) = o;
    const float e[4] = {o.x, o.y, o.z, o.w};
    bf16x4 hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hi[q] = static_cast<__bf16>(e[q]);
      lo[q] = static_cast<__bf16>(e[q] - static_cast<float>(hi[q]));
    }
    *reinterpret_cast<bf16x4*>(&o_hi[half][c]) = hi;
    *reinterpret_cast<bf16x4*>(&o_lo[half][c]) = lo;
    if (p.lse && real && gt == 0) p.lse[bh] = lse;
  }
  __syncthreads();   // the merged rows are in LDS

  // ---- projection on MFMA, one 16-column block per wave (waves 0..7): the
  // wave waits for its own 16 weight rows only, so each block starts as soon
  // as its rows land.  A = the weight rows (16 columns x 32 latent features
  // per k-step), B = the two merged rows as a bf16 high part plus a bf16
  // residual (~16 significant bits), the other 14 columns of B zero.
  if (wgw < kPairMaxDv / 16 && 16 * wgw < p.dv) {
    wait_vm<0>();
    const int m = lane & 15, g = lane >> 4;
    const char* wrow = g_w + (16 * wgw + m) * kWRowBytes + 16 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < kPairR / 32; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow + 64 * ks);
      bf16x8 hi = {}, lo = {};
      if (m < 2) {
        hi = *reinterpret_cast<const bf16x8*>(&o_hi[m][32 * ks + 8 * g]);
        lo = *reinterpret_cast<const bf16x8*>(&o_lo[m][32 * ks + 8 * g]);
      }
      acc = mfma16x16x32(a, hi, acc);
      acc = mfma16x16x32(a, lo, acc);
    }
    // lane (m, g) holds columns 16 wgw + 4 g + (0..3) of pair row m
    const int bo = 2 * blockIdx.y + m;
    if (m < 2 && bo < p.rows) {
      float* dst = p.ctx + static_cast<int64_t>(bo) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv;
      const int col = 16 * wgw + 4 * g;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (col + ii < p.dv) dst[col + ii] = acc[ii];
    }
  }
}

// ---- The fused merge + projection for many rows (bf16 weights, r = 512,
// v_head <= 128): one workgroup of 16 waves per (head, block of 16 rows).
// The pair kernel fetches a head's value block once per two rows, which at
// 64 rows and more is 32+ fetches of each block through L2; here each block
// serves 16 rows.  Wave w merges row b0 + w alone (lane l owns latent
// features 8 l .. 8 l + 7), batches of 8 splits with all their loads in
// flight: rows of a many-row launch hold few splits each.  The merged rows go
// to LDS in fp32; the projection runs on MFMA with the merged row as a bf16
// high part plus a bf16 residual (~16 significant bits), wave (nt, kh)
// taking output columns 16 nt .. 16 nt + 15 over latent half kh, its weight
// fragments requested at entry so that they arrive during the merge.
constexpr int kRowsBlock = 16;
constexpr int kRowsThreads = kRowsBlock * kWave;
constexpr int kRowsBatch = 8;                      // splits per batch of loads
constexpr int kRowsStride = kPairR * 4 + 32;       // merged row in LDS: an odd number of 32-byte units
constexpr int kRowsMin = 16;                       // fewest rows that take this kernel

// eight consecutive partial features as fp32
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename PT>
__global__ __launch_bounds__(kRowsThreads) void combine_v_rows_kernel(CombineParams p) {
  __shared__ __attribute__((aligned(16))) char o_sh[kRowsBlock * kRowsStride];
  __shared__ float psum[kRowsBlock][kPairMaxDv];
  const int h = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int m = lane & 15, g = lane >> 4;
  const int b0 = blockIdx.y * kRowsBlock;

  // this wave's projection tile and its weight fragments (B[k][n] = W_UV[h][16 nt + n][k])
  const int nt = wave & 7, kh = wave >> 3;
  const bool proj = 16 * nt < p.dv;
  bf16x8 bw[8];
  if (proj) {
    const int col = min(16 * nt + m, p.dv - 1);   // columns past dv re-read the last one (never stored)
    const uint16_t* wr = static_cast<const uint16_t*>(p.w) +
                         (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + col) * kPairR + 256 * kh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bw[ks] = *reinterpret_cast<const bf16x8*>(wr + 32 * ks);
  }

  // ---- merge row b0 + wave
  const int b = b0 + wave;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, L = 0.f;
  if (b < p.rows) {
    const int n = p.n_splits[b];
    const int64_t bh = static_cast<int64_t>(b) * p.heads + h;
    const float* lse_in = p.part_lse + bh * p.s_max;
    const PT* po = static_cast<const PT*>(p.part_o) + bh * p.s_max * kPairR + 8 * lane;
    for (int s0 = 0; s0 < n; s0 += kRowsBatch) {
      float ls[kRowsBatch], v[kRowsBatch][8];
#pragma unroll
      for (int u = 0; u < kRowsBatch; ++u) {
        const int sc = min(s0 + u, n - 1);   // splits past n re-read the last one, weight 0
        ls[u] = lse_in[sc];
        load8(po + static_cast<int64_t>(sc) * kPairR, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kRowsBatch; ++u)
        if (s0 + u >= n) ls[u] = -INFINITY;
      float bm = ls[0];
#pragma unroll
      for (int u = 1; u < kRowsBatch; ++u) bm = fmaxf(bm, ls[u]);
      const float mn = fmaxf(M, bm);
      if (mn == -INFINITY) continue;   // no token in these splits yet
      const float rs = weight_of(M, mn);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= rs;
      L *= rs;
      M = mn;
#pragma unroll
      for (int u = 0; u < kRowsBatch; ++u) {
        const float w = weight_of(ls[u], M);
        L += w;
        if (w != 0.f) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[u][i], acc[i]);
        }
      }
    }
    float lse = -INFINITY;
    if (M != -INFINITY) {
      const float inv = 1.f / L;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= inv;
      lse = M + logf(L);
    }
    if (p.o_lat) {
      float* ol = p.o_lat + bh * kPairR + 8 * lane;
      *reinterpret_cast<float4*>(ol) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(ol + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    if (p.lse && lane == 0) p.lse[bh] = lse;
  }
  // rows past the launch stay zero: their projections are never stored
  float* orow = reinterpret_cast<float*>(o_sh + wave * kRowsStride) + 8 * lane;
  *reinterpret_cast<float4*>(orow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(orow + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();

  // ---- projection: ctx[b0 + row][16 nt + n] over latent half kh
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  if (proj) {
    const float* arow = reinterpret_cast<const float*>(o_sh + m * kRowsStride) + 256 * kh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float4 u = *reinterpret_cast<const float4*>(arow + 32 * ks);
      const float4 v = *reinterpret_cast<const float4*>(arow + 32 * ks + 4);
      const bf16x8 hi = to_bf16x8(u, v);
      const float4 ru = make_float4(u.x - static_cast<float>(hi[0]), u.y - static_cast<float>(hi[1]),
                                    u.z - static_cast<float>(hi[2]), u.w - static_cast<float>(hi[3]));
      const float4 rv = make_float4(v.x - static_cast<float>(hi[4]), v.y - static_cast<float>(hi[5]),
                                    v.z - static_cast<float>(hi[6]), v.w - static_cast<float>(hi[7]));
      c = mfma16x16x32(hi, bw[ks], c);
      c = mfma16x16x32(to_bf16x8(ru, rv), bw[ks], c);
    }
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) psum[4 * g + i][16 * nt + m] = c[i];
    }
  }
  __syncthreads();
  if (proj && kh == 0) {
    const int col = 16 * nt + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bo = b0 + 4 * g + i;
      if (bo < p.rows && col < p.dv)
        p.ctx[static_cast<int64_t>(bo) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv + col] =
            c[i] + psum[4 * g + i][col];
    }
  }
}

template <typename PT>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  // whole 4-feature partial groups from aligned bases (16 bytes fp32, 8 bf16)
  const uintptr_t pa = reinterpret_cast<uintptr_t>(p.part_o) & (4 * sizeof(PT) - 1);
  const bool vec = p.r >= 4 && (p.r & 3) == 0 && pa == 0 && (reinterpret_cast<uintptr_t>(p.o_lat) & 15) == 0;
  const dim3 grid(p.heads, p.rows), block(kThreads);
  if (!p.ctx) {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<PT, true, kVNone>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((combine_kernel<PT, false, kVNone>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  // the pair kernel: bf16 weights with r = 512, dv <= 128 (16-byte aligned weight rows)
  if (vec && p.w_dtype == kBF16 && p.r == kPairR && p.dv <= kPairMaxDv && (reinterpret_cast<uintptr_t>(p.w) & 15) == 0) {
    if (p.rows >= kRowsMin)
      hipLaunchKernelGGL((combine_v_rows_kernel<PT>), dim3(p.heads, (p.rows + kRowsBlock - 1) / kRowsBlock),
                         dim3(kRowsThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((combine_v_pair_kernel<PT>), dim3(p.heads, (p.rows + 1) / 2), dim3(kPairThreads), 0, stream, p);
    return hipGetLastError();
  }
  const bool fast = vec && p.w_dtype == kBF16 && p.r % 64 == 0 && p.r / 64 <= kFastLoads &&
                    p.dv <= kFastCols * kFastPasses && (reinterpret_cast<uintptr_t>(p.w) & 15) == 0;
  if (fast)
    hipLaunchKernelGGL((combine_kernel<PT, true, kVFastBf16>), grid, block, 0, stream, p);
  else if (vec)
    hipLaunchKernelGGL((combine_kernel<PT, true, kVGeneric>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((combine_kernel<PT, false, kVGeneric>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  return p.part_bf16 ? launch_combine_t<uint16_t>(p, stream) : launch_combine_t<float>(p, stream);
}

}  // namespace mla
