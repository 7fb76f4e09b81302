// Reconstructed causal prefill, any geometry, fp32 or bf16 storage (page
// "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts: Glm52Mla.project for q_b_proj and
// the q RoPE, attendReconstructed for the kv_b_proj expansion, causal mask,
// softmax and P.V; page "mlx-bun 0.2.0 -> 0.4.0": left-padding mask).
//
// Three passes over a fp32 workspace:
//   1. Q  [B,T,H,dn+dr] = q_c . w_q_b^T       (tiled GEMM, both operands K-contiguous)
//      KV [B,K,H,dn+dv] = latent . w_kv_b^T
//   2. RoPE of Q's rope slice in place at q_offsets[b] + t
//   3. one workgroup per (query, head, row): online-softmax attention over the
//      visible keys left_pad[b] <= k <= (K - T) + t.
// The bf16 geometry of the GLM workload has an MFMA implementation instead.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

hipError_t launch_gemm_nt_generic(int32_t dtype, const void* a, int64_t lda, const void* b, int64_t ldb,
                                  float* c, int64_t ldc, int64_t m, int64_t n, int64_t k, hipStream_t stream);

namespace {

constexpr int kGT = 64;     // GEMM tile (M and N)
constexpr int kGK = 16;     // GEMM K step

// C[m, n] = sum_k A[m, k] B[n, k]; 256 threads, each a 4x4 block of the 64x64 tile.
template <typename T>
__global__ __launch_bounds__(256) void gemm_nt_generic_kernel(const T* __restrict__ a, int64_t lda,
                                                              const T* __restrict__ b, int64_t ldb,
                                                              float* __restrict__ c, int64_t ldc,
                                                              int64_t m, int64_t n, int64_t k) {
  __shared__ float as[kGK][kGT + 1];
  __shared__ float bs[kGK][kGT + 1];
  const int tid = threadIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kGT;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kGT;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < k; k0 += kGK) {
    for (int e = tid; e < kGT * kGK; e += 256) {
      const int r = e / kGK, kk = e % kGK;
      const int64_t gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      as[kk][r] = (gm < m && gk < k) ? ld(a + gm * lda + gk) : 0.f;
      bs[kk][r] = (gn < n && gk < k) ? ld(b + gn * ldb + gk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = as[kk][tm + i]; bv[i] = bs[kk][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gm = m0 + tm + i, gn = n0 + tn + j;
      if (gm < m && gn < n) c[gm * ldc + gn] = acc[i][j];
    }
}

constexpr int kAT = 256;
constexpr int kMaxQK = 256;
constexpr int kRowsPerLaunch = 128;

struct AttnParams {
  const float* q;        // [B,T,H,qk] fp32, rope part rotated
  const float* kv;       // [B,K,H,dn+dv] fp32
  const void* rope;      // [B,K,dr] storage type, rotated keys
  float* ctx;            // [B,T,H*dv]
  int32_t rows, tokens, keys, heads, dn, dr, dv;
  float scale;
  int32_t pad[kRowsPerLaunch];
};

template <typename T>
__global__ __launch_bounds__(kAT) void prefill_attn_generic_kernel(AttnParams p) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int qk = p.dn + p.dr, kvw = p.dn + p.dv;
  __shared__ float q_s[kMaxQK];
  __shared__ float w_s[kAT];
  __shared__ float red[kAT / kWave];
  const float* q = p.q + ((static_cast<int64_t>(b) * p.tokens + t) * p.heads + h) * qk;
  for (int d = tid; d < qk; d += kAT) q_s[d] = q[d];
  __syncthreads();
  const int k_lo = p.pad[b];
  const int k_hi = p.keys - p.tokens + t;     // inclusive
  const float* kvb = p.kv + static_cast<int64_t>(b) * p.keys * p.heads * kvw + static_cast<int64_t>(h) * kvw;
  const T* rope = static_cast<const T*>(p.rope) + static_cast<int64_t>(b) * p.keys * p.dr;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int kt = k_lo; kt <= k_hi; kt += kAT) {
    const int kk = kt + tid;
    float score = -INFINITY;
    if (kk <= k_hi) {
      const float* kn = kvb + static_cast<int64_t>(kk) * p.heads * kvw;
      const T* kr = rope + static_cast<int64_t>(kk) * p.dr;
      float acc = 0.f;
      for (int d = 0; d < p.dn; ++d) acc = fmaf(q_s[d], kn[d], acc);
      for (int d = 0; d < p.dr; ++d) acc = fmaf(q_s[p.dn + d], ld(kr + d), acc);
      score = acc * p.scale;
    }
    const float tmax = block_reduce(score, MaxOp(), red);
    const float m_new = fmaxf(m, tmax);
    const float pj = kk <= k_hi ? expf(score - m_new) : 0.f;
    const float alpha = m == -INFINITY ? 0.f : expf(m - m_new);
    w_s[tid] = pj;
    const float tsum = block_reduce(pj, SumOp(), red);
    l = l * alpha + tsum;
    if (tid < p.dv) {
      float acc = o * alpha;
      const int nt = min(kAT, k_hi - kt + 1);
      for (int j = 0; j < nt; ++j)
        acc = fmaf(w_s[j], kvb[static_cast<int64_t>(kt + j) * p.heads * kvw + p.dn + tid], acc);
      o = acc;
    }
    m = m_new;
    __syncthreads();
  }
  if (tid < p.dv)
    p.ctx[(static_cast<int64_t>(b) * p.tokens + t) * p.heads * p.dv + static_cast<int64_t>(h) * p.dv + tid] =
        l > 0.f ? o / l : 0.f;
}

}  // namespace

hipError_t launch_gemm_nt_generic(int32_t dtype, const void* a, int64_t lda, const void* b, int64_t ldb,
                                  float* c, int64_t ldc, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((n + kGT - 1) / kGT), static_cast<uint32_t>((m + kGT - 1) / kGT));
  if (dtype == kBF16)
    hipLaunchKernelGGL(gemm_nt_generic_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b), ldb, c, ldc, m, n, k);
  else
    hipLaunchKernelGGL(gemm_nt_generic_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(a), lda, static_cast<const float*>(b), ldb, c, ldc, m, n, k);
  return hipGetLastError();
}

size_t prefill_generic_workspace_bytes(const PrefillParams& p) {
  const size_t q = static_cast<size_t>(p.batch) * p.tokens * p.heads * (p.dn + p.dr) * sizeof(float);
  const size_t kv = static_cast<size_t>(p.batch) * p.keys * p.heads * (p.dn + p.dv) * sizeof(float);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(q) + up(kv);
}

hipError_t launch_prefill_generic(const PrefillParams& p, hipStream_t stream) {
  const int qk = p.dn + p.dr, kvw = p.dn + p.dv;
  const size_t q_bytes = static_cast<size_t>(p.batch) * p.tokens * p.heads * qk * sizeof(float);
  float* q = static_cast<float*>(p.workspace);
  float* kv = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + (q_bytes + 255) / 256 * 256);
  const size_t es = p.dtype == kBF16 ? 2 : 4;
  hipError_t e;
  e = launch_gemm_nt_generic(p.dtype, p.q_c, p.ql, p.w_qb, p.ql, q, static_cast<int64_t>(p.heads) * qk,
                             static_cast<int64_t>(p.batch) * p.tokens, static_cast<int64_t>(p.heads) * qk, p.ql,
                             stream);
  if (e != hipSuccess) return e;
  e = launch_gemm_nt_generic(p.dtype, p.latent, p.r, p.w_kvb, p.r, kv, static_cast<int64_t>(p.heads) * kvw,
                             static_cast<int64_t>(p.batch) * p.keys, static_cast<int64_t>(p.heads) * kvw, p.r,
                             stream);
  if (e != hipSuccess) return e;
  // RoPE of the rope slice of Q: logical [B, T, H, dr] at q + dn.
  RopeParams rp{};
  rp.tokens = p.tokens;
  rp.inner = p.heads;
  rp.feat = p.dr;
  rp.st = static_cast<int64_t>(p.heads) * qk;
  rp.si = qk;
  rp.sb = static_cast<int64_t>(p.tokens) * p.heads * qk;
  rp.rotary = p.dr;
  rp.per_row = 1;
  rp.copy_tail = 0;
  rope_inverse_frequencies(p.dr, p.theta, rp.inv);
  for (int b0 = 0; b0 < p.batch; b0 += kRopeRowsPerLaunch) {
    rp.rows = p.batch - b0 < kRopeRowsPerLaunch ? p.batch - b0 : kRopeRowsPerLaunch;
    rp.x = rp.y = q + b0 * rp.sb + p.dn;
    for (int i = 0; i < rp.rows; ++i) rp.off[i] = p.q_offsets[b0 + i];
    e = launch_rope(kF32, rp, stream);
    if (e != hipSuccess) return e;
  }
  AttnParams ap{};
  ap.tokens = p.tokens;
  ap.keys = p.keys;
  ap.heads = p.heads;
  ap.dn = p.dn;
  ap.dr = p.dr;
  ap.dv = p.dv;
  ap.scale = p.scale;
  for (int b0 = 0; b0 < p.batch; b0 += kRowsPerLaunch) {
    ap.rows = p.batch - b0 < kRowsPerLaunch ? p.batch - b0 : kRowsPerLaunch;
    ap.q = q + static_cast<int64_t>(b0) * p.tokens * p.heads * qk;
    ap.kv = kv + static_cast<int64_t>(b0) * p.keys * p.heads * kvw;
    ap.rope = static_cast<const char*>(p.rope) + static_cast<int64_t>(b0) * p.keys * p.dr * es;
    ap.ctx = p.ctx + static_cast<int64_t>(b0) * p.tokens * p.heads * p.dv;
    for (int i = 0; i < ap.rows; ++i) ap.pad[i] = p.left_pad ? p.left_pad[b0 + i] : 0;
    dim3 grid(p.tokens, p.heads, ap.rows);
    if (p.dtype == kBF16)
      hipLaunchKernelGGL(prefill_attn_generic_kernel<uint16_t>, grid, dim3(kAT), 0, stream, ap);
    else
      hipLaunchKernelGGL(prefill_attn_generic_kernel<float>, grid, dim3(kAT), 0, stream, ap);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
