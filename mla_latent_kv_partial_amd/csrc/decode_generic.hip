// Latent decode attention, any geometry (kv_lora_rank <= 1024, rope <= 256),
// fp32 or bf16 storage: split-T partials of the page's absorbed decode
// (page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts, attendAbsorbed: scores =
// scale * (q_lat . latent + q_rope . rope), softmax, P . latent), with the
// DSA gather and the right-aligned ragged rows.
//
// One workgroup per (split, head, row); tokens of the split are walked in
// tiles of 256 with an online softmax kept in fp32.  This path serves small
// and unusual shapes; the bf16 r=512 / rope=64 geometry has an MFMA kernel.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kTile = 256;
constexpr int kMaxRank = 1024;
constexpr int kMaxRope = 256;
constexpr int kPerThread = kMaxRank / kTile;   // latent features per thread

template <typename T>
__global__ __launch_bounds__(kTile) void decode_generic_kernel(DecodeParams p) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int n_att = p.tab.n_att[b];
  const int n_split = (n_att + p.chunk - 1) / p.chunk;
  if (s >= n_split) return;
  const int j0 = s * p.chunk;
  const int j1 = min(n_att, j0 + p.chunk);
  const int len = p.tab.kv_len[b];
  const int sel_off = p.tab.sel_off[b];

  __shared__ float q_s[kMaxRank];
  __shared__ float qr_s[kMaxRope];
  __shared__ float w_s[kTile];
  __shared__ int slot_s[kTile];
  __shared__ float red[kTile / kWave];

  const T* ql = static_cast<const T*>(p.q_lat) + (static_cast<int64_t>(b) * p.heads + h) * p.r;
  const T* qr = static_cast<const T*>(p.q_rope) + b * p.qr_sb + h * p.qr_sh;
  for (int c = tid; c < p.r; c += kTile) q_s[c] = ld(ql + c);
  for (int c = tid; c < p.dr; c += kTile) qr_s[c] = ld(qr + c);
  __syncthreads();

  const T* lat = static_cast<const T*>(p.latent) + b * p.lat_sb;
  const T* rop = static_cast<const T*>(p.rope) + b * p.rope_sb;
  float m = -INFINITY, l = 0.f;
  float o[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) o[k] = 0.f;

  for (int jt = j0; jt < j1; jt += kTile) {
    const int j = jt + tid;
    float score = -INFINITY;
    int slot = -1;
    if (j < j1) {
      const int idx = sel_off < 0 ? j : p.sel[sel_off + j];
      if (idx >= 0 && idx < len) {
        slot = p.width - len + idx;
        const T* c = lat + static_cast<int64_t>(slot) * p.lat_st;
        const T* rr = rop + static_cast<int64_t>(slot) * p.rope_st;
        float acc = 0.f;
        for (int f = 0; f < p.r; ++f) acc = fmaf(q_s[f], ld(c + f), acc);
        for (int f = 0; f < p.dr; ++f) acc = fmaf(qr_s[f], ld(rr + f), acc);
        score = acc * p.scale;
      } else if (p.dev_err) {
        atomicOr(p.dev_err, 1);
      }
    }
    const float tmax = block_reduce(score, MaxOp(), red);
    const float m_new = fmaxf(m, tmax);
    const float pj = slot >= 0 ? expf(score - m_new) : 0.f;
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    w_s[tid] = pj;
    slot_s[tid] = slot;
    const float tsum = block_reduce(pj, SumOp(), red);   // also publishes w_s / slot_s
    l = l * alpha + tsum;
    const int nt = min(kTile, j1 - jt);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int c = tid + k * kTile;
      if (c < p.r) {
        float acc = o[k] * alpha;
        for (int jj = 0; jj < nt; ++jj) {
          const int sl = slot_s[jj];
          if (sl >= 0) acc = fmaf(w_s[jj], ld(lat + static_cast<int64_t>(sl) * p.lat_st + c), acc);
        }
        o[k] = acc;
      }
    }
    if (m_new != -INFINITY) m = m_new;
    __syncthreads();
  }

  const int64_t ps = (static_cast<int64_t>(b) * p.heads + h) * p.s_max + s;
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int c = tid + k * kTile;
    if (c < p.r) {
      if (p.part_bf16)
        static_cast<uint16_t*>(p.part_o)[ps * p.r + c] = f32_to_bf16(o[k] * inv_l);
      else
        static_cast<float*>(p.part_o)[ps * p.r + c] = o[k] * inv_l;
    }
  }
  if (tid == 0) p.part_lse[ps] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_decode_generic(int32_t dtype, const DecodeParams& p, hipStream_t stream) {
  if (p.rows == 0 || p.s_launch == 0) return hipSuccess;
  dim3 grid(p.s_launch, p.heads, p.rows);
  if (dtype == kBF16)
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, dim3(kTile), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(kTile), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
