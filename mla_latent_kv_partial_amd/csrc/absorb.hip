// Weight absorption around latent attention (page "mlx-bun 0.0.11 -> 0.0.13",
// glm52-mla.ts, Glm52Mla.attendAbsorbed).  kv_b_proj holds, per head h,
// W_UK[h] = rows [h(dn+dv), h(dn+dv)+dn) and W_UV[h] = the next dv rows, each
// row kv_lora_rank wide.
//   absorb_q:  q_lat[b,h,:] = q_nope[b,h,:] . W_UK[h]        ([dn] x [dn,r])
//   absorb_v:  ctx[b,h*dv+v] = o_lat[b,h,:] . W_UV[h][v,:]    ([r] x [r,dv])
//
// These are the generic kernels (fp32 weights and geometries outside the
// MFMA kernels' limits); bf16 weights of the usual geometry go to the MFMA
// kernels.  Every weight element is read once per launch and used for all
// batch rows: absorb_q walks W_UK row by row (coalesced along r) with up to
// kRowsQ batch rows of accumulators per thread; absorb_v gives each wave one
// output feature and reduces along r.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kRowsQ = 8;

template <typename T>
__global__ __launch_bounds__(256) void absorb_q_kernel(AbsorbQParams p) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const int b0 = blockIdx.z * kRowsQ;
  if (c >= p.r) return;
  const int nb = min(kRowsQ, p.batch - b0);
  const T* w = static_cast<const T*>(p.w) + static_cast<int64_t>(h) * (p.dn + p.dv) * p.r + c;
  const T* q = static_cast<const T*>(p.q) + b0 * p.q_sb + h * p.q_sh;
  float acc[kRowsQ];
#pragma unroll
  for (int j = 0; j < kRowsQ; ++j) acc[j] = 0.f;
  for (int d = 0; d < p.dn; ++d) {
    const float wv = ld(w + static_cast<int64_t>(d) * p.r);
#pragma unroll
    for (int j = 0; j < kRowsQ; ++j)
      if (j < nb) acc[j] = fmaf(ld(q + j * p.q_sb + d), wv, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < kRowsQ; ++j)
    if (j < nb) st(static_cast<T*>(p.q_lat) + (static_cast<int64_t>(b0 + j) * p.heads + h) * p.r + c, acc[j]);
}

template <typename T>
__global__ __launch_bounds__(256) void absorb_v_kernel(AbsorbVParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;   // output feature h*dv+v
  if (n >= p.heads * p.dv) return;
  const int h = n / p.dv;
  const int v = n - h * p.dv;
  const T* w = static_cast<const T*>(p.w) + (static_cast<int64_t>(h) * (p.dn + p.dv) + p.dn + v) * p.r;
  for (int b = 0; b < p.batch; ++b) {
    const float* o = p.o_lat + (static_cast<int64_t>(b) * p.heads + h) * p.r;
    float acc = 0.f;
    for (int c = lane; c < p.r; c += kWave) acc = fmaf(o[c], ld(w + c), acc);
    acc = wave_reduce(acc, SumOp());
    if (lane == 0) p.ctx[static_cast<int64_t>(b) * p.heads * p.dv + n] = acc;
  }
}

}  // namespace

bool absorb_q_mfma_ok(const AbsorbQParams& p);
bool absorb_v_mfma_ok(const AbsorbVParams& p);
hipError_t launch_absorb_q_mfma(const AbsorbQParams& p, hipStream_t stream);
hipError_t launch_absorb_q_rope_mfma(const AbsorbQParams& p, const RopeParams& rp, hipStream_t stream);
hipError_t launch_absorb_v_mfma(const AbsorbVParams& p, hipStream_t stream);

hipError_t launch_absorb_q(int32_t dtype, const AbsorbQParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (dtype == kBF16 && absorb_q_mfma_ok(p)) return launch_absorb_q_mfma(p, stream);
  dim3 grid((p.r + 255) / 256, p.heads, (p.batch + kRowsQ - 1) / kRowsQ);
  if (dtype == kBF16)
    hipLaunchKernelGGL(absorb_q_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(absorb_q_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_absorb_q_rope(int32_t dtype, const AbsorbQParams& p, const RopeParams& rp, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (dtype == kBF16 && absorb_q_mfma_ok(p)) return launch_absorb_q_rope_mfma(p, rp, stream);
  const hipError_t e = launch_rope(dtype, rp, stream);
  return e != hipSuccess ? e : launch_absorb_q(dtype, p, stream);
}

hipError_t launch_absorb_v(int32_t dtype, const AbsorbVParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (dtype == kBF16 && absorb_v_mfma_ok(p)) return launch_absorb_v_mfma(p, stream);
  const int outs = p.heads * p.dv;
  dim3 grid((outs + 3) / 4);
  if (dtype == kBF16)
    hipLaunchKernelGGL(absorb_v_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(absorb_v_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
