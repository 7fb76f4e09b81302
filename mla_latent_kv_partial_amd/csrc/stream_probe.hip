// Streaming probe of the latent decode attention (measurement, no arithmetic).
// It reads exactly the cache bytes mla_decode_latent_attn reads for dense rows
// of a packed bf16 [B, W, 576] cache, with the same launch geometry and the
// same copy schedule: one workgroup of 512 threads per (row, split) in the
// same compact order; 32-token tiles of 1184-byte LDS rows copied by
// non-temporal global_load_lds_dwordx4 (37 copies of 1 KB per tile, the same lane plan)
// into a 4-stage ring of the same size, two tiles ahead, with the same waits
// and barriers.  It computes nothing and writes no partials, so its time is
// the floor of the attention's copy path at that shape; the attention's time
// over it is what the arithmetic, the queries and the partial writes add.
#include "cdna4.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kPNT = 32;                                     // tokens per tile
constexpr int kPRowChunks = 74;                              // 16-byte chunks per LDS token row
constexpr int kPDmaPerTile = (kPNT * kPRowChunks + 63) / 64;  // 37
constexpr int kPStageBytes = kPDmaPerTile * 1024 + kPNT * 4;  // as the attention's stages
constexpr int kPStages = 4;
constexpr int kPWaves = 8;
constexpr int kPMaxDma = (kPDmaPerTile + kPWaves - 1) / kPWaves;   // 5

__shared__ __attribute__((aligned(1024))) char g_probe[kPStages * kPStageBytes];

__global__ __launch_bounds__(kPWaves * kWave) void stream_probe_kernel(DecodeParams p) {
  const int wg = blockIdx.x;
  int b = 0, hi = p.rows;
  while (hi - b > 1) {
    const int mid = (b + hi) >> 1;
    if (p.tab.split_begin[mid] <= wg) b = mid; else hi = mid;
  }
  const int s = wg - p.tab.split_begin[b];
  const int j0 = s * p.chunk;
  const int n_tok = min(p.chunk, p.tab.n_att[b] - j0);
  const int nt = (n_tok + kPNT - 1) / kPNT;
  const int pad = p.width - p.tab.kv_len[b];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* lat_base = static_cast<const char*>(p.latent) + static_cast<int64_t>(b) * p.lat_sb * 2;
  const uint32_t lat_st = static_cast<uint32_t>(p.lat_st * 2);

  // copy i of this wave moves stage chunk k = 64 (wave + 8 i) + lane: chunk c
  // of token row k / 74 (latent and rope are contiguous in the packed row)
  const int n_dma = (kPDmaPerTile - wave + kPWaves - 1) / kPWaves;
  int c_row[kPMaxDma];
  uint32_t c_off[kPMaxDma];
#pragma unroll
  for (int i = 0; i < kPMaxDma; ++i) {
    const int k = 64 * (wave + kPWaves * i) + lane;
    const int row = k / kPRowChunks;
    const int c = k - row * kPRowChunks;
    c_row[i] = min(row, kPNT - 1);
    c_off[i] = c < 72 ? static_cast<uint32_t>(c) * 16u : 0u;
  }
  auto issue = [&](int st, int tile) {
    const uint32_t dst = lds_addr(g_probe + st * kPStageBytes);
    const int first = tile * kPNT;
#pragma unroll
    for (int i = 0; i < kPMaxDma; ++i) {
      if (i == kPMaxDma - 1 && n_dma != kPMaxDma) break;
      const int slot = first + c_row[i] < n_tok ? pad + j0 + first + c_row[i] : p.width - 1;
      dma16_off_nt(lat_base, static_cast<uint32_t>(slot) * lat_st + c_off[i], dst + (wave + kPWaves * i) * 1024);
    }
  };
  issue(0, 0);
  issue(1, 1);   // also for single-tile splits, as the attention does
  for (int i = 0; i < nt; ++i) {
    wait_vm_upto<kPMaxDma>(i == 0 || i + 1 < nt ? n_dma : 0);
    lds_barrier();
    if (i + 2 < nt) issue((i + 2) % kPStages, i + 2);
  }
  wait_vm<0>();
}

}  // namespace

hipError_t launch_stream_probe(const DecodeParams& p, hipStream_t stream) {
  if (p.rows == 0 || p.s_total == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(p.s_total), dim3(kPWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
