// gfx950 building blocks shared by the MFMA kernels: bf16 vector types, the
// 16x16x32 bf16 MFMA, the LDS transposing read, and the hand-driven HBM -> LDS
// copy instructions with their waits.
#pragma once

#pragma clang diagnostic ignored "-Winline-asm"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// D[16x16] += A[16x32] B[32x16]; lane l holds A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16]
// and D[4(l/16)..+4][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4 of
// the 8-byte chunks addressed by lanes i/4 + 4j (j = 0..3).  With lane q
// pointing at row r0 + q/4, columns c0 + 4(q%4) of a row-major bf16 tile, lane i
// receives rows r0..r0+3 of column c0 + i.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Convert 8 fp32 to bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(float4 u, float4 v) {
  bf16x8 q;
  q[0] = static_cast<__bf16>(u.x); q[1] = static_cast<__bf16>(u.y);
  q[2] = static_cast<__bf16>(u.z); q[3] = static_cast<__bf16>(u.w);
  q[4] = static_cast<__bf16>(v.x); q[5] = static_cast<__bf16>(v.y);
  q[6] = static_cast<__bf16>(v.z); q[7] = static_cast<__bf16>(v.w);
  return q;
}

// HBM -> LDS copies, waits and barrier are issued as instructions whose order
// the compiler keeps ("memory" clobbers) but does not track, so the number of
// copies in flight is exactly what the calling code states.  The copies set
// m0 (the LDS destination); the compiler reserves m0 and warns about the
// clobber, but allocates it for nothing in these kernels (a host test scans
// the compiled ISA for any other use of m0).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// The LDS destination must sit in an SGPR for m0.  The compiler may keep a
// wave-uniform value in a VGPR (it then prints a VGPR for an "s" operand, which
// does not assemble); readfirstlane moves it to an SGPR (no-op when it is one).
__device__ __forceinline__ uint32_t sgpr(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Each lane copies 16 bytes from `src` to lds + 16 * lane (lds is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(sgpr(lds)) : "memory", "m0");
}

// Same, from the wave-uniform base `sbase` plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_off(const void* sbase, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "s"(sgpr(lds))
               : "memory", "m0");
}

// Non-temporal forms, for bytes read once per pass (the decode attention's
// dense-row KV cache stream, ~170 MB per layer): with the hint the
// attention's launch ran 7 % faster (37.6 -> 34.9 us per ragged layer,
// kernel trace) and the kernels around it gained too.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(sgpr(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma16_off_nt(const void* sbase, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(sbase), "s"(sgpr(lds))
               : "memory", "m0");
}

// Each active lane copies 4 bytes from `src` to lds + 4 * lane.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(sgpr(lds)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
// Loads (register or LDS destination) complete in issue order, so this also
// waits for every load issued before the N most recent ones.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vm with a wave-uniform count; counts above MAX wait for MAX.
template <int MAX>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (MAX > 0) {
    if (n >= MAX) {
      wait_vm<MAX>();
      return;
    }
    wait_vm_upto<MAX - 1>(n);
  } else {
    wait_vm<0>();
  }
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace mla
