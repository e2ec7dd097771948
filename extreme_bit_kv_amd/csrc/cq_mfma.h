// Device helpers of the matrix-core decode kernels (gfx950, wave64): the
// int8 16x16x64 product, spreading packed code words into byte operands,
// and the hand-off of probability digits through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace cqm {

typedef int v4i __attribute__((ext_vector_type(4)));

// element i of a float32 or float16 array
__device__ __forceinline__ float ld_any(const void* p, size_t i, int is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[i] : __half2float(reinterpret_cast<const __half*>(p)[i]);
}

// 1-bit words: elements 0..15 / 16..31 of a packed word as 16 bytes (0 or 1)
// in element order, thanks to the interleaved layout (element e at bit
// 8 (e mod 4) + floor(e / 4)).
__device__ __forceinline__ v4i spread_lo(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x01010101u);
  r[1] = (int)((w >> 1) & 0x01010101u);
  r[2] = (int)((w >> 2) & 0x01010101u);
  r[3] = (int)((w >> 3) & 0x01010101u);
  return r;
}
__device__ __forceinline__ v4i spread_hi(uint32_t w) {
  v4i r;
  r[0] = (int)((w >> 4) & 0x01010101u);
  r[1] = (int)((w >> 5) & 0x01010101u);
  r[2] = (int)((w >> 6) & 0x01010101u);
  r[3] = (int)((w >> 7) & 0x01010101u);
  return r;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// byte `pl` of four registers, packed into one dword
__device__ __forceinline__ uint32_t gather_byte(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3, int pl) {
  const uint32_t lo = __builtin_amdgcn_perm(f1, f0, (uint32_t)pl | ((uint32_t)(pl + 4) << 8) | 0x0C0C0000u);
  const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x00000C0Cu | ((uint32_t)pl << 16) | ((uint32_t)(pl + 4) << 24));
  return lo | hi;
}

// LDS written by some lanes of a wave, then read by others of the same wave
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every global load the wave has in flight (its fence covers all memory), so a
// barrier placed after a prefetch would wait for the prefetch; this one
// waits only for the wave's own LDS accesses.  Use it only where the threads
// exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace cqm
