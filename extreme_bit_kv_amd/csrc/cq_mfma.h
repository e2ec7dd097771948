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

// 1-bit words masked in place, one AND per register: element e (at bit
// 8 (e mod 4) + floor(e / 4)) is left in byte e mod 4 of register
// floor(e / 4) mod 4 as c_e 2^s(e), s(e) = min(floor(e / 4), 6).  The top bit
// of each byte is moved down one place so that every byte is a non-negative
// int8.  The other operand of the product carries 2^(7 - s(e)) for element e
// (see bit_weight), so every product comes out as 2^7 c_e times its factor.
__device__ __forceinline__ v4i bits_lo(uint32_t w) {
  return v4i{(int)(w & 0x01010101u), (int)(w & 0x02020202u), (int)(w & 0x04040404u), (int)(w & 0x08080808u)};
}
__device__ __forceinline__ v4i bits_hi(uint32_t w) {
  return v4i{(int)(w & 0x10101010u), (int)(w & 0x20202020u), (int)(w & 0x40404040u),
             (int)((w >> 1) & 0x40404040u)};
}
// log2 of the compensating factor of element e of a word: 7 - s(e)
__device__ __forceinline__ int bit_weight(int e) { return 7 - min((e >> 2) & 7, 6); }

// 4 x 4 byte transpose: o_p holds byte p of f0, f1, f2, f3 (in that order)
__device__ __forceinline__ void transpose_bytes(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3,
                                                uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  const uint32_t t0 = __builtin_amdgcn_perm(f1, f0, 0x05010400u);   // f0.0 f1.0 f0.1 f1.1
  const uint32_t t1 = __builtin_amdgcn_perm(f1, f0, 0x07030602u);   // f0.2 f1.2 f0.3 f1.3
  const uint32_t t2 = __builtin_amdgcn_perm(f3, f2, 0x05010400u);   // f2.0 f3.0 f2.1 f3.1
  const uint32_t t3 = __builtin_amdgcn_perm(f3, f2, 0x07030602u);   // f2.2 f3.2 f2.3 f3.3
  o0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
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
