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
// floor(e / 4) mod 4 as c_e 2^s(e), s(e) = floor(e / 4) mod 4.  bits_lo
// takes elements 0..15 straight from the word; bits_hi takes elements 16..31
// from the word shifted down by 4 (bits 4..7 of each byte move to bits 0..3
// of the same byte), so every byte is a code bit of weight 1, 2, 4 or 8.  The
// other operand of the product carries 2^(3 - s(e)) for element e (see
// bit_weight), so every product comes out as 2^3 c_e times its factor.
__device__ __forceinline__ v4i bits_lo(uint32_t w) {
  return v4i{(int)(w & 0x01010101u), (int)(w & 0x02020202u), (int)(w & 0x04040404u), (int)(w & 0x08080808u)};
}
__device__ __forceinline__ v4i bits_hi(uint32_t w) {
  const uint32_t x = w >> 4;
  return v4i{(int)(x & 0x01010101u), (int)(x & 0x02020202u), (int)(x & 0x04040404u), (int)(x & 0x08080808u)};
}
// log2 of the compensating factor of element e of a word: 3 - s(e)
__device__ __forceinline__ int bit_weight(int e) { return 3 - ((e >> 2) & 3); }

// Probability p in [0, 1] (up to rounding) as the fixed-point integer
// P = round(p 2^27): float32 keeps 24 significant bits of p, so P is p to
// 2^-24 relative, and to 2^-28 absolute below 2^-4.  A p slightly above 1
// from rounding gives P slightly above 2^27, which every user tolerates.
constexpr float kPOne = 134217728.f;          // 2^27
__device__ __forceinline__ uint32_t p_fixed(float p) { return (uint32_t)fmaf(p, kPOne, 0.5f); }
// The fixed point straight from the exponent: x27 = log2(p) + 27, so
// 2^x27 = p 2^27, truncated: P = floor(p 2^27), one instruction fewer than
// scaling p.  The numerator and the normalizer take the same P, and each P is
// below p 2^27 by less than one unit (2^-27 of the largest weight).  A weight
// of 0 (x27 = -inf) stays 0.
__device__ __forceinline__ uint32_t p_fixed_exp2(float x27) { return (uint32_t)__builtin_amdgcn_exp2f(x27); }

// Four signed base-256 digits of |x| < 2^30: the bytes of x + 0x808080 with
// the low three offset back by 128, so x = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3
// with every d_k a signed byte.
__device__ __forceinline__ uint32_t sdigits(uint32_t x) { return (x + 0x00808080u) ^ 0x00808080u; }

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

// ---- reductions across lanes in the VALU ------------------------------
// __shfl_xor compiles to ds_bpermute here: one round trip through the LDS unit
// per step, and a chain of them costs about a hundred cycles a step on a busy
// CU.  DPP row rotations and lane reads stay in the VALU.

// x rotated by R lanes within each row of 16 lanes (DPP row_ror)
template <int R>
__device__ __forceinline__ float ror16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + R, 0xF, 0xF,
                                                               false));
}
template <int R>
__device__ __forceinline__ double ror16(double x) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x120 + R, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x120 + R, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Over each row of 16 lanes, in every lane of the row.  Rotations by 8, 4, 2
// and 1 lanes: lane i adds the value of lane i + R (mod 16), which after the
// earlier steps equals that of lane i ^ R, so a sum is formed by the same
// additions, operand for operand, as an xor butterfly over 8, 4, 2, 1.
template <typename F>
__device__ __forceinline__ F row_sum16(F x) {
  x += ror16<8>(x);
  x += ror16<4>(x);
  x += ror16<2>(x);
  x += ror16<1>(x);
  return x;
}
// N row sums at once, the steps of the N sums interleaved so that each DPP
// read is not right behind the write it depends on (same additions as N
// separate row_sum16 calls)
template <int N>
__device__ __forceinline__ void row_sum16x(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += ror16<8>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += ror16<4>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += ror16<2>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += ror16<1>(x[i]);
}
__device__ __forceinline__ float row_min16(float x) {
  x = fminf(x, ror16<8>(x));
  x = fminf(x, ror16<4>(x));
  x = fminf(x, ror16<2>(x));
  return fminf(x, ror16<1>(x));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, ror16<8>(x));
  x = fmaxf(x, ror16<4>(x));
  x = fmaxf(x, ror16<2>(x));
  return fmaxf(x, ror16<1>(x));
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ double lane_d(double x, int l) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Over the 64 lanes of the wave (every lane receives it; all lanes active):
// each row of 16, then the four rows as ((r0 + r1) + (r2 + r3)).
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
__device__ __forceinline__ double wave_sum(double x) {
  x = row_sum16(x);
  return (lane_d(x, 0) + lane_d(x, 16)) + (lane_d(x, 32) + lane_d(x, 48));
}
__device__ __forceinline__ float wave_min(float x) {
  x = row_min16(x);
  return fminf(fminf(lane_f(x, 0), lane_f(x, 16)), fminf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

}  // namespace cqm
