// Device-side helpers shared by the libcq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace cqd {

constexpr int kD = 128;          // head dimension supported by this build

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __half from_f32<__half>(float v) { return __float2half_rn(v); }

// 16-byte load with the non-temporal hint, for data read once: the line is
// not kept in the caches, which measurably shortens the load latency of
// streaming workgroups.
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Bit offset of element e inside a packed 32-bit word (see cq.h).
__host__ __device__ __forceinline__ int code_off(int e, int bits) {
  return 8 * (e & 3) + bits * (e >> 2);
}

// Error-free sum: a + b == s + e exactly (round-to-nearest, no reassociation).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Exact sign of a + b + c for finite doubles (Shewchuk's grow-expansion: the
// result is a non-overlapping expansion whose most significant non-zero
// component carries the sign of the exact sum).
__device__ __forceinline__ int exact_sign3(double a, double b, double c) {
  double q, h0;
  two_sum(b, a, q, h0);            // a + b = q + h0
  double g0, g1, q2, q3;
  two_sum(c, h0, q2, g0);          // grow by c
  two_sum(q2, q, q3, g1);
  double top = q3 != 0.0 ? q3 : (g1 != 0.0 ? g1 : g0);
  return (top > 0.0) - (top < 0.0);
}

// The exact half-integer test of exact_code, kept out of line: inlined, the
// compiler evaluates it for every element and selects, although it is needed
// only near a half-integer.
__device__ __noinline__ int exact_tie_code(float x, float mn, float mx, int k, int L) {
  k = k < 0 ? 0 : (k > L - 1 ? L - 1 : k);
  const int s = exact_sign3(2.0 * L * (double)x, -(double)(2 * k + 1) * (double)mx,
                            (double)(2 * k + 1 - 2 * L) * (double)mn);
  return k + ((s > 0) || (s == 0 && (k & 1)));
}

// Round-half-to-even code of (x - mn) * L / (mx - mn), decided exactly.
// `t` is an estimate of that quotient whose absolute error is below `window`
// (by a safe margin); when it is farther than `window` from a half-integer
// the nearest integer is already certain, otherwise the half-integer
// threshold k + 1/2 is tested exactly via sign(2L*x - (2k+1)*mx +
// (2k+1-2L)*mn); each product is exact in float64 because x, mn, mx are
// float32-representable and the factors are < 2^10.
__device__ __forceinline__ int exact_code(float x, float mn, float mx, double t, int L,
                                          double window = 0.0078125) {
  const double fl = floor(t);
  int c;
  if (fabs((t - fl) - 0.5) > window) {
    c = (int)rint(t);
  } else {
    c = exact_tie_code(x, mn, mx, (int)fl, L);
  }
  return c < 0 ? 0 : (c > L ? L : c);
}

// Order-preserving map float -> int32 (for integer atomics on floats).
__device__ __forceinline__ int f2ord(float f) {
  int i = __float_as_int(f);
  return i >= 0 ? i : (i ^ 0x7FFFFFFF);
}
__device__ __forceinline__ float ord2f(int i) {
  return __int_as_float(i >= 0 ? i : (i ^ 0x7FFFFFFF));
}

}  // namespace cqd
