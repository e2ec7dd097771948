// Quantization of a visual segment that is written chunk by chunk (chunked
// prefill, frames appended to a video), in two steps that need no
// rendezvous between workgroups:
//
//   * range update: the per-channel minimum and maximum of a block of rows,
//     merged into a running range with float atomics; a per-(batch, head)
//     flag says whether the range became wider;
//   * row quantization: the codes of a block of rows on a GIVEN range, into a
//     code buffer laid out for the whole segment.
//
// QbitAI article on CalibQuant, "Method" part 1: the quantizer's range is
// the per-channel min and max over the tokens of one head.  Min and max are
// associative, so the range gathered over the chunks of a segment is the
// segment's range, and rows coded on it are the one-shot codes.  Values
// outside a given range take the nearest level (code 0 or L).
//
// The 1-bit float16 row kernel keeps the fused quantizer's register tile and
// code stage (cq_tile1.h): one 512-token tile per workgroup, loaded once,
// thresholds from the given range, sign bits of t - x, coalesced stores.
// Other bit widths and float32 rows use the generic pack kernels.
#include "cq_device.h"
#include "cq_internal.h"
#include "cq_tile1.h"

namespace {

using namespace cqt;

constexpr int kUpdRows = 256;          // rows of one range-update workgroup
constexpr int kUpdThreads = 256;

// Float atomics on the range arrays.  Zero is canonical (+0) before it is
// merged.  For a non-negative value the int order of the bit patterns is the
// float order (and every negative pattern is below it); for a negative value
// the unsigned order is the reverse of the float order (and every
// non-negative pattern is below it).  The returned flag compares the value
// with what was stored before, as floats, so -0 against +0 widens nothing.
__device__ __forceinline__ bool atomic_min_f32(float* p, float v) {
  v = v + 0.0f;
  float old;
  if (!__builtin_signbit(v))
    old = __int_as_float(atomicMin(reinterpret_cast<int*>(p), __float_as_int(v)));
  else
    old = __uint_as_float(atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v)));
  return v < old;
}
__device__ __forceinline__ bool atomic_max_f32(float* p, float v) {
  v = v + 0.0f;
  float old;
  if (!__builtin_signbit(v))
    old = __int_as_float(atomicMax(reinterpret_cast<int*>(p), __float_as_int(v)));
  else
    old = __uint_as_float(atomicMin(reinterpret_cast<unsigned int*>(p), __float_as_uint(v)));
  return v > old;
}

// reset: range <- (+inf, -inf); grew <- 0 (when given)
__global__ void rg_init(float* __restrict__ mn, float* __restrict__ mx, uint32_t* __restrict__ grew, long count,
                        int units, int reset) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (reset && i < count) {
    mn[i] = INFINITY;
    mx[i] = -INFINITY;
  }
  if (grew != nullptr && i < units) grew[i] = 0u;
}

// Workgroup (row block, unit): channel min/max of rows [t0 + 256 bx, ..) of
// x[unit] (unit stride x_rows rows), merged into mn/mx[unit].  A thread
// reads 16 bytes of a row (8 float16 or 4 float32 channels).
template <typename T>
__global__ void __launch_bounds__(kUpdThreads) rg_update(const T* __restrict__ x, long x_rows, int t0, int m,
                                                          float* __restrict__ mn, float* __restrict__ mx,
                                                          uint32_t* __restrict__ grew) {
  constexpr int kVec = 16 / (int)sizeof(T), kTpr = cqd::kD / kVec, kStep = kUpdThreads / kTpr;
  const int unit = blockIdx.y;
  const int r0 = blockIdx.x * kUpdRows, r1 = min(m, r0 + kUpdRows);
  const T* xu = x + ((size_t)unit * x_rows + t0) * cqd::kD;
  const int cg = threadIdx.x % kTpr, rr = threadIdx.x / kTpr;
  __shared__ float slo[kStep][cqd::kD], shi[kStep][cqd::kD];
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  float lo[kVec], hi[kVec];
  if constexpr (sizeof(T) == 2) {
    // packed float16 min/max, four channel pairs per thread
    uint32_t a[4], b[4];
    const uint4 first = *reinterpret_cast<const uint4*>(xu + (size_t)min(r0 + rr, r1 - 1) * cqd::kD + cg * kVec);
    a[0] = b[0] = first.x; a[1] = b[1] = first.y; a[2] = b[2] = first.z; a[3] = b[3] = first.w;
#pragma unroll 8
    for (int i = r0 + rr + kStep; i < r1; i += kStep) {
      const uint4 v = *reinterpret_cast<const uint4*>(xu + (size_t)i * cqd::kD + cg * kVec);
      a[0] = hmin2u(a[0], v.x); b[0] = hmax2u(b[0], v.x);
      a[1] = hmin2u(a[1], v.y); b[1] = hmax2u(b[1], v.y);
      a[2] = hmin2u(a[2], v.z); b[2] = hmax2u(b[2], v.z);
      a[3] = hmin2u(a[3], v.w); b[3] = hmax2u(b[3], v.w);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[2 * q] = lo_f(a[q]); lo[2 * q + 1] = hi_f(a[q]);
      hi[2 * q] = lo_f(b[q]); hi[2 * q + 1] = hi_f(b[q]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kVec; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
#pragma unroll 8
    for (int i = r0 + rr; i < r1; i += kStep) {
      const float4 v = *reinterpret_cast<const float4*>(xu + (size_t)i * cqd::kD + cg * kVec);
      lo[0] = fminf(lo[0], v.x); hi[0] = fmaxf(hi[0], v.x);
      lo[1] = fminf(lo[1], v.y); hi[1] = fmaxf(hi[1], v.y);
      lo[2] = fminf(lo[2], v.z); hi[2] = fmaxf(hi[2], v.z);
      lo[3] = fminf(lo[3], v.w); hi[3] = fmaxf(hi[3], v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    slo[rr][cg * kVec + e] = lo[e];
    shi[rr][cg * kVec + e] = hi[e];
  }
  __syncthreads();
  if (threadIdx.x < cqd::kD) {
    const int c = threadIdx.x;
    float l = slo[0][c], h = shi[0][c];
#pragma unroll
    for (int r = 1; r < kStep; ++r) {
      l = fminf(l, slo[r][c]);
      h = fmaxf(h, shi[r][c]);
    }
    const size_t o = (size_t)unit * cqd::kD + c;
    const bool wider = atomic_min_f32(mn + o, l) | atomic_max_f32(mx + o, h);
    if (wider) any = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && any && grew != nullptr) atomicOr(grew + unit, 1u);
}

// float32 nearest to the exact (mx - mn)/L, ties to even (b = 1: L = 1).
__device__ float scale_rn1(float mn, float mx) {
  double rh, rl;
  cqd::two_sum((double)mx, -(double)mn, rh, rl);
  float f = (float)rh;                                  // rh = RN64(mx - mn): one more rounding
  // correct the double rounding: f is within one ulp of the exact difference
  for (int it = 0; it < 2; ++it) {
    const float up = nextafterf(f, INFINITY), dn = nextafterf(f, -INFINITY);
    const int su = cqd::exact_sign3(0.5 * ((double)f + (double)up), -rh, -rl);   // mid_up - exact
    const int sd = cqd::exact_sign3(0.5 * ((double)f + (double)dn), -rh, -rl);
    const bool even = (__float_as_uint(f) & 1u) == 0;
    if (su < 0 || (su == 0 && !even)) { f = up; continue; }
    if (sd > 0 || (sd == 0 && !even)) { f = dn; continue; }
    break;
  }
  return f;
}

// Workgroup = one 512-token tile of one unit: codes of rows [t0, t0 + m) of
// x[unit] on the range mn/mx[unit], into the unit's code words laid out for
// n_codes tokens.  Tile 0 also writes the unit's scale and minimum.
template <int LAYOUT>
__global__ void __launch_bounds__(kWaves * 64) qr_b1(const __half* __restrict__ x, long x_rows, int t0, int m,
                                                     int tiles, const float* __restrict__ mn,
                                                     const float* __restrict__ mx,
                                                     const uint32_t* __restrict__ unit_mask, int n_codes,
                                                     uint32_t* __restrict__ codes, float* __restrict__ scale,
                                                     float* __restrict__ minv) {
  const int u = blockIdx.x / tiles, s = blockIdx.x % tiles;
  if (unit_mask != nullptr && unit_mask[u] == 0u) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = 4 * wave + (lane >> 4), k = lane & 15;
  const int base = t0 + s * kTile, last = t0 + m - 1;
  const __half* xu = x + (size_t)u * x_rows * 128;
  uint4 v[kRows];
#pragma unroll
  for (int it = 0; it < kRows; ++it) {
    const int tok = min(base + kRows * pair + it, last);
    v[it] = cqd::ld_nt(xu + (size_t)tok * 128 + 8 * k);   // the rows' last read
  }
  __shared__ uint32_t thr[64];                 // per channel pair: float16 thresholds
  if (tid < 128) {
    const float lo = mn[(size_t)u * 128 + tid], hi = mx[(size_t)u * 128 + tid];
    reinterpret_cast<unsigned short*>(thr)[tid] = mid_threshold(lo, hi);
    if (s == 0) {
      scale[(size_t)u * 128 + tid] = hi > lo ? scale_rn1(lo, hi) : 0.0f;
      minv[(size_t)u * 128 + tid] = lo;
    }
  }
  __syncthreads();
  const uint32_t q0 = thr[4 * k + 0], q1 = thr[4 * k + 1], q2 = thr[4 * k + 2], q3 = thr[4 * k + 3];
  uint32_t* cu = codes + (size_t)u * (LAYOUT == CQ_LAYOUT_K ? 4 * (size_t)n_codes
                                                            : 128 * (size_t)((n_codes + 31) >> 5));
  store_tile_codes<LAYOUT>(v, q0, q1, q2, q3, cu, base, t0 + m, n_codes, pair, k);
}

}  // namespace

namespace cqi {

hipError_t range_update(const RowsArgs& a, float* mn, float* mx, int reset, uint32_t* grew) {
  const int units = a.B * a.H;
  if (units == 0) return hipSuccess;
  if (reset || grew != nullptr) {
    const long count = (long)units * a.d;
    const long cover = reset ? count : units;
    CQ_LAUNCH(rg_init, dim3((unsigned)((cover + 255) / 256)), dim3(256), 0, a.stream, mn, mx, grew, count, units,
              reset);
  }
  if (a.m == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.m + kUpdRows - 1) / kUpdRows), (unsigned)units);
  if (a.dtype == CQ_F16)
    CQ_LAUNCH(rg_update<__half>, grid, dim3(kUpdThreads), 0, a.stream, (const __half*)a.x, a.x_rows, a.t0, a.m,
              mn, mx, grew);
  else
    CQ_LAUNCH(rg_update<float>, grid, dim3(kUpdThreads), 0, a.stream, (const float*)a.x, a.x_rows, a.t0, a.m, mn,
              mx, grew);
  return hipSuccess;
}

hipError_t quant_rows(const RowsArgs& a, int bits, int layout, const float* mn, const float* mx,
                      const uint32_t* unit_mask, int n_codes, uint32_t* codes, float* scale, float* minv) {
  const int units = a.B * a.H;
  if (units == 0 || a.m == 0) return hipSuccess;
  if (a.dtype == CQ_F16 && bits == 1) {
    const int tiles = (a.m + kTile - 1) / kTile;
    const long grid = (long)units * tiles;
    if (grid > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
    if (layout == CQ_LAYOUT_K)
      CQ_LAUNCH(qr_b1<CQ_LAYOUT_K>, dim3((unsigned)grid), dim3(kWaves * 64), 0, a.stream, (const __half*)a.x,
                a.x_rows, a.t0, a.m, tiles, mn, mx, unit_mask, n_codes, codes, scale, minv);
    else
      CQ_LAUNCH(qr_b1<CQ_LAYOUT_V>, dim3((unsigned)grid), dim3(kWaves * 64), 0, a.stream, (const __half*)a.x,
                a.x_rows, a.t0, a.m, tiles, mn, mx, unit_mask, n_codes, codes, scale, minv);
    return hipSuccess;
  }
  return quant_rows_generic(a, bits, layout, mn, mx, unit_mask, n_codes, codes, scale, minv);
}

}  // namespace cqi
