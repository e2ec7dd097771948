// Channel-wise b-bit quantization, general path: any bits in {1,2,4,8},
// float16 or float32 input, either packed layout.
//
// QbitAI article on CalibQuant, "Method" part 1: the range used by the
// uniform integer quantizer is refined per channel over the n tokens of one
// head, and every row is quantized element-wise with it; V is handled alike.
//
// Three launches: (1) per-(unit, token chunk) channel min/max, (2) per-unit
// reduction of the chunks into min, max, the stored float32 scale and the
// quotient estimate used for rounding, (3) code decision and packing.  The
// input is read twice; the fused single-read kernel (quantize_fused.hip)
// replaces this path for 1-bit float16 inputs.  Head dimension 128.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kChunk = 512;      // tokens per stats block
constexpr int kThreads = 256;
constexpr int kD = 128;          // head dimension (the only one the library takes)

struct QParams {                 // per (unit, channel), in the workspace
  float mn, mx;
  double inv;                    // L / (mx - mn), 0 for a constant channel
};

// Values of 16 bytes of row data (8 float16 or 4 float32).
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& raw, float* v) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __half2float(__ushort_as_half((unsigned short)(w[k] & 0xFFFFu)));
      v[2 * k + 1] = __half2float(__ushort_as_half((unsigned short)(w[k] >> 16)));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(w[k]);
  }
}

// N consecutive values from p (16-byte vector loads; 8-byte ones for four float16).
template <typename T, int N>
__device__ __forceinline__ void load_vals(const T* p, float (&v)[N]) {
  constexpr int kPer = 16 / (int)sizeof(T);
  if constexpr (N >= kPer) {
#pragma unroll
    for (int k = 0; k < N / kPer; ++k) unpack16<T>(reinterpret_cast<const uint4*>(p)[k], v + k * kPer);
  } else {
    static_assert(sizeof(T) == 2 && N == 4, "four float16 values");
    const uint2 raw = *reinterpret_cast<const uint2*>(p);
    v[0] = __half2float(__ushort_as_half((unsigned short)(raw.x & 0xFFFFu)));
    v[1] = __half2float(__ushort_as_half((unsigned short)(raw.x >> 16)));
    v[2] = __half2float(__ushort_as_half((unsigned short)(raw.y & 0xFFFFu)));
    v[3] = __half2float(__ushort_as_half((unsigned short)(raw.y >> 16)));
  }
}

// Per-(unit, chunk) channel min/max: a thread reads 16 bytes of a row
// (channels kVec cg .. +kVec-1), kRows rows of the chunk at a time.
template <typename T>
__global__ void __launch_bounds__(kThreads) qz_stats(const T* __restrict__ x, int n, int chunks,
                                                     float2* __restrict__ part, int* status) {
  if (status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;
  constexpr int kVec = 16 / (int)sizeof(T), kTpr = kD / kVec, kRows = kThreads / kTpr;
  const int unit = blockIdx.y, chunk = blockIdx.x;
  const T* xu = x + (size_t)unit * n * kD;
  const int cg = threadIdx.x % kTpr, r0 = threadIdx.x / kTpr;
  const int i0 = chunk * kChunk, i1 = min(n, i0 + kChunk);
  float lo[kVec], hi[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
#pragma unroll 4
  for (int i = i0 + r0; i < i1; i += kRows) {
    float v[kVec];
    load_vals<T, kVec>(xu + (size_t)i * kD + cg * kVec, v);
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      lo[e] = fminf(lo[e], v[e]);
      hi[e] = fmaxf(hi[e], v[e]);
    }
  }
  __shared__ float slo[kRows][kD], shi[kRows][kD];
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    slo[r0][cg * kVec + e] = lo[e];
    shi[r0][cg * kVec + e] = hi[e];
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    float l = INFINITY, h = -INFINITY;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      l = fminf(l, slo[r][c]);
      h = fmaxf(h, shi[r][c]);
    }
    part[((size_t)unit * chunks + chunk) * kD + c] = make_float2(l, h);
  }
}

// float32 nearest to the exact quotient (mx - mn)/L, ties to even.
__device__ float scale_rn(float mn, float mx, int L) {
  double rh, rl;
  cqd::two_sum((double)mx, -(double)mn, rh, rl);          // mx - mn == rh + rl exactly
  float f = (float)((rh + rl) / (double)L);
  for (int it = 0; it < 2; ++it) {                         // candidate is within one ulp
    float up = nextafterf(f, INFINITY), dn = nextafterf(f, -INFINITY);
    double mid_up = 0.5 * ((double)f + (double)up);        // exact in float64
    double mid_dn = 0.5 * ((double)f + (double)dn);
    int su = cqd::exact_sign3(mid_up * L, -rh, -rl);       // sign(mid_up*L - r)
    int sd = cqd::exact_sign3(mid_dn * L, -rh, -rl);
    bool f_even = (__float_as_uint(f) & 1u) == 0;
    if (su < 0 || (su == 0 && !f_even)) { f = up; continue; }
    if (sd > 0 || (sd == 0 && !f_even)) { f = dn; continue; }
    break;
  }
  return f;
}

__global__ void qz_params(const float2* __restrict__ part, int chunks, int d, int bits,
                          float* __restrict__ scale, float* __restrict__ minv,
                          QParams* __restrict__ prm) {
  const int unit = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  float lo = INFINITY, hi = -INFINITY;
  for (int k = 0; k < chunks; ++k) {
    float2 v = part[((size_t)unit * chunks + k) * d + c];
    lo = fminf(lo, v.x);
    hi = fmaxf(hi, v.y);
  }
  const int L = (1 << bits) - 1;
  QParams p;
  p.mn = lo;
  p.mx = hi;
  if (hi > lo) {
    double rh, rl;
    cqd::two_sum((double)hi, -(double)lo, rh, rl);
    p.inv = (double)L / (rh + rl);
    scale[(size_t)unit * d + c] = scale_rn(lo, hi, L);
  } else {
    p.inv = 0.0;
    scale[(size_t)unit * d + c] = 0.0f;
  }
  minv[(size_t)unit * d + c] = lo;
  prm[(size_t)unit * d + c] = p;
}

// The float64 estimate t of (x - mn) L / (mx - mn) is off the exact quotient
// by at most 3 * 2^-53 * L < 2^-43 (x - mn is exact in float64 for
// float32-representable operands; inv and the product are one rounding each),
// so the exact test is needed only within 2^-30 of a half-integer: in
// practice for exact ties alone, and whole wavefronts seldom take it.
__device__ __forceinline__ int code_of(float x, const QParams& p, int L) {
  if (!(p.inv > 0.0)) return 0;
  const double t = ((double)x - (double)p.mn) * p.inv;
  if (t <= -1.0) return 0;                      // far outside a given range: an end level
  if (t >= L + 1.0) return L;
  return cqd::exact_code(x, p.mn, p.mx, t, L, 0x1p-30);
}

// Rows coded by one pack launch: tokens [t_first, n_end) of every unit; x has
// x_rows rows per unit, the code words are laid out for n_codes tokens.
struct Rows {
  long x_rows;
  int t_first, n_end, n_codes;
};

// The unit's channel parameters into LDS: from the workspace (one-shot path)
// or from a given range (row path; tile 0 then stores scale and minimum).
__device__ __forceinline__ void load_params(QParams* sp, const QParams* __restrict__ prm, const float* __restrict__ mn,
                                            const float* __restrict__ mx, int unit, int L, float* __restrict__ scale,
                                            float* __restrict__ minv) {
  if (threadIdx.x >= kD) return;
  const size_t o = (size_t)unit * kD + threadIdx.x;
  if (prm != nullptr) {
    sp[threadIdx.x] = prm[o];
    return;
  }
  QParams p;
  p.mn = mn[o];
  p.mx = mx[o];
  p.inv = 0.0;
  float sc = 0.0f;
  if (p.mx > p.mn) {
    double rh, rl;
    cqd::two_sum((double)p.mx, -(double)p.mn, rh, rl);
    p.inv = (double)L / (rh + rl);
    sc = scale_rn(p.mn, p.mx, L);
  }
  sp[threadIdx.x] = p;
  if (blockIdx.x == 0) {
    scale[o] = sc;
    minv[o] = p.mn;
  }
}

// K layout: a block packs kTok tokens.  Words are computed with the word
// index fastest across threads (a wave reads whole rows), staged in LDS, and
// written plane by plane (kTok consecutive words of a plane per wave).
constexpr int kTok = 64;
template <typename T, int BITS>
__global__ void __launch_bounds__(kThreads) qz_pack_k(const T* __restrict__ x, Rows g,
                                                      const QParams* __restrict__ prm, const float* __restrict__ mn,
                                                      const float* __restrict__ mx,
                                                      const uint32_t* __restrict__ unit_mask,
                                                      uint32_t* __restrict__ codes, float* __restrict__ scale,
                                                      float* __restrict__ minv) {
  constexpr int E = 32 / BITS, W = kD / E, L = (1 << BITS) - 1;
  const int unit = blockIdx.y, i0 = g.t_first + blockIdx.x * kTok;
  if (unit_mask != nullptr && unit_mask[unit] == 0u) return;
  const int n = g.n_end;
  __shared__ QParams sp[kD];                     // the unit's channel parameters
  __shared__ uint32_t sw[W][kTok + 1];
  load_params(sp, prm, mn, mx, unit, L, scale, minv);
  __syncthreads();
  for (int q = threadIdx.x; q < kTok * W; q += kThreads) {
    const int w = q % W, ti = q / W, i = i0 + ti;
    uint32_t word = 0;
    if (i < n) {
      float v[E];
      load_vals<T, E>(x + ((size_t)unit * g.x_rows + i) * kD + w * E, v);
#pragma unroll
      for (int e = 0; e < E; ++e) word |= (uint32_t)code_of(v[e], sp[w * E + e], L) << cqd::code_off(e, BITS);
    }
    sw[w][ti] = word;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTok * W; q += kThreads) {
    const int w = q / kTok, ti = q % kTok, i = i0 + ti;
    if (i < n) codes[((size_t)unit * W + w) * g.n_codes + i] = sw[w][ti];
  }
}

// V layout: thread (r, cg) packs the words (r, 8 cg .. 8 cg + 7): per token of
// the row it reads 16 bytes (8 channels) and stores two 16-byte word groups.
template <typename T, int BITS>
__global__ void __launch_bounds__(kThreads) qz_pack_v(const T* __restrict__ x, Rows g,
                                                      const QParams* __restrict__ prm, const float* __restrict__ mn,
                                                      const float* __restrict__ mx,
                                                      const uint32_t* __restrict__ unit_mask,
                                                      uint32_t* __restrict__ codes, float* __restrict__ scale,
                                                      float* __restrict__ minv) {
  constexpr int E = 32 / BITS, L = (1 << BITS) - 1;
  const int unit = blockIdx.y;
  if (unit_mask != nullptr && unit_mask[unit] == 0u) return;
  const int n = g.n_end;
  const int r_first = g.t_first / E, R_end = (n + E - 1) / E, R = (g.n_codes + E - 1) / E;
  __shared__ QParams sp[kD];
  load_params(sp, prm, mn, mx, unit, L, scale, minv);
  __syncthreads();
  const long idx = (long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long)(R_end - r_first) * (kD / 8)) return;
  const int r = r_first + (int)(idx / (kD / 8)), cg = (int)(idx % (kD / 8));
  const T* xu = x + (size_t)unit * g.x_rows * kD + 8 * cg;
  uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int e = 0; e < E; ++e) {
    const int i = r * E + e;
    if (i < n) {
      float v[8];
      load_vals<T, 8>(xu + (size_t)i * kD, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) word[c] |= (uint32_t)code_of(v[c], sp[8 * cg + c], L) << cqd::code_off(e, BITS);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + ((size_t)unit * R + r) * kD + 8 * cg);
  dst[0] = make_uint4(word[0], word[1], word[2], word[3]);
  dst[1] = make_uint4(word[4], word[5], word[6], word[7]);
}

// Empty cache: scale = minv = 0.
__global__ void qz_zero(float* scale, float* minv, long count, int* status) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (status != nullptr && i == 0) *status = 0;
  if (i < count) {
    scale[i] = 0.0f;
    minv[i] = 0.0f;
  }
}

template <typename T, int BITS>
hipError_t pack(int layout, const T* x, Rows g, const QParams* prm, const float* mn, const float* mx,
                const uint32_t* unit_mask, uint32_t* codes, float* scale, float* minv, int units, hipStream_t st) {
  constexpr int E = 32 / BITS;
  const int m = g.n_end - g.t_first;
  if (layout == CQ_LAYOUT_K) {
    CQ_LAUNCH((qz_pack_k<T, BITS>), dim3((unsigned)((m + kTok - 1) / kTok), units), dim3(kThreads), 0, st, x, g, prm,
              mn, mx, unit_mask, codes, scale, minv);
  } else {
    const long threads = (long)((g.n_end + E - 1) / E - g.t_first / E) * (kD / 8);
    CQ_LAUNCH((qz_pack_v<T, BITS>), dim3((unsigned)((threads + kThreads - 1) / kThreads), units), dim3(kThreads),
              0, st, x, g, prm, mn, mx, unit_mask, codes, scale, minv);
  }
  return hipSuccess;
}

template <typename T>
hipError_t pack_bits(int bits, int layout, const T* x, Rows g, const QParams* prm, const float* mn, const float* mx,
                     const uint32_t* unit_mask, uint32_t* codes, float* scale, float* minv, int units,
                     hipStream_t st) {
  switch (bits) {
    case 1: return pack<T, 1>(layout, x, g, prm, mn, mx, unit_mask, codes, scale, minv, units, st);
    case 2: return pack<T, 2>(layout, x, g, prm, mn, mx, unit_mask, codes, scale, minv, units, st);
    case 4: return pack<T, 4>(layout, x, g, prm, mn, mx, unit_mask, codes, scale, minv, units, st);
    default: return pack<T, 8>(layout, x, g, prm, mn, mx, unit_mask, codes, scale, minv, units, st);
  }
}

template <typename T>
hipError_t run(const cqi::QuantArgs& a) {
  const int units = a.B * a.H;
  if (units == 0) return hipSuccess;
  if (a.n == 0) {
    long cnt = (long)units * a.d;
    CQ_LAUNCH(qz_zero, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, a.stream,
                       a.scale, a.minv, cnt, a.reset_status && a.ws != nullptr ? (int*)a.ws : nullptr);
    return hipSuccess;
  }
  const int chunks = (a.n + kChunk - 1) / kChunk;
  int* status = a.reset_status ? (int*)a.ws : nullptr;       // this path never waits: status 0
  float2* part = (float2*)((char*)a.ws + cqi::kWsHeader);
  QParams* prm = (QParams*)((char*)part + cqi::align_up((size_t)units * chunks * a.d * sizeof(float2), 256));
  const T* x = (const T*)a.x;
  CQ_LAUNCH(qz_stats<T>, dim3(chunks, units), dim3(kThreads), 0, a.stream, x, a.n, chunks, part, status);
  CQ_LAUNCH(qz_params, dim3(units), dim3(a.d), 0, a.stream, part, chunks, a.d, a.bits, a.scale, a.minv,
                     prm);
  const Rows g{(long)a.n, 0, a.n, a.n};
  return pack_bits<T>(a.bits, a.layout, x, g, prm, nullptr, nullptr, nullptr, a.codes, nullptr, nullptr, units,
                      a.stream);
}

}  // namespace

namespace cqi {

size_t quant_generic_ws(int B, int H, int n, int d) {
  const size_t units = (size_t)B * H;
  const size_t chunks = (size_t)(n + kChunk - 1) / kChunk;
  return kWsHeader + align_up(units * chunks * d * sizeof(float2), 256) + align_up(units * d * sizeof(QParams), 256);
}

hipError_t quant_generic(const QuantArgs& a) {
  return a.dtype == CQ_F16 ? run<__half>(a) : run<float>(a);
}

hipError_t quant_rows_generic(const RowsArgs& a, int bits, int layout, const float* mn, const float* mx,
                              const uint32_t* unit_mask, int n_codes, uint32_t* codes, float* scale, float* minv) {
  const int units = a.B * a.H;
  if (units == 0 || a.m == 0) return hipSuccess;
  const Rows g{a.x_rows, a.t0, a.t0 + a.m, n_codes};
  if (a.dtype == CQ_F16)
    return pack_bits<__half>(bits, layout, (const __half*)a.x, g, nullptr, mn, mx, unit_mask, codes, scale, minv,
                             units, a.stream);
  return pack_bits<float>(bits, layout, (const float*)a.x, g, nullptr, mn, mx, unit_mask, codes, scale, minv, units,
                          a.stream);
}

}  // namespace cqi
