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
// replaces this path for float16 inputs where it applies.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kChunk = 512;      // tokens per stats block
constexpr int kThreads = 256;

struct QParams {                 // per (unit, channel), in the workspace
  float mn, mx;
  double inv;                    // L / (mx - mn), 0 for a constant channel
};

template <typename T>
__global__ void __launch_bounds__(kThreads) qz_stats(const T* __restrict__ x, int n, int d,
                                                     int chunks, float2* __restrict__ part) {
  const int unit = blockIdx.y, chunk = blockIdx.x;
  const T* xu = x + (size_t)unit * n * d;
  const int c = threadIdx.x % d, r0 = threadIdx.x / d, rs = kThreads / d;
  const int i0 = chunk * kChunk, i1 = min(n, i0 + kChunk);
  float lo = INFINITY, hi = -INFINITY;
  for (int i = i0 + r0; i < i1; i += rs) {
    float v = cqd::to_f32(xu[(size_t)i * d + c]);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  __shared__ float slo[kThreads], shi[kThreads];
  slo[threadIdx.x] = lo;
  shi[threadIdx.x] = hi;
  __syncthreads();
  if (r0 == 0) {
    for (int r = 1; r < rs; ++r) {
      lo = fminf(lo, slo[r * d + c]);
      hi = fmaxf(hi, shi[r * d + c]);
    }
    part[((size_t)unit * chunks + chunk) * d + c] = make_float2(lo, hi);
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

template <typename T>
__device__ __forceinline__ int code_of(T xv, const QParams& p, int L) {
  if (!(p.inv > 0.0)) return 0;
  float x = cqd::to_f32(xv);
  double t = ((double)x - (double)p.mn) * p.inv;
  return cqd::exact_code(x, p.mn, p.mx, t, L);
}

// K layout: one thread per word (w, i).
template <typename T>
__global__ void __launch_bounds__(kThreads) qz_pack_k(const T* __restrict__ x, int n, int d, int bits,
                                                      const QParams* __restrict__ prm,
                                                      uint32_t* __restrict__ codes) {
  const int unit = blockIdx.y;
  const int E = 32 / bits, W = d / E, L = (1 << bits) - 1;
  const long idx = (long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long)W * n) return;
  const int w = (int)(idx / n), i = (int)(idx % n);
  const T* row = x + ((size_t)unit * n + i) * d + w * E;
  const QParams* pu = prm + (size_t)unit * d + w * E;
  uint32_t word = 0;
  for (int e = 0; e < E; ++e) word |= (uint32_t)code_of(row[e], pu[e], L) << cqd::code_off(e, bits);
  codes[((size_t)unit * W + w) * n + i] = word;
}

// V layout: one thread per word (r, j).
template <typename T>
__global__ void __launch_bounds__(kThreads) qz_pack_v(const T* __restrict__ x, int n, int d, int bits,
                                                      const QParams* __restrict__ prm,
                                                      uint32_t* __restrict__ codes) {
  const int unit = blockIdx.y;
  const int E = 32 / bits, R = (n + E - 1) / E, L = (1 << bits) - 1;
  const long idx = (long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long)R * d) return;
  const int r = (int)(idx / d), j = (int)(idx % d);
  const QParams p = prm[(size_t)unit * d + j];
  const T* col = x + (size_t)unit * n * d + j;
  uint32_t word = 0;
  for (int e = 0; e < E; ++e) {
    int i = r * E + e;
    if (i < n) word |= (uint32_t)code_of(col[(size_t)i * d], p, L) << cqd::code_off(e, bits);
  }
  codes[((size_t)unit * R + r) * d + j] = word;
}

// Empty cache: scale = minv = 0.
__global__ void qz_zero(float* scale, float* minv, long count) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    scale[i] = 0.0f;
    minv[i] = 0.0f;
  }
}

template <typename T>
hipError_t run(const cqi::QuantArgs& a) {
  const int units = a.B * a.H;
  if (units == 0) return hipSuccess;
  if (a.n == 0) {
    long cnt = (long)units * a.d;
    CQ_LAUNCH(qz_zero, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, a.stream,
                       a.scale, a.minv, cnt);
    return hipSuccess;
  }
  const int chunks = (a.n + kChunk - 1) / kChunk;
  float2* part = (float2*)a.ws;
  QParams* prm = (QParams*)((char*)a.ws + cqi::align_up((size_t)units * chunks * a.d * sizeof(float2), 256));
  const T* x = (const T*)a.x;
  CQ_LAUNCH(qz_stats<T>, dim3(chunks, units), dim3(kThreads), 0, a.stream, x, a.n, a.d, chunks, part);
  CQ_LAUNCH(qz_params, dim3(units), dim3(a.d), 0, a.stream, part, chunks, a.d, a.bits, a.scale, a.minv,
                     prm);
  const int E = 32 / a.bits;
  if (a.layout == CQ_LAYOUT_K) {
    long words = (long)(a.d / E) * a.n;
    CQ_LAUNCH(qz_pack_k<T>, dim3((unsigned)((words + kThreads - 1) / kThreads), units), dim3(kThreads), 0,
                       a.stream, x, a.n, a.d, a.bits, prm, a.codes);
  } else {
    long words = (long)((a.n + E - 1) / E) * a.d;
    CQ_LAUNCH(qz_pack_v<T>, dim3((unsigned)((words + kThreads - 1) / kThreads), units), dim3(kThreads), 0,
                       a.stream, x, a.n, a.d, a.bits, prm, a.codes);
  }
  return hipSuccess;
}

}  // namespace

namespace cqi {

size_t quant_generic_ws(int B, int H, int n, int d) {
  const size_t units = (size_t)B * H;
  const size_t chunks = (size_t)(n + kChunk - 1) / kChunk;
  return align_up(units * chunks * d * sizeof(float2), 256) + align_up(units * d * sizeof(QParams), 256);
}

hipError_t quant_generic(const QuantArgs& a) {
  return a.dtype == CQ_F16 ? run<__half>(a) : run<float>(a);
}

}  // namespace cqi
