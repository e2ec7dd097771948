// The calibration map g applied to a matrix of pre-softmax scores, row by
// row (QbitAI article on CalibQuant, "Method" part 3: a linear map sends the
// interval [m, M] that holds a row's scores onto a target interval before the
// softmax, taming the extreme scores that 1-bit reconstruction produces).
// One block per row: min/max reduction, then the affine map in float64.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) cal_rows(const float* s, int n, int enabled, float a_lo,
                                                     float c_lo, float a_hi, float c_hi, float* out,
                                                     float* __restrict__ mm) {
  const size_t row = blockIdx.x;
  const float* sr = s + row * n;
  float* orow = out + row * n;
  float lo = INFINITY, hi = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    float v = sr[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  __shared__ float rlo[kThreads], rhi[kThreads];
  rlo[threadIdx.x] = lo;
  rhi[threadIdx.x] = hi;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      rlo[threadIdx.x] = fminf(rlo[threadIdx.x], rlo[threadIdx.x + off]);
      rhi[threadIdx.x] = fmaxf(rhi[threadIdx.x], rhi[threadIdx.x + off]);
    }
    __syncthreads();
  }
  const double m = rlo[0], M = rhi[0];
  if (mm != nullptr && threadIdx.x == 0) {
    mm[row * 2 + 0] = (float)m;
    mm[row * 2 + 1] = (float)M;
  }
  const double t_lo = (double)a_lo * m + (double)c_lo;
  const double t_hi = (double)a_hi * M + (double)c_hi;
  const double span = M - m;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    float v = sr[i];
    float r;
    if (!enabled) r = v;
    else if (span > 0.0) r = (float)(t_lo + ((double)v - m) * (t_hi - t_lo) / span);
    else r = (float)t_lo;
    orow[i] = r;
  }
}

}  // namespace

namespace cqi {

hipError_t calibrate_rows(const float* scores, int R, int n, int enabled, float a_lo, float c_lo, float a_hi,
                          float c_hi, float* out, float* row_minmax, hipStream_t st) {
  if (R == 0) return hipSuccess;
  CQ_LAUNCH(cal_rows, dim3(R), dim3(kThreads), 0, st, scores, n, enabled, a_lo, c_lo, a_hi, c_hi, out,
                     row_minmax);
  return hipSuccess;
}

}  // namespace cqi
