// Unquantized float16 split-K decode attention: the comparison baseline for
// the 1-bit path (not part of the method).  Each block owns one token split
// of one (batch, kv head) and makes one pass over it with an online softmax
// (flash-decoding): K and V rows are read together, so each byte crosses HBM
// once.  A 16-lane group holds one 256-byte row (16 B per lane); a wave reads
// four rows per load and keeps four loads of K and four of V in flight.
// Scores use packed fp16 dot products with float32 accumulation; every
// 16-lane group keeps its own running max, sum and float32 p*V accumulator,
// and the groups and waves combine at the end.  A second launch merges the
// split partials by log-sum-exp.
#include "cq_device.h"
#include "cq_internal.h"

#include <algorithm>

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kD = cqd::kD;
constexpr int kRows = 4;              // rows per 16-lane group per step
constexpr int kStep = kWaves * 4 * kRows;   // rows per block per step
constexpr int kRec = kD + 2;          // [max (log2 domain), l, acc[d]]
constexpr int kSplitRows = 1024;     // rows per split when that gives enough blocks
constexpr int kMinBlocks = 1024;     // two rounds of resident blocks (2 per CU)

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

struct Shape {
  int B, Hq, Hkv, G, N, S, per;
};

// x + x rotated by R lanes within its row of 16 lanes (DPP row_ror).
template <int R>
__device__ __forceinline__ float add_ror(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + R,
                                                                   0xF, 0xF, false));
}

// Sums over the 16 lanes of a row (every lane receives its row's sum): rotations
// by 8, 4, 2 and 1 lanes, the independent sums interleaved so that each DPP
// read is not right behind the write it depends on.
template <int N>
__device__ __forceinline__ void row_sum16(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = add_ror<8>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = add_ror<4>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = add_ror<2>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = add_ror<1>(x[i]);
}

__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }

template <int G>
__global__ void __launch_bounds__(kThreads) f16_split(Shape sh, const __half* __restrict__ q,
                                                      const __half* __restrict__ k,
                                                      const __half* __restrict__ v, float sm_log2,
                                                      float* __restrict__ part) {
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / sh.Hkv, h = unit % sh.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 4, cl = lane & 15;          // row within a 4-row load, 8-channel chunk
  const int t0 = min(sh.N, split * sh.per), t1 = min(sh.N, t0 + sh.per);

  uint4 qw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {   // q is only 4-byte aligned
    const uint32_t* qp = reinterpret_cast<const uint32_t*>(q + ((size_t)b * sh.Hq + h * G + g) * kD + cl * 8);
    qw[g] = make_uint4(qp[0], qp[1], qp[2], qp[3]);
  }
  const __half* ku = k + (size_t)unit * sh.N * kD + cl * 8;
  const __half* vu = v + (size_t)unit * sh.N * kD + cl * 8;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
  }
  for (int base = t0 + wave * 4 * kRows; base < t1; base += kStep) {
    // rows past the split re-read its last row (in bounds) and get p = 0;
    // K and V are read once, so the loads are non-temporal
    uint4 kr[kRows], vr[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      kr[r] = cqd::ld_nt(ku + (size_t)min(base + r * 4 + sub, t1 - 1) * kD);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      vr[r] = cqd::ld_nt(vu + (size_t)min(base + r * 4 + sub, t1 - 1) * kD);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float d = 0.f;
        d = __builtin_amdgcn_fdot2(as_h2(qw[g].x), as_h2(kr[r].x), d, false);
        d = __builtin_amdgcn_fdot2(as_h2(qw[g].y), as_h2(kr[r].y), d, false);
        d = __builtin_amdgcn_fdot2(as_h2(qw[g].z), as_h2(kr[r].z), d, false);
        d = __builtin_amdgcn_fdot2(as_h2(qw[g].w), as_h2(kr[r].w), d, false);
        s[r] = d;
      }
      row_sum16(s);
#pragma unroll
      for (int r = 0; r < kRows; ++r) s[r] = base + r * 4 + sub < t1 ? s[r] * sm_log2 : -INFINITY;
      float mn = m[g];
#pragma unroll
      for (int r = 0; r < kRows; ++r) mn = fmaxf(mn, s[r]);
      const float mu = mn == -INFINITY ? 0.f : mn;   // a fully masked group keeps p = alpha = 0
      // v_exp_f32 directly: results below 2^-126 flush to 0, which a softmax weight can lose
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mu);
      float p[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - mu);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < kRows; ++r) ps += p[r];
      l[g] = l[g] * alpha + ps;
      m[g] = mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= alpha;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const uint32_t w[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const h2 vv = as_h2(w[c]);
          acc[g][2 * c] = fmaf(p[r], (float)vv.x, acc[g][2 * c]);
          acc[g][2 * c + 1] = fmaf(p[r], (float)vv.y, acc[g][2 * c + 1]);
        }
      }
    }
  }
  // combine the four row groups of the wave (lanes 16 and 32 apart)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = fmaxf(m[g], __shfl_xor(m[g], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float sc = M == -INFINITY ? 0.f : exp2f(m[g] - M);
    l[g] *= sc;
    l[g] += __shfl_xor(l[g], 16);
    l[g] += __shfl_xor(l[g], 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a = acc[g][c] * sc;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[g][c] = a;
    }
    m[g] = M;
  }
  // combine the waves
  __shared__ float s_acc[kWaves][G][kD];
  __shared__ float s_ml[kWaves][G][2];
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wave][g][cl * 8 + c] = acc[g][c];
      if (cl == 0) {
        s_ml[wave][g][0] = m[g];
        s_ml[wave][g][1] = l[g];
      }
    }
  }
  __syncthreads();
  float* rec = part + ((size_t)unit * sh.S + split) * G * kRec;
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    const int g = idx / kD, j = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][g][0]);
    float a = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = s_ml[w][g][0] == -INFINITY ? 0.f : exp2f(s_ml[w][g][0] - M);
      a = fmaf(sc, s_acc[w][g][j], a);
      ls = fmaf(sc, s_ml[w][g][1], ls);
    }
    rec[g * kRec + 2 + j] = a;
    if (j == 0) {
      rec[g * kRec + 0] = M;
      rec[g * kRec + 1] = ls;
    }
  }
}

// One block of kD threads per (batch, query head).  Each wave forms the
// log-sum-exp weights of the S split partials itself (lanes over splits),
// then thread j sums weight * acc[j] over the splits.
__global__ void __launch_bounds__(kD) f16_merge(Shape sh, const float* __restrict__ part,
                                                __half* __restrict__ out) {
  const int hq_all = blockIdx.x;
  const int b = hq_all / sh.Hq, hq = hq_all % sh.Hq, h = hq / sh.G, g = hq % sh.G;
  const int unit = b * sh.Hkv + h, j = threadIdx.x, lane = threadIdx.x & 63;
  const float* base = part + (size_t)unit * sh.S * sh.G * kRec + (size_t)g * kRec;
  const size_t stride = (size_t)sh.G * kRec;   // between splits
  float mx = -INFINITY;
  for (int s = lane; s < sh.S; s += 64) {
    const float* rec = base + s * stride;
    if (rec[1] > 0.f) mx = fmaxf(mx, rec[0]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float den = 0.f;
  for (int s = lane; s < sh.S; s += 64) {
    const float* rec = base + s * stride;
    if (rec[1] > 0.f) den = fmaf(exp2f(rec[0] - mx), rec[1], den);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  float num = 0.f;
#pragma unroll 4
  for (int s = 0; s < sh.S; ++s) {
    const float* rec = base + s * stride;
    const float w = rec[1] > 0.f ? exp2f(rec[0] - mx) : 0.f;
    num = fmaf(w, rec[2 + j], num);
  }
  out[(size_t)hq_all * kD + j] = __float2half_rn(num / den);
}

// Scores only: scores[b][hq][i] = sm * q . k_i, float32, for the fp16 cache.
// Block (64-token chunk, unit); a 16-lane group takes one row (16 B per
// lane), as in the split kernel.
template <int G>
__global__ void __launch_bounds__(256) f16_scores(int Hq, int Hkv, int N, const __half* __restrict__ q,
                                                  const __half* __restrict__ k, float sm,
                                                  float* __restrict__ scores) {
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 4, cl = lane & 15;
  uint4 qw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {   // q is only 4-byte aligned
    const uint32_t* qp = reinterpret_cast<const uint32_t*>(q + ((size_t)b * Hq + h * G + g) * kD + cl * 8);
    qw[g] = make_uint4(qp[0], qp[1], qp[2], qp[3]);
  }
  const int t0 = blockIdx.x * 64 + wave * 16;
  uint4 kr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    kr[r] = *reinterpret_cast<const uint4*>(k + ((size_t)unit * N + min(t0 + r * 4 + sub, N - 1)) * kD + cl * 8);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float d[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = 0.f;
      x = __builtin_amdgcn_fdot2(as_h2(qw[g].x), as_h2(kr[r].x), x, false);
      x = __builtin_amdgcn_fdot2(as_h2(qw[g].y), as_h2(kr[r].y), x, false);
      x = __builtin_amdgcn_fdot2(as_h2(qw[g].z), as_h2(kr[r].z), x, false);
      x = __builtin_amdgcn_fdot2(as_h2(qw[g].w), as_h2(kr[r].w), x, false);
      d[r] = x;
    }
    row_sum16(d);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = t0 + r * 4 + sub;
      if (cl == 0 && tok < N) scores[((size_t)b * Hq + h * G + g) * N + tok] = d[r] * sm;
    }
  }
}

// Splits of about kSplitRows rows, more and shorter ones when that leaves
// fewer than kMinBlocks blocks; each split a multiple of one step of rows and
// non-empty.
Shape make_shape(int B, int Hq, int Hkv, int N) {
  const long units = (long)B * Hkv;
  int S = std::max((N + kSplitRows - 1) / kSplitRows, (int)std::min<long>(N, (kMinBlocks + units - 1) / units));
  S = std::max(S, 1);
  int per = (N + S - 1) / S;
  per = std::max(kStep, (per + kStep - 1) / kStep * kStep);
  S = (N + per - 1) / per;
  return Shape{B, Hq, Hkv, Hq / Hkv, N, S, per};
}

template <int G>
hipError_t launch_split(const Shape& sh, const void* q, const void* k, const void* v, float sm_log2, float* part,
                  hipStream_t st) {
  CQ_LAUNCH(f16_split<G>, dim3(sh.S, sh.B * sh.Hkv), dim3(kThreads), 0, st, sh, (const __half*)q,
            (const __half*)k, (const __half*)v, sm_log2, part);
  return hipSuccess;
}

}  // namespace

namespace cqi {

size_t decode_fp16_ws(int B, int Hq, int Hkv, int N, int d) {
  Shape sh = make_shape(B, Hq, Hkv, N);
  return align_up((size_t)B * Hkv * sh.S * sh.G * kRec * sizeof(float), 256);
}

hipError_t decode_fp16(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N, int d,
                       float sm_scale, void* out, void* ws, hipStream_t st) {
  if (B == 0) return hipSuccess;
  Shape sh = make_shape(B, Hq, Hkv, N);
  float* part = (float*)ws;
  const float sl = sm_scale * 1.4426950408889634f;   // scores in the log2 domain
  hipError_t e;
  switch (sh.G) {
    case 1: e = launch_split<1>(sh, q, k, v, sl, part, st); break;
    case 2: e = launch_split<2>(sh, q, k, v, sl, part, st); break;
    case 3: e = launch_split<3>(sh, q, k, v, sl, part, st); break;
    case 4: e = launch_split<4>(sh, q, k, v, sl, part, st); break;
    case 5: e = launch_split<5>(sh, q, k, v, sl, part, st); break;
    case 6: e = launch_split<6>(sh, q, k, v, sl, part, st); break;
    case 7: e = launch_split<7>(sh, q, k, v, sl, part, st); break;
    case 8: e = launch_split<8>(sh, q, k, v, sl, part, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  CQ_LAUNCH(f16_merge, dim3(B * Hq), dim3(kD), 0, st, sh, part, (__half*)out);
  return hipSuccess;
}

hipError_t scores_fp16(const void* q, const void* k, int B, int Hq, int Hkv, int N, float sm_scale, float* scores,
                       hipStream_t st) {
  if (B == 0 || N == 0) return hipSuccess;
  const dim3 grid((N + 63) / 64, B * Hkv);
  const __half* qh = (const __half*)q;
  const __half* kh = (const __half*)k;
  switch (Hq / Hkv) {
    case 1: CQ_LAUNCH(f16_scores<1>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 2: CQ_LAUNCH(f16_scores<2>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 3: CQ_LAUNCH(f16_scores<3>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 4: CQ_LAUNCH(f16_scores<4>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 5: CQ_LAUNCH(f16_scores<5>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 6: CQ_LAUNCH(f16_scores<6>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 7: CQ_LAUNCH(f16_scores<7>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    case 8: CQ_LAUNCH(f16_scores<8>, grid, dim3(256), 0, st, Hq, Hkv, N, qh, kh, sm_scale, scores); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

}  // namespace cqi
