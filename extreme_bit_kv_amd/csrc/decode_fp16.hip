// Unquantized float16 split-K decode attention: the comparison baseline for
// the 1-bit path (not part of the method).  Each block owns one token split
// of one (batch, kv head): it computes the scores of its tokens for every
// query head of the group into LDS, takes their max, and accumulates
// p * V in float32; a second launch merges the split partials by
// log-sum-exp.  A wave reads four 256-byte rows per load (16 lanes x 16 B),
// so K and V stream through HBM once, fully coalesced.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGMax = 8;
constexpr int kD = cqd::kD;
constexpr int kMaxSplit = 1024;     // tokens per split (scores live in LDS)
constexpr int kRec = kD + 2;        // [max, l, acc[d]]

struct Shape {
  int B, Hq, Hkv, G, N, S, per;
};

__device__ __forceinline__ void load8(const __half* p, float* f) {
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float2 v = __half22float2(h[k]);
    f[2 * k] = v.x;
    f[2 * k + 1] = v.y;
  }
}

__global__ void __launch_bounds__(kThreads) f16_split(Shape sh, const __half* __restrict__ q,
                                                      const __half* __restrict__ k,
                                                      const __half* __restrict__ v, float sm,
                                                      float* __restrict__ part) {
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / sh.Hkv, h = unit % sh.Hkv, G = sh.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 4, cl = lane & 15;          // token row within the wave load, channel chunk
  const int t0 = min(sh.N, split * sh.per), t1 = min(sh.N, t0 + sh.per);
  __shared__ float sc[kGMax][kMaxSplit];
  __shared__ float red[kGMax][kWaves * 4];
  __shared__ float accs[kWaves][kGMax][kD];

  float qr[kGMax][8];
#pragma unroll
  for (int g = 0; g < kGMax; ++g) {
    if (g < G) {
      load8(q + ((size_t)b * sh.Hq + h * G + g) * kD + cl * 8, qr[g]);
#pragma unroll
      for (int c = 0; c < 8; ++c) qr[g][c] *= sm;
    }
  }
  const __half* ku = k + (size_t)unit * sh.N * kD;
  const __half* vu = v + (size_t)unit * sh.N * kD;
  // ---- scores ------------------------------------------------------------
  float mloc[kGMax];
#pragma unroll
  for (int g = 0; g < kGMax; ++g) mloc[g] = -INFINITY;
  for (int base = t0; base < t1; base += kWaves * 4) {
    const int tok = base + wave * 4 + sub;
    float kf[8];
    if (tok < t1) load8(ku + (size_t)tok * kD + cl * 8, kf);
    else {
#pragma unroll
      for (int c = 0; c < 8; ++c) kf[c] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      if (g < G) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qr[g][c], kf[c], s);
        s += __shfl_xor(s, 8);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 1);
        if (tok < t1) {
          if (cl == 0) sc[g][tok - t0] = s;
          mloc[g] = fmaxf(mloc[g], s);
        }
      }
    }
  }
  // block max per head
  if (cl == 0) {
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
      if (g < G) red[g][wave * 4 + sub] = mloc[g];
  }
  __syncthreads();
  __shared__ float smax[kGMax], ssum[kGMax];
  if (threadIdx.x < G) {
    float m = -INFINITY;
    for (int k2 = 0; k2 < kWaves * 4; ++k2) m = fmaxf(m, red[threadIdx.x][k2]);
    smax[threadIdx.x] = m;
  }
  __syncthreads();
  // probabilities in place, and their sums
  const int cnt = t1 - t0;
  __shared__ float red2[kGMax][kWaves];
  for (int g = 0; g < G; ++g) {
    float l = 0.f;
    for (int i = threadIdx.x; i < cnt; i += kThreads) {
      float p = __expf(sc[g][i] - smax[g]);
      sc[g][i] = p;
      l += p;
    }
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) red2[g][wave] = l;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float l = 0.f;
    for (int w = 0; w < kWaves; ++w) l += red2[threadIdx.x][w];
    ssum[threadIdx.x] = l;
  }
  // ---- values ------------------------------------------------------------
  float acc[kGMax][8];
#pragma unroll
  for (int g = 0; g < kGMax; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
  for (int base = t0; base < t1; base += kWaves * 4) {
    const int tok = base + wave * 4 + sub;
    if (tok < t1) {
      float vf[8];
      load8(vu + (size_t)tok * kD + cl * 8, vf);
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        if (g < G) {
          float p = sc[g][tok - t0];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(p, vf[c], acc[g][c]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kGMax; ++g) {
    if (g < G) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float a = acc[g][c];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        if (sub == 0) accs[wave][g][cl * 8 + c] = a;
      }
    }
  }
  __syncthreads();
  float* rec = part + ((size_t)unit * sh.S + split) * G * kRec;
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    int g = idx / kD, j = idx % kD;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += accs[w][g][j];
    rec[g * kRec + 2 + j] = a;
  }
  if (threadIdx.x < G) {
    rec[threadIdx.x * kRec + 0] = smax[threadIdx.x];
    rec[threadIdx.x * kRec + 1] = cnt > 0 ? ssum[threadIdx.x] : 0.f;
  }
}

__global__ void f16_merge(Shape sh, const float* __restrict__ part, __half* __restrict__ out) {
  const int hq_all = blockIdx.x;
  const int b = hq_all / sh.Hq, hq = hq_all % sh.Hq, h = hq / sh.G, g = hq % sh.G;
  const int unit = b * sh.Hkv + h, j = threadIdx.x;
  const float* base = part + (size_t)unit * sh.S * sh.G * kRec;
  float Mx = -INFINITY;
  for (int s = 0; s < sh.S; ++s) {
    const float* rec = base + ((size_t)s * sh.G + g) * kRec;
    if (rec[1] > 0.f) Mx = fmaxf(Mx, rec[0]);
  }
  float num = 0.f, den = 0.f;
  for (int s = 0; s < sh.S; ++s) {
    const float* rec = base + ((size_t)s * sh.G + g) * kRec;
    if (!(rec[1] > 0.f)) continue;
    float w = __expf(rec[0] - Mx);
    den = fmaf(w, rec[1], den);
    num = fmaf(w, rec[2 + j], num);
  }
  out[(size_t)hq_all * kD + j] = __float2half_rn(num / den);
}

Shape make_shape(int B, int Hq, int Hkv, int N) {
  const int units = B * Hkv;
  int S = (N + kMaxSplit - 1) / kMaxSplit;
  while ((long)units * S < 2048 && (N + S * 2 - 1) / (S * 2) >= 128) S *= 2;
  int per = (N + S - 1) / S;
  per = (per + 15) / 16 * 16;
  if (per > kMaxSplit) per = kMaxSplit;
  S = (N + per - 1) / per;
  return Shape{B, Hq, Hkv, Hq / Hkv, N, S, per};
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
  CQ_LAUNCH(f16_split, dim3(sh.S, B * Hkv), dim3(kThreads), 0, st, sh, (const __half*)q,
                     (const __half*)k, (const __half*)v, sm_scale, part);
  CQ_LAUNCH(f16_merge, dim3(B * Hq), dim3(kD), 0, st, sh, part, (__half*)out);
  return hipSuccess;
}

}  // namespace cqi
