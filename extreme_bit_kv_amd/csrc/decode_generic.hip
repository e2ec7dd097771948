// Decode attention over the packed visual cache, general path: any bits in
// {1,2,4,8}, GQA group sizes up to 8, float16/float32 query, tail and output.
//
// QbitAI article on CalibQuant, "Method" part 2 (post-scaling): the
// per-channel dequantization is deferred into the vector products, so the
// kernels multiply integer codes by q*scale_K (keys) and accumulate
// p*code before applying scale_V (values); part 3 (calibration): the
// pre-softmax scores of each query head are mapped by g using their min and
// max.  Only the visual cache is quantized; the text tail stays float.
//
// Launches: (1) scores of every visual token for every query head, written
// to the workspace, plus each split's score min/max; (2) per split, the
// calibrated probabilities and the integer-code value accumulation (one extra
// block per (batch, kv head) handles the tail); (3) log-sum-exp merge of the
// split partials and the final scale_V / min_V application.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kGMax = 8;
constexpr int kD = cqd::kD;
constexpr int kMaxSplits = 64;

struct Shape {
  int B, Hq, Hkv, G, n, T, d, bits, S;
  int nc;    // token capacity of the code buffers (their layout is that of nc >= n tokens)
};

__device__ __forceinline__ void split_range(int n, int S, int s, int& t0, int& t1) {
  // splits are multiples of 32 tokens so that V words never straddle two splits
  int rows = (n + 31) / 32;
  int per = (rows + S - 1) / S;
  t0 = min(n, s * per * 32);
  t1 = min(n, (s + 1) * per * 32);
}

template <typename QT>
__global__ void __launch_bounds__(kThreads) dg_scores(Shape sh, const QT* __restrict__ q,
                                                      const uint32_t* __restrict__ kc,
                                                      const float* __restrict__ ks,
                                                      const float* __restrict__ km, float sm,
                                                      float* __restrict__ scores,
                                                      float2* __restrict__ mm) {
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / sh.Hkv, h = unit % sh.Hkv, G = sh.G;
  __shared__ float qp[kGMax][kD];
  __shared__ float qm[kGMax][kD];
  __shared__ float c0[kGMax];
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    int g = idx / kD, j = idx % kD;
    float qv = cqd::to_f32(q[((size_t)b * sh.Hq + h * G + g) * kD + j]);
    qp[g][j] = sm * qv * ks[(size_t)unit * kD + j];
    qm[g][j] = sm * qv * km[(size_t)unit * kD + j];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float s = 0.f;
    for (int j = 0; j < kD; ++j) s += qm[threadIdx.x][j];
    c0[threadIdx.x] = s;
  }
  __syncthreads();
  int t0, t1;
  split_range(sh.n, sh.S, split, t0, t1);
  const int E = 32 / sh.bits, W = kD / E, L = (1 << sh.bits) - 1;
  float lo[kGMax], hi[kGMax];
#pragma unroll
  for (int g = 0; g < kGMax; ++g) { lo[g] = INFINITY; hi[g] = -INFINITY; }
  for (int i = t0 + threadIdx.x; i < t1; i += kThreads) {
    float acc[kGMax];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) acc[g] = 0.f;
    for (int w = 0; w < W; ++w) {
      uint32_t word = kc[((size_t)unit * W + w) * sh.nc + i];
      for (int e = 0; e < E; ++e) {
        float c = (float)((word >> cqd::code_off(e, sh.bits)) & L);
        int j = w * E + e;
#pragma unroll
        for (int g = 0; g < kGMax; ++g)
          if (g < G) acc[g] = fmaf(qp[g][j], c, acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      if (g < G) {
        float s = acc[g] + c0[g];
        scores[((size_t)b * sh.Hq + h * G + g) * sh.n + i] = s;
        lo[g] = fminf(lo[g], s);
        hi[g] = fmaxf(hi[g], s);
      }
    }
  }
  if (mm == nullptr) return;                    // scores only (cq_visual_scores)
  __shared__ float rlo[kThreads], rhi[kThreads];
  for (int g = 0; g < G; ++g) {
    rlo[threadIdx.x] = lo[g];
    rhi[threadIdx.x] = hi[g];
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
      if (threadIdx.x < off) {
        rlo[threadIdx.x] = fminf(rlo[threadIdx.x], rlo[threadIdx.x + off]);
        rhi[threadIdx.x] = fmaxf(rhi[threadIdx.x], rhi[threadIdx.x + off]);
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) mm[((size_t)unit * sh.S + split) * G + g] = make_float2(rlo[0], rhi[0]);
    __syncthreads();
  }
}

struct CalibP {
  int on;
  float a_lo, c_lo, a_hi, c_hi;
};

// Partial record per (unit, split, head): [shift, l, acc[0..d)].
constexpr int kRec = kD + 2;

template <typename QT, typename TT>
__global__ void __launch_bounds__(kThreads) dg_attend(Shape sh, CalibP cal, const QT* __restrict__ q,
                                                      const float* __restrict__ scores,
                                                      const float2* __restrict__ mm,
                                                      const uint32_t* __restrict__ vc,
                                                      const TT* __restrict__ kt, const TT* __restrict__ vt,
                                                      float sm, float* __restrict__ tail_s,
                                                      float* __restrict__ part) {
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / sh.Hkv, h = unit % sh.Hkv, G = sh.G;
  const int nsplit = sh.S + (sh.T > 0 ? 1 : 0);
  __shared__ float lam[kGMax], mu[kGMax], shift[kGMax];
  __shared__ float pbuf[kGMax][32];
  __shared__ float red[kThreads];
  float acc[kGMax];
#pragma unroll
  for (int g = 0; g < kGMax; ++g) acc[g] = 0.f;
  float lsum = 0.f;     // thread-partial sum of p for head (threadIdx.x / 32)

  if (split < sh.S) {
    // ---- visual split -------------------------------------------------
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float m = INFINITY, M = -INFINITY;
      for (int s = 0; s < sh.S; ++s) {
        float2 v = mm[((size_t)unit * sh.S + s) * G + g];
        m = fminf(m, v.x);
        M = fmaxf(M, v.y);
      }
      if (cal.on) {
        float t_lo = cal.a_lo * m + cal.c_lo, t_hi = cal.a_hi * M + cal.c_hi;
        float l = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
        lam[g] = l;
        mu[g] = t_lo - l * m;
        shift[g] = M > m ? fmaxf(t_lo, t_hi) : t_lo;    // the largest value of g
      } else {
        lam[g] = 1.f;
        mu[g] = 0.f;
        shift[g] = M;
      }
    }
    __syncthreads();
    int t0, t1;
    split_range(sh.n, sh.S, split, t0, t1);
    const int E = 32 / sh.bits, L = (1 << sh.bits) - 1, R = (sh.nc + E - 1) / E;   // word rows per unit
    const int pg = threadIdx.x / 32, pe = threadIdx.x % 32;     // (head, element) of the p producer
    for (int r = t0 / E; r * E < t1; ++r) {
      if (pg < G && pe < E) {
        int i = r * E + pe;
        float p = 0.f;
        if (i < t1) {
          float s = scores[((size_t)b * sh.Hq + h * G + pg) * sh.n + i];
          p = __expf(lam[pg] * s + mu[pg] - shift[pg]);
        }
        pbuf[pg][pe] = p;
        lsum += p;
      }
      __syncthreads();
      if (threadIdx.x < kD) {
        uint32_t word = vc[((size_t)unit * R + r) * kD + threadIdx.x];
        for (int e = 0; e < E; ++e) {
          float c = (float)((word >> cqd::code_off(e, sh.bits)) & L);
#pragma unroll
          for (int g = 0; g < kGMax; ++g)
            if (g < G) acc[g] = fmaf(pbuf[g][e], c, acc[g]);
        }
      }
      __syncthreads();
    }
  } else {
    // ---- text-tail block ------------------------------------------------
    __shared__ float qf[kGMax][kD];
    for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
      int g = idx / kD, j = idx % kD;
      qf[g][j] = sm * cqd::to_f32(q[((size_t)b * sh.Hq + h * G + g) * kD + j]);
    }
    __syncthreads();
    float* ts = tail_s + (size_t)unit * G * sh.T;
    const TT* ktu = kt + (size_t)unit * sh.T * kD;
    const TT* vtu = vt + (size_t)unit * sh.T * kD;
    for (int idx = threadIdx.x; idx < G * sh.T; idx += kThreads) {
      int g = idx / sh.T, j = idx % sh.T;
      float s = 0.f;
      for (int c = 0; c < kD; ++c) s = fmaf(qf[g][c], cqd::to_f32(ktu[(size_t)j * kD + c]), s);
      ts[g * sh.T + j] = s;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      float M = -INFINITY;
      for (int j = 0; j < sh.T; ++j) M = fmaxf(M, ts[threadIdx.x * sh.T + j]);
      shift[threadIdx.x] = M;
    }
    __syncthreads();
    if (threadIdx.x < kD) {
      for (int j = 0; j < sh.T; ++j) {
        float v = cqd::to_f32(vtu[(size_t)j * kD + threadIdx.x]);
#pragma unroll
        for (int g = 0; g < kGMax; ++g)
          if (g < G) acc[g] = fmaf(__expf(ts[g * sh.T + j] - shift[g]), v, acc[g]);
      }
    }
    if (threadIdx.x < G * 32) {
      int g = threadIdx.x / 32;
      for (int j = threadIdx.x % 32; j < sh.T; j += 32) lsum += __expf(ts[g * sh.T + j] - shift[g]);
    }
  }
  // ---- write the partial record ------------------------------------------
  red[threadIdx.x] = lsum;
  __syncthreads();
  float* rec = part + ((size_t)unit * nsplit + split) * G * kRec;
  if (threadIdx.x < G) {
    float l = 0.f;
    for (int k = 0; k < 32; ++k) l += red[threadIdx.x * 32 + k];
    rec[threadIdx.x * kRec + 0] = shift[threadIdx.x];
    rec[threadIdx.x * kRec + 1] = l;
  }
  if (threadIdx.x < kD) {
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
      if (g < G) rec[g * kRec + 2 + threadIdx.x] = acc[g];
  }
}

template <typename OT>
__global__ void dg_merge(Shape sh, const float* __restrict__ part, const float* __restrict__ vs,
                         const float* __restrict__ vm, OT* __restrict__ out) {
  const int hq_all = blockIdx.x;
  const int b = hq_all / sh.Hq, hq = hq_all % sh.Hq, h = hq / sh.G, g = hq % sh.G;
  const int unit = b * sh.Hkv + h;
  const int nsplit = sh.S + (sh.T > 0 ? 1 : 0);
  const int j = threadIdx.x;
  const float* base = part + (size_t)unit * nsplit * sh.G * kRec;
  float Mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) {
    const float* rec = base + ((size_t)s * sh.G + g) * kRec;
    if (rec[1] > 0.f) Mx = fmaxf(Mx, rec[0]);
  }
  float num = 0.f, pvis = 0.f, den = 0.f, tail = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* rec = base + ((size_t)s * sh.G + g) * kRec;
    if (!(rec[1] > 0.f)) continue;
    float w = __expf(rec[0] - Mx);
    den = fmaf(w, rec[1], den);
    if (s < sh.S) {
      num = fmaf(w, rec[2 + j], num);
      pvis = fmaf(w, rec[1], pvis);
    } else {
      tail = fmaf(w, rec[2 + j], tail);
    }
  }
  float o = 0.f;
  if (sh.S > 0) o = vs[(size_t)unit * kD + j] * num + pvis * vm[(size_t)unit * kD + j];
  o = (o + tail) / den;
  out[(size_t)hq_all * kD + j] = cqd::from_f32<OT>(o);
}

template <typename QT, typename TT, typename OT>
hipError_t run(const cqi::DecodeArgs& a, int S) {
  Shape sh{a.B, a.Hq, a.Hkv, a.Hq / a.Hkv, a.n, a.T, a.d, a.bits, S, a.nc};
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  const int nsplit = S + (a.T > 0 ? 1 : 0);
  char* ws = (char*)a.ws;
  float* scores = (float*)ws;
  ws += cqi::align_up((size_t)a.B * a.Hq * a.n * sizeof(float), 256);
  float2* mm = (float2*)ws;
  ws += cqi::align_up((size_t)units * S * sh.G * sizeof(float2), 256);
  float* tail_s = (float*)ws;
  ws += cqi::align_up((size_t)units * sh.G * a.T * sizeof(float), 256);
  float* part = (float*)ws;
  CalibP cal{a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi};
  if (S > 0)
    CQ_LAUNCH(dg_scores<QT>, dim3(S, units), dim3(kThreads), 0, a.stream, sh, (const QT*)a.q,
                       a.k_codes, a.k_scale, a.k_min, a.sm_scale, scores, mm);
  CQ_LAUNCH((dg_attend<QT, TT>), dim3(nsplit, units), dim3(kThreads), 0, a.stream, sh, cal,
                     (const QT*)a.q, scores, mm, a.v_codes, (const TT*)a.k_tail, (const TT*)a.v_tail,
                     a.sm_scale, tail_s, part);
  CQ_LAUNCH(dg_merge<OT>, dim3(a.B * a.Hq), dim3(kD), 0, a.stream, sh, part, a.v_scale, a.v_min,
                     (OT*)a.out);
  return hipSuccess;
}

template <typename QT, typename TT>
hipError_t pick_out(const cqi::DecodeArgs& a, int S) {
  return a.out_dtype == CQ_F16 ? run<QT, TT, __half>(a, S) : run<QT, TT, float>(a, S);
}
template <typename QT>
hipError_t pick_tail(const cqi::DecodeArgs& a, int S) {
  return a.tail_dtype == CQ_F16 ? pick_out<QT, __half>(a, S) : pick_out<QT, float>(a, S);
}

}  // namespace

namespace cqi {

int decode_generic_splits(int n, int units, int requested) {
  if (n == 0) return 0;
  const int rows = (n + 31) / 32;
  int S = requested > 0 ? (requested < kMaxSplits ? requested : kMaxSplits) : 0;
  if (S == 0) {
    S = 1;
    while (S < kMaxSplits && (long)units * S < 1024 && rows / (S * 2) >= 4) S *= 2;
  }
  if (S > rows) S = rows;
  return S;
}

size_t decode_generic_ws(int B, int Hq, int Hkv, int n, int T, int d, int S) {
  const size_t units = (size_t)B * Hkv, G = Hq / Hkv;
  const size_t nsplit = S + (T > 0 ? 1 : 0);
  return align_up((size_t)B * Hq * n * sizeof(float), 256) + align_up(units * S * G * sizeof(float2), 256) +
         align_up(units * G * T * sizeof(float), 256) + align_up(units * nsplit * G * kRec * sizeof(float), 256);
}

hipError_t decode_generic(const DecodeArgs& a) {
  const int S = decode_generic_splits(a.n, a.B * a.Hkv, a.splits);
  return a.q_dtype == CQ_F16 ? pick_tail<__half>(a, S) : pick_tail<float>(a, S);
}

hipError_t visual_scores(const void* q, int q_dtype, const uint32_t* k_codes, const float* k_scale,
                         const float* k_min, int B, int Hq, int Hkv, int n, int bits, float sm_scale,
                         float* scores, hipStream_t st) {
  const int units = B * Hkv;
  if (units == 0 || n == 0) return hipSuccess;
  const int S = decode_generic_splits(n, units, 0);
  Shape sh{B, Hq, Hkv, Hq / Hkv, n, 0, kD, bits, S, n};
  if (q_dtype == CQ_F16)
    CQ_LAUNCH(dg_scores<__half>, dim3(S, units), dim3(kThreads), 0, st, sh, (const __half*)q, k_codes, k_scale,
              k_min, sm_scale, scores, (float2*)nullptr);
  else
    CQ_LAUNCH(dg_scores<float>, dim3(S, units), dim3(kThreads), 0, st, sh, (const float*)q, k_codes, k_scale,
              k_min, sm_scale, scores, (float2*)nullptr);
  return hipSuccess;
}

}  // namespace cqi
