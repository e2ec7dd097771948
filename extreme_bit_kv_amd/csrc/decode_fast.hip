// 1-bit post-scaled, calibrated decode attention on the matrix cores (gfx950).
//
// QbitAI article on CalibQuant, "Method" part 2: with per-channel scale and
// minimum, q . k_hat_i = (q * scale_K) . c_i + q . min_K and
// sum_i p_i v_hat_i = scale_V * sum_i p_i c_i + (sum_i p_i) min_V, so only the
// integer codes enter the products; part 3: the visual scores of each query
// head are mapped by the affine g fixed by their min and max before softmax.
//
// One workgroup (16 waves) per (batch, kv head); its query heads (G <= 4)
// share every code it reads.  A wave owns 128-token tiles.
//
// K side, per tile: C[16 x 16] += A[16 x 64] B[64 x 16] with
// v_mfma_i32_16x16x64_i8, twice (128 channels).  Rows of A are
// (head, digit plane): q * scale_K of each head is held as a 22-bit
// fixed-point integer split into three signed base-256 digits (row 4h + p,
// p < 3; row 4h + 3 is zero), so the int32 accumulation is exact.  Columns
// are tokens; B bytes are code bits, spread out of a packed word by
// (w >> s) & 0x01010101, which yields channels 4s..4s+3 of the word's group
// thanks to the interleaved packed layout.  Each lane ends up holding all
// planes of one (head, token) score: s = (a0 + 256 a1 + 65536 a2) 2^-F + c0.
// The scores stay in registers until the workgroup knows every head's min and
// max, which fix g.
//
// V side, per tile: C[16 x 16] += A[16 x 64] B[64 x 16], rows again
// (head, plane), columns channels, contraction over tokens.  p = exp(g(s) -
// max) in (0, 1] becomes P = round(p 2^22); its three bytes, the low two
// offset by -128 (xor 0x80) so that they are valid int8, are the digit
// planes.  Row 4h + 3 is all ones and counts the set code bits, which
// restores the -128 offsets.  A lane produces the digits of 8 consecutive
// tokens of one head, so one LDS write / read pair per wave hands them to the
// lanes that feed A, already in the byte order of the packed V words.
//
// The text tail (float K/V) is handled in plain float32 arithmetic.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 128;
constexpr int kMaxTail = 256;
constexpr int kPreTail = 64;          // tail tokens whose loads are issued in the prologue
constexpr float kLog2e = 1.4426950408889634f;

typedef int v4i __attribute__((ext_vector_type(4)));

struct Params {
  const void* q;
  const uint32_t* kc;
  const float* ks;
  const float* km;
  const uint32_t* vc;
  const float* vs;
  const float* vm;
  const void* kt;
  const void* vt;
  void* out;
  int Hq, Hkv, n, T;
  int q_f32, tail_f32, out_f32;
  float sm;
  int calib_on;
  float a_lo, c_lo, a_hi, c_hi;
};

__device__ __forceinline__ float ld_any(const void* p, size_t i, int is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[i] : __half2float(reinterpret_cast<const __half*>(p)[i]);
}

__device__ __forceinline__ v4i spread_lo(uint32_t w) {         // elements 0..15 of a packed word
  v4i r;
  r[0] = (int)(w & 0x01010101u);
  r[1] = (int)((w >> 1) & 0x01010101u);
  r[2] = (int)((w >> 2) & 0x01010101u);
  r[3] = (int)((w >> 3) & 0x01010101u);
  return r;
}
__device__ __forceinline__ v4i spread_hi(uint32_t w) {         // elements 16..31
  v4i r;
  r[0] = (int)((w >> 4) & 0x01010101u);
  r[1] = (int)((w >> 5) & 0x01010101u);
  r[2] = (int)((w >> 6) & 0x01010101u);
  r[3] = (int)((w >> 7) & 0x01010101u);
  return r;
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

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int G, int MAXT>
__global__ void __launch_bounds__(kThreads) df_b1(Params P) {
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T;
  const int ntiles = (n + kTile - 1) / kTile;
  const int R = n >> 5;

  __shared__ float s_q[4][128];                 // sm * q, float
  __shared__ float s_qp[4][128];                // sm * q * scale_K
  __shared__ double s_c0[4];
  __shared__ float s_inv2f[4];
  __shared__ int s_F[4];
  __shared__ uint32_t s_adig[4][3][32];         // K-side A digits: [head][plane][128 channel bytes]
  __shared__ float s_ts[4][kMaxTail];           // tail scores, then tail probabilities
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_lam[4], s_mu[4], s_tmax[4], s_ptail[4];
  __shared__ float s_tailred[8][4][128];        // tail values per token phase
  // Scores of tiles kRegT..MAXT-1 of each wave, one private 32-byte row per
  // lane (a 16-wave workgroup has 128 registers per lane; the first kRegT
  // tiles stay in registers).  After the value phase the same storage holds
  // the per-wave value partials.  With every tile in LDS, a wave stages its
  // V-side A digits ([head][plane][128 token bytes]) in the score rows of
  // the tile it has just read; otherwise in s_pdig.
  constexpr int kRegT = MAXT == 4 ? 0 : MAXT;
  constexpr bool kPdInSc = kRegT == 0;
  __shared__ uint32_t s_pdig[kPdInSc ? 1 : kWaves][4][3][32];
  constexpr int kLdsT = MAXT > kRegT ? MAXT - kRegT : 0;
  constexpr int kScBytes = kLdsT * kWaves * 64 * 32;
  constexpr int kRedBytes = kWaves * 4 * 128 * 4;
  __shared__ float4 s_big[(kScBytes > kRedBytes ? kScBytes : kRedBytes) / 16];
  float4 (*s_sc)[kWaves][64][2] = reinterpret_cast<float4 (*)[kWaves][64][2]>(s_big);
  float (*s_vred)[4][128] = reinterpret_cast<float (*)[4][128]>(s_big);
  __shared__ float s_psum[kWaves][4];

  // ---- prologue: post-scaled query, fixed-point digits -------------------
  __shared__ double s_c0p[8];
  __shared__ float s_mqp[8];
  if (tid < 4 * 128) {                          // waves 0..7: head = wave / 2
    const int hh = tid >> 7, j = tid & 127;
    float qv = 0.f, qp = 0.f;
    double pr = 0.0;
    if (hh < G) {
      qv = P.sm * ld_any(P.q, ((size_t)b * P.Hq + h * G + hh) * 128 + j, P.q_f32);
      qp = qv * P.ks[(size_t)unit * 128 + j];
      pr = (double)qv * (double)P.km[(size_t)unit * 128 + j];
    }
    s_q[hh][j] = qv;
    s_qp[hh][j] = qp;
    float aq = fabsf(qp);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      pr += __shfl_xor(pr, off);
      aq = fmaxf(aq, __shfl_xor(aq, off));
    }
    if (lane == 0) {
      s_c0p[wave] = pr;
      s_mqp[wave] = aq;
    }
  }
  __syncthreads();
  if (tid < 4) {
    const double c0 = s_c0p[2 * tid] + s_c0p[2 * tid + 1];
    const float mq = fmaxf(s_mqp[2 * tid], s_mqp[2 * tid + 1]);
    int F = 0;
    if (mq > 0.f) F = 21 - ilogbf(mq);
    s_F[tid] = F;
    s_inv2f[tid] = ldexpf(1.f, -F);
    s_c0[tid] = c0;
  }
  __syncthreads();
  if (tid < 4 * 128) {
    const int hh = tid >> 7, j = tid & 127;
    const int Q = (int)rintf(ldexpf(s_qp[hh][j], s_F[hh]));        // |Q| <= 2^22
    const int d0 = ((Q + 128) & 255) - 128;
    const int Q1 = (Q - d0) >> 8;
    const int d1 = ((Q1 + 128) & 255) - 128;
    const int d2 = (Q1 - d1) >> 8;
    unsigned char* ad = reinterpret_cast<unsigned char*>(&s_adig[hh][0][0]);
    ad[0 * 128 + j] = (unsigned char)d0;
    ad[1 * 128 + j] = (unsigned char)d1;
    ad[2 * 128 + j] = (unsigned char)d2;
  }
  __syncthreads();

  // ---- phase 1: visual scores ------------------------------------------
  const int i16 = lane & 15, g4 = lane >> 4;     // A/B operand lane coordinates
  const int rh = i16 >> 2, rp = i16 & 3;        // A row = (head rh, plane rp)
  v4i ak0 = {0, 0, 0, 0}, ak1 = {0, 0, 0, 0};
  if (rp < 3 && rh < G) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
    const uint4 x1 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4 + 4]);
    ak0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
    ak1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  const int oh = lane >> 4;                     // output lane: head
  const float inv2f = s_inv2f[oh < G ? oh : 0];
  const float c0f = (float)s_c0[oh < G ? oh : 0];
  float sc[kRegT > 0 ? kRegT : 1][8];
  float vmin = INFINITY, vmax = -INFINITY;
  auto load_k = [&](int t, uint4& w0, uint4& w1) {
    const int tile = wave + kWaves * t;
    const int tok = tile * kTile + 8 * i16;
    if (tile < ntiles && tok < n) {
      const uint4* src = reinterpret_cast<const uint4*>(P.kc + ((size_t)unit * 4 + g4) * n + tok);
      w0 = src[0];
      w1 = src[1];
    } else {
      w0 = make_uint4(0, 0, 0, 0);
      w1 = make_uint4(0, 0, 0, 0);
    }
  };
  uint4 kn0, kn1;                               // one tile of look-ahead
  load_k(0, kn0, kn1);
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const int tile = wave + kWaves * t;
    const uint32_t wd[8] = {kn0.x, kn0.y, kn0.z, kn0.w, kn1.x, kn1.y, kn1.z, kn1.w};
    if (t + 1 < MAXT) load_k(t + 1, kn0, kn1);
    const int tokb = tile * kTile + 8 * (lane & 15);   // this lane's output tokens tokb + m
    float st[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      v4i acc = {0, 0, 0, 0};
      acc = mfma(ak0, spread_lo(wd[m]), acc);
      acc = mfma(ak1, spread_hi(wd[m]), acc);
      const int dot = acc[0] + (acc[1] << 8) + (acc[2] << 16);
      const float s = fmaf((float)dot, inv2f, c0f);
      const bool valid = tile < ntiles && tokb + m < n;
      st[m] = s;
      if (valid) {
        vmin = fminf(vmin, s);
        vmax = fmaxf(vmax, s);
      }
    }
    if (t < kRegT) {
      // pin the finished scores: without this the compiler keeps the four
      // accumulator registers per token alive instead, and spills
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        asm volatile("" : "+v"(st[m]));
        sc[t < kRegT ? t : 0][m] = st[m];
      }
    } else {
      s_sc[t >= kRegT ? t - kRegT : 0][wave][lane][0] = make_float4(st[0], st[1], st[2], st[3]);
      s_sc[t >= kRegT ? t - kRegT : 0][wave][lane][1] = make_float4(st[4], st[5], st[6], st[7]);
    }
  }
  // the first value tile is requested before the score statistics settle
  auto load_v = [&](int t, uint4& w0, uint4& w1) {
    const int row = (wave + kWaves * t) * 4 + g4;   // V word row of this lane, channels 8*i16 .. +7
    if (row < R) {
      const uint4* src = reinterpret_cast<const uint4*>(P.vc + ((size_t)unit * R + row) * 128 + 8 * i16);
      w0 = src[0];
      w1 = src[1];
    } else {
      w0 = make_uint4(0, 0, 0, 0);
      w1 = make_uint4(0, 0, 0, 0);
    }
  };
  uint4 vn0, vn1;
  load_v(0, vn0, vn1);
  // ... and so are the first kPreTail tail tokens: keys as (token
  // 4 wave + lane/16, channels 8 (lane%16) ..+7), values as (channel
  // tid%128, tokens tid/128 + 8i).
  const int tsub = lane >> 4, tcl = lane & 15;
  uint4 ktp0 = make_uint4(0, 0, 0, 0), ktp1 = make_uint4(0, 0, 0, 0);
  {
    const int j = 4 * wave + tsub;
    if (j < T) {
      if (P.tail_f32) {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(P.kt) +
                                                          ((size_t)unit * T + j) * 128 + 8 * tcl);
        ktp0 = src[0];
        ktp1 = src[1];
      } else {
        ktp0 = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(P.kt) +
                                               ((size_t)unit * T + j) * 128 + 8 * tcl);
      }
    }
  }
  const int vtj = tid & 127, vtq = tid >> 7;
  float vtp[kPreTail / 8];
#pragma unroll
  for (int i = 0; i < kPreTail / 8; ++i) {
    const int t = vtq + 8 * i;
    vtp[i] = t < T ? ld_any(P.vt, ((size_t)unit * T + t) * 128 + vtj, P.tail_f32) : 0.f;
  }
  // ---- text tail scores ---------------------------------------------------
  {
    const int sub = tsub, cl = tcl;
    for (int j0 = 4 * wave; j0 < T; j0 += 4 * kWaves) {
      const int j = j0 + sub;
      float kf[8];
      if (j0 == 4 * wave) {                     // prefetched in the prologue
        if (P.tail_f32) {
          kf[0] = __uint_as_float(ktp0.x); kf[1] = __uint_as_float(ktp0.y);
          kf[2] = __uint_as_float(ktp0.z); kf[3] = __uint_as_float(ktp0.w);
          kf[4] = __uint_as_float(ktp1.x); kf[5] = __uint_as_float(ktp1.y);
          kf[6] = __uint_as_float(ktp1.z); kf[7] = __uint_as_float(ktp1.w);
        } else {
          const uint32_t hw[4] = {ktp0.x, ktp0.y, ktp0.z, ktp0.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          kf[c] = j < T ? ld_any(P.kt, ((size_t)unit * T + j) * 128 + 8 * cl + c, P.tail_f32) : 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(s_q[hh][8 * cl + c], kf[c], s);
        s += __shfl_xor(s, 8);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 1);
        if (cl == 0 && j < T) s_ts[hh][j] = s;
      }
    }
  }
  // ---- min / max of every head's visual scores ---------------------------
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  if ((lane & 15) == 0) {
    s_red[wave][oh][0] = vmin;
    s_red[wave][oh][1] = vmax;
  }
  __syncthreads();
  if (wave < G) {                               // wave hh settles head hh
    const int hh = wave;
    float m = lane < kWaves ? s_red[lane][hh][0] : INFINITY;
    float M = lane < kWaves ? s_red[lane][hh][1] : -INFINITY;
    float tmax = -INFINITY;
    for (int j = lane; j < T; j += 64) tmax = fmaxf(tmax, s_ts[hh][j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      m = fminf(m, __shfl_xor(m, off));
      M = fmaxf(M, __shfl_xor(M, off));
      tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    }
    if (lane == 0) {
      float lam = 1.f, mu = 0.f, vis_max = M;
      if (P.calib_on && n > 0) {
        const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
        lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
        mu = t_lo - lam * m;
        vis_max = fmaxf(t_lo, t_hi);
      }
      const float top = fmaxf(n > 0 ? vis_max : -INFINITY, tmax);
      s_lam[hh] = lam * kLog2e;                 // p = 2^(s * lam' + mu')
      s_mu[hh] = (mu - top) * kLog2e;
      s_tmax[hh] = top;
    }
  }
  __syncthreads();
  // tail probabilities (in place) and their sum, wave hh for head hh
  if (wave < G) {
    const int hh = wave;
    const float top = s_tmax[hh];
    float pt = 0.f;
    for (int j = lane; j < T; j += 64) {
      const float pj = exp2f((s_ts[hh][j] - top) * kLog2e);
      s_ts[hh][j] = pj;
      pt += pj;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pt += __shfl_xor(pt, off);
    if (lane == 0) s_ptail[hh] = pt;
  }
  __syncthreads();
  // text-tail values: thread (channel vtj, phase vtq) sums the tail tokens
  // vtq + 8i for every head, the first kPreTail from the prologue's loads
  {
    float ta[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kPreTail / 8; ++i) {
      const int t = vtq + 8 * i;
      if (t < T) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) ta[hh] = fmaf(s_ts[hh][t], vtp[i], ta[hh]);
      }
    }
    for (int t = kPreTail + vtq; t < T; t += 8) {
      const float v = ld_any(P.vt, ((size_t)unit * T + t) * 128 + vtj, P.tail_f32);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) ta[hh] = fmaf(s_ts[hh][t], v, ta[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s_tailred[vtq][hh][vtj] = ta[hh];
  }

  // ---- phase 2: values ------------------------------------------------------
  const float lam2 = s_lam[oh < G ? oh : 0], mu2 = s_mu[oh < G ? oh : 0];
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const int tile = wave + kWaves * t;
    if (tile >= ntiles) break;
    const uint4 vw0 = vn0, vw1 = vn1;
    if (t + 1 < MAXT) load_v(t + 1, vn0, vn1);
    // probabilities of this lane's 8 tokens (head oh), as 22-bit fixed point
    const int tokb = tile * kTile + 8 * (lane & 15);
    float st[8];
    if (t < kRegT) {
#pragma unroll
      for (int m = 0; m < 8; ++m) st[m] = sc[t < kRegT ? t : 0][m];
    } else {
      const float4 a0 = s_sc[t >= kRegT ? t - kRegT : 0][wave][lane][0], a1 = s_sc[t >= kRegT ? t - kRegT : 0][wave][lane][1];
      st[0] = a0.x; st[1] = a0.y; st[2] = a0.z; st[3] = a0.w;
      st[4] = a1.x; st[5] = a1.y; st[6] = a1.z; st[7] = a1.w;
    }
    // the wave's lanes have read their rows above; LDS keeps a wave's
    // accesses in order, so the digits may now overwrite them
    unsigned char* pd = kPdInSc ? reinterpret_cast<unsigned char*>(&s_sc[t >= kRegT ? t - kRegT : 0][wave][0][0])
                                : reinterpret_cast<unsigned char*>(&s_pdig[kPdInSc ? 0 : wave][0][0][0]);
    uint32_t fb[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float p = 0.f;
      if (oh < G && tokb + m < n) p = exp2f(fmaf(st[m], lam2, mu2));
      psum += p;
      fb[m] = __float_as_uint(fmaf(p, 4194304.f, 8388608.f)) ^ 0x00008080u;   // bytes: P^0x80, (P>>8)^0x80, P>>16
    }
    if (oh < G) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint32_t d0 = gather_byte(fb[0], fb[1], fb[2], fb[3], pl);
        const uint32_t d1 = gather_byte(fb[4], fb[5], fb[6], fb[7], pl);
        *reinterpret_cast<uint2*>(pd + (oh * 3 + pl) * 128 + 8 * (lane & 15)) = make_uint2(d0, d1);
      }
    }
    wave_sync_lds();
    v4i av0, av1;
    if (rp < 3) {
      if (rh < G) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(pd + (rh * 3 + rp) * 128 + 32 * g4);
        const uint4 x1 = *reinterpret_cast<const uint4*>(pd + (rh * 3 + rp) * 128 + 32 * g4 + 16);
        av0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
        av1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      } else {
        av0 = v4i{0, 0, 0, 0};
        av1 = av0;
      }
    } else {
      av0 = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
      av1 = av0;
    }
    const uint32_t vwd[8] = {vw0.x, vw0.y, vw0.z, vw0.w, vw1.x, vw1.y, vw1.z, vw1.w};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      vacc[ct] = mfma(av0, spread_lo(vwd[ct]), vacc[ct]);
      vacc[ct] = mfma(av1, spread_hi(vwd[ct]), vacc[ct]);
    }
    wave_sync_lds();                       // digits read before the next tile overwrites them
  }

  // ---- combine planes, reduce over waves --------------------------------
  __syncthreads();                          // every wave is done with the score rows
  // lane (head oh, column i16): channels 8*i16 + ct
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const float cnt128 = 128.f * (float)vacc[ct][3];
    const float sv = ((float)vacc[ct][0] + cnt128) + 256.f * ((float)vacc[ct][1] + cnt128) +
                     65536.f * (float)vacc[ct][2];
    s_vred[wave][oh][8 * i16 + ct] = sv * (1.f / 4194304.f);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
  if ((lane & 15) == 0) s_psum[wave][oh] = psum;
  __syncthreads();
  if (tid < G * 128) {
    const int hh = tid >> 7, j = tid & 127;
    float sv = 0.f, pv = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      sv += s_vred[w][hh][j];
      pv += s_psum[w][hh];
    }
    float tail = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) tail += s_tailred[q][hh][j];
    const float pt = T > 0 ? s_ptail[hh] : 0.f;
    float o = tail;
    if (n > 0) o += P.vs[(size_t)unit * 128 + j] * sv + pv * P.vm[(size_t)unit * 128 + j];
    o /= (pv + pt);
    const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
    if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
    else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
  }
}

template <int G>
hipError_t launch_g(const Params& p, int maxt, int units, hipStream_t st) {
  switch (maxt) {
    case 1: CQ_LAUNCH((df_b1<G, 1>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess;
    case 2: CQ_LAUNCH((df_b1<G, 2>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess;
    default: CQ_LAUNCH((df_b1<G, 4>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess;
  }
}

}  // namespace

namespace cqi {

size_t decode_fast_ws(int, int, int, int, int, int) { return 0; }

bool decode_fast_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  const int tiles = (a.n + kTile - 1) / kTile;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 &&
         tiles <= 4 * kWaves && a.T <= kMaxTail && (a.T == 0 || a.tail_dtype == a.q_dtype);
}

hipError_t decode_fast(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi};
  const int tiles = (a.n + kTile - 1) / kTile;
  const int maxt = tiles <= kWaves ? 1 : (tiles <= 2 * kWaves ? 2 : 4);
  const int G = a.Hq / a.Hkv;
  if (G == 1) return launch_g<1>(p, maxt, units, a.stream);
  if (G == 2) return launch_g<2>(p, maxt, units, a.stream);
  return launch_g<4>(p, maxt, units, a.stream);
}

}  // namespace cqi
