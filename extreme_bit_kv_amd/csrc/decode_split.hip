// 1-bit post-scaled, calibrated decode attention as two launches over token
// chunks (gfx950).
//
// QbitAI article on CalibQuant, "Method" part 2 (post-scaling: only the
// integer codes enter the products) and part 3 (the visual scores of each
// query head are mapped by the affine g fixed by their min and max before
// softmax).  The arithmetic is that of the one-launch kernel in
// decode_fast.hip: the same 22-bit fixed-point query digits, the same int8
// matrix-core products, the same probability digits.  What differs is the
// schedule.
//
// g is affine on [m, M], so once every head's visual min and max are known
// the largest calibrated visual score is max(t_lo, t_hi), and the softmax
// reference top = max(that, largest tail score) is known before any
// probability is formed.  Every chunk then uses the same reference, and the
// chunks' partial sums simply add: no running maximum, no rescaling.
//
//   ds_keys   workgroup (unit, chunk): scores of the chunk's key tiles, their
//             min and max per head -> mm.  Chunk 0 also scores the text tail
//             (tsc, tmx).
//   ds_vals   workgroup (unit, chunk): g and top from all chunks' mm; the key
//             tiles again (the first launch left them in the Infinity
//             Cache), the same scores recomputed exactly, p, the value
//             product; the chunk's sum_i P_i c_i and sum_i P_i -> part.
//             Chunk 0 also forms the text tail's sums.
//   ds_merge  workgroup (unit): adds the records -> out.
//
// Against one workgroup per unit, the two big launches are plain streams over
// the codes: no phase in which all of the device waits on reductions while
// HBM idles, and many more workgroups than CUs, so the dispatcher balances
// them.  The merge is a launch of its own rather than the last workgroup of
// each unit: on gfx950 the agent-scope fences such a hand-off needs write back
// and invalidate a whole L2, and the launch boundary gives the same ordering
// once.
#include "cq_device.h"
#include "cq_internal.h"
#include "cq_mfma.h"

namespace {

using namespace cqm;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 128;                  // tokens per key / value tile
constexpr int kMaxTail = 256;
constexpr int kPart = 132;                  // floats per (chunk, head): 128 channels, sum P, padding
constexpr int kMinBlocks = 1024;            // workgroups wanted per launch: one round at 4 per CU
constexpr int kKeyAhead = 2;                // key tiles per wave in flight in the key pass
constexpr float kLog2e = 1.4426950408889634f;

struct SParams {
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
  int out_f32;
  float sm;
  int calib_on;
  float a_lo, c_lo, a_hi, c_hi;
  int nc;              // chunks per unit
  int ct;              // key tiles per chunk
  float* mm;           // [unit][chunk][4][2]: min, max of each head's visual scores
  float* tsc;          // [unit][4][T]: text-tail scores
  float* tmx;          // [unit][4]: their max
  float* part;         // [unit][nc + 1][4][kPart]: chunk records, then the tail record
  int ncap;            // token capacity of the code buffers (their layout is that of ncap >= n tokens)
};

struct QSmem {
  float q[4][128];                          // sm * q, float (tail scores)
  __align__(16) uint32_t adig[4][3][32];    // [head][plane][128 channel bytes]
  double c0[4];
  float inv2f[4];
  int F[4];
  double c0p[8];
  float mqp[8];
};

// The query-side inputs of one thread (head idx / 128, channel idx % 128 for
// idx = tid + kThreads it).  They are requested before the code tiles: loads
// complete in order, so a prologue that asked for them after the tiles would
// wait for every tile first.  The loads take no branch (heads >= G read head
// G - 1 and are zeroed later): at a branch join the compiler loses count of
// the loads in flight and waits for all of them.
constexpr int kQIt = 512 / kThreads;
struct QLoad {
  uint32_t q[kQIt];             // raw bits: float32, or float16 in the low half
  float ks[kQIt], km[kQIt];
};

template <int G, bool F32>
__device__ __forceinline__ QLoad q_load(const SParams& P, int unit, int b, int h) {
  QLoad l;
#pragma unroll
  for (int it = 0; it < kQIt; ++it) {
    const int idx = threadIdx.x + kThreads * it, hh = idx >> 7, j = idx & 127;
    const size_t qi = ((size_t)b * P.Hq + h * G + (hh < G ? hh : G - 1)) * 128 + j;
    if constexpr (F32) l.q[it] = reinterpret_cast<const uint32_t*>(P.q)[qi];
    else l.q[it] = reinterpret_cast<const unsigned short*>(P.q)[qi];
    l.ks[it] = P.ks[(size_t)unit * 128 + j];
    l.km[it] = P.km[(size_t)unit * 128 + j];
  }
  return l;
}

// Post-scaled query of every head as three signed base-256 digits of a 22-bit
// fixed-point integer, and c0 = sm q . min_K: the operations, and their order,
// of the one-launch kernel, so both produce identical scores.
template <int G, bool F32>
__device__ __forceinline__ void q_prologue(const SParams& P, const QLoad& l, QSmem& s) {
  const int tid = threadIdx.x, lane = tid & 63;
  float qps[kQIt];
#pragma unroll
  for (int it = 0; it < kQIt; ++it) {
    const int idx = tid + kThreads * it, hh = idx >> 7, j = idx & 127;
    // selects, not a branch (see q_load)
    const float qr = F32 ? __uint_as_float(l.q[it]) : __half2float(__ushort_as_half((unsigned short)l.q[it]));
    const float qv = hh < G ? P.sm * qr : 0.f;
    const float qp = qv * l.ks[it];
    const double pr0 = (double)qv * (double)l.km[it];
    double pr = hh < G ? pr0 : 0.0;
    s.q[hh][j] = qv;
    qps[it] = qp;
    float aq = fabsf(qp);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      pr += __shfl_xor(pr, off);
      aq = fmaxf(aq, __shfl_xor(aq, off));
    }
    if (lane == 0) {
      s.c0p[idx >> 6] = pr;
      s.mqp[idx >> 6] = aq;
    }
  }
  lds_barrier();
  if (tid < 4) {
    const double c0 = s.c0p[2 * tid] + s.c0p[2 * tid + 1];
    const float mq = fmaxf(s.mqp[2 * tid], s.mqp[2 * tid + 1]);
    int F = 0;
    if (mq > 0.f) F = 21 - ilogbf(mq);
    s.F[tid] = F;
    s.inv2f[tid] = ldexpf(1.f, -F);
    s.c0[tid] = c0;
  }
  lds_barrier();
#pragma unroll
  for (int it = 0; it < kQIt; ++it) {
    const int idx = tid + kThreads * it, hh = idx >> 7, j = idx & 127;
    const int Q = (int)rintf(ldexpf(qps[it], s.F[hh]));           // |Q| <= 2^22
    const int d0 = ((Q + 128) & 255) - 128;
    const int Q1 = (Q - d0) >> 8;
    const int d1 = ((Q1 + 128) & 255) - 128;
    const int d2 = (Q1 - d1) >> 8;
    unsigned char* ad = reinterpret_cast<unsigned char*>(&s.adig[hh][0][0]);
    ad[0 * 128 + j] = (unsigned char)d0;
    ad[1 * 128 + j] = (unsigned char)d1;
    ad[2 * 128 + j] = (unsigned char)d2;
  }
  lds_barrier();
}

// Key operands and score scaling of this lane: A rows (head rh, plane rp),
// output head oh.
struct KeyOp {
  v4i ak0, ak1;
  float inv2f, c0f;
};

template <int G>
__device__ __forceinline__ KeyOp key_op(const QSmem& s, int lane) {
  const int i16 = lane & 15, g4 = lane >> 4, rh = i16 >> 2, rp = i16 & 3, oh = lane >> 4;
  KeyOp k;
  k.ak0 = v4i{0, 0, 0, 0};
  k.ak1 = v4i{0, 0, 0, 0};
  if (rp < 3 && rh < G) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(&s.adig[rh][rp][8 * g4]);
    const uint4 x1 = *reinterpret_cast<const uint4*>(&s.adig[rh][rp][8 * g4 + 4]);
    k.ak0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
    k.ak1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  k.inv2f = s.inv2f[oh < G ? oh : 0];
  k.c0f = (float)s.c0[oh < G ? oh : 0];
  return k;
}

// Scores of this lane's 8 tokens (head oh, tokens tok_of(i16, m)) from one key tile.
__device__ __forceinline__ void tile_scores(const KeyOp& k, const uint4& w0, const uint4& w1, float (&st)[8]) {
  const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    v4i acc = {0, 0, 0, 0};
    acc = mfma(k.ak0, spread_lo(wd[m]), acc);
    acc = mfma(k.ak1, spread_hi(wd[m]), acc);
    const int dot = acc[0] + (acc[1] << 8) + (acc[2] << 16);
    st[m] = fmaf((float)dot, k.inv2f, k.c0f);
    asm volatile("" : "+v"(st[m]));          // the score, not the accumulators, stays live
  }
}

// Code tiles are loaded without a branch (a load under a branch is waited for
// at the join), from addresses clamped into the unit: tokens past n read the
// last ones again.  Their scores are never used (`ok`), and their probability
// is 0, which makes their value codes drop out of the product (digits -128,
// -128, 0 plus the count row: -128 c - 128 * 256 c + 128 (1 + 256) c = 0).

// Each load instruction reads 16 B per lane with the 16 lanes of a row group
// back to back (256 B), so every byte an instruction fetches is used by it:
// a lane holds word positions 4 i16 .. +3 and 64 + 4 i16 .. +3, not 8
// consecutive ones (with those, each instruction would take every other
// 16 B, and its partner would fetch the same lines again once the caches had
// dropped them).

// Key words of this lane for a tile: plane g4 of tokens tile*128 + tok_of(i16, m).
__device__ __forceinline__ int tok_of(int i16, int m) { return (m < 4 ? 4 * i16 : 64 + 4 * i16 - 4) + m; }

__device__ __forceinline__ void load_key(const uint32_t* kc, int unit, int n, int ncap, int tile, int lane,
                                         uint4& w0, uint4& w1) {
  const int i16 = lane & 15, g4 = lane >> 4;
  const uint32_t* plane = kc + ((size_t)unit * 4 + g4) * ncap;
  w0 = *reinterpret_cast<const uint4*>(plane + min(tile * kTile + 4 * i16, n - 4));
  w1 = *reinterpret_cast<const uint4*>(plane + min(tile * kTile + 64 + 4 * i16, n - 4));
}

// Value words of this lane for a tile: word row 4 tile + g4 (32 tokens) of
// channels ch_of(i16, c), c < 8.
__device__ __forceinline__ int ch_of(int i16, int c) { return (c < 4 ? 4 * i16 : 64 + 4 * i16 - 4) + c; }

__device__ __forceinline__ void load_val(const uint32_t* vc, int unit, int R, int Rcap, int tile, int lane,
                                         uint4& w0, uint4& w1) {
  const int i16 = lane & 15, g4 = lane >> 4;
  const uint32_t* row = vc + ((size_t)unit * Rcap + min(tile * 4 + g4, R - 1)) * 128;
  w0 = *reinterpret_cast<const uint4*>(row + 4 * i16);
  w1 = *reinterpret_cast<const uint4*>(row + 64 + 4 * i16);
}

// ---- launch 1: key pass ---------------------------------------------------
// MT key tiles per wave, kKeyAhead of them in flight: the first right after
// the query inputs, each later one as a tile is taken.
template <int G, bool F32, int MT>
__global__ void __launch_bounds__(kThreads, 4) ds_keys(SParams P) {
  const int unit = blockIdx.x / P.nc, chunk = blockIdx.x % P.nc;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T, ntiles = (n + kTile - 1) / kTile;
  const int i16 = lane & 15, oh = lane >> 4;
  __shared__ QSmem qs;
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_ts[4][kMaxTail];

  constexpr int D = MT < kKeyAhead ? MT : kKeyAhead;
  const QLoad ql = q_load<G, F32>(P, unit, b, h);
  uint4 kw[D][2];
#pragma unroll
  for (int t = 0; t < D; ++t)
    load_key(P.kc, unit, n, P.ncap, chunk * P.ct + wave + kWaves * t, lane, kw[t][0], kw[t][1]);
  q_prologue<G, F32>(P, ql, qs);
  const KeyOp ko = key_op<G>(qs, lane);

  float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tile = chunk * P.ct + wave + kWaves * t;
    // n % 32 == 0: each group of 4 tokens of this lane is all valid or none
    const bool okA = tile < ntiles && tile * kTile + tok_of(i16, 0) < n;
    const bool okB = tile < ntiles && tile * kTile + tok_of(i16, 4) < n;
    float st[8];
    const uint4 w0 = kw[t % D][0], w1 = kw[t % D][1];
    if (t + D < MT) load_key(P.kc, unit, n, P.ncap, tile + kWaves * D, lane, kw[t % D][0], kw[t % D][1]);
    tile_scores(ko, w0, w1, st);
    const float amin = fminf(fminf(st[0], st[1]), fminf(st[2], st[3]));
    const float amax = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
    const float bmin = fminf(fminf(st[4], st[5]), fminf(st[6], st[7]));
    const float bmax = fmaxf(fmaxf(st[4], st[5]), fmaxf(st[6], st[7]));
    if (okA) {
      vmin = fminf(vmin, amin);
      vmax = fmaxf(vmax, amax);
    }
    if (okB) {
      vmin = fminf(vmin, bmin);
      vmax = fmaxf(vmax, bmax);
    }
    asm volatile("" : "+v"(vmin), "+v"(vmax));   // fold tile by tile
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  if (i16 == 0) {
    s_red[wave][oh][0] = vmin;
    s_red[wave][oh][1] = vmax;
  }
  // chunk 0: text-tail scores, 16 lanes per token (8 channels each)
  if (chunk == 0) {
    const int sub = lane >> 4, cl = lane & 15;
    for (int j0 = 4 * wave; j0 < T; j0 += 4 * kWaves) {
      const int j = j0 + sub;
      float kf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) kf[c] = 0.f;
      if (j < T) {
        if constexpr (F32) {
          const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(P.kt) +
                                                            ((size_t)unit * T + j) * 128 + 8 * cl);
          const uint4 a = src[0], c4 = src[1];
          kf[0] = __uint_as_float(a.x); kf[1] = __uint_as_float(a.y);
          kf[2] = __uint_as_float(a.z); kf[3] = __uint_as_float(a.w);
          kf[4] = __uint_as_float(c4.x); kf[5] = __uint_as_float(c4.y);
          kf[6] = __uint_as_float(c4.z); kf[7] = __uint_as_float(c4.w);
        } else {
          const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(P.kt) +
                                                          ((size_t)unit * T + j) * 128 + 8 * cl);
          const uint32_t hw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qs.q[hh][8 * cl + c], kf[c], s);
        s += __shfl_xor(s, 8);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 1);
        if (cl == 0 && j < T) s_ts[hh][j] = s;
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = INFINITY, M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      m = fminf(m, s_red[w][tid][0]);
      M = fmaxf(M, s_red[w][tid][1]);
    }
    float* dst = P.mm + ((size_t)unit * P.nc + chunk) * 8 + 2 * tid;
    dst[0] = m;
    dst[1] = M;
  }
  if (chunk == 0 && wave < G) {
    const int hh = wave;
    float tm = -INFINITY;
    for (int j = lane; j < T; j += 64) {
      const float s = s_ts[hh][j];
      P.tsc[((size_t)unit * 4 + hh) * T + j] = s;
      tm = fmaxf(tm, s);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
    if (lane == 0) P.tmx[(size_t)unit * 4 + hh] = tm;
  }
}

// ---- launch 2: value pass ---------------------------------------------------
// Record c < nc of a unit: the visual chunk c (alpha sum_i P_i c_i / 2^27 per
// channel, then alpha sum_i P_i / 2^27, with P_i the fixed-point weight of
// token i relative to the largest visual one and alpha that one's weight
// relative to the softmax reference).  Record nc, written by chunk 0: the text tail
// (sum_j p_j vt_j per channel, then sum_j p_j).
template <int G, bool F32, int MT>
__global__ void __launch_bounds__(kThreads, 4) ds_vals(SParams P) {
  const int unit = blockIdx.x / P.nc, chunk = blockIdx.x % P.nc;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T, ntiles = (n + kTile - 1) / kTile, R = n >> 5;
  const int i16 = lane & 15, g4 = lane >> 4, rh = i16 >> 2, rp = i16 & 3, oh = lane >> 4;
  __shared__ QSmem qs;
  __shared__ __align__(16) uint32_t s_pdig[kWaves][4][4][32];   // [head][plane][128 token bytes]
  __shared__ unsigned long long s_vsum[4][128];   // sum P c per head and channel (2^-27 units)
  __shared__ double s_psum[4];                     // sum P per head (2^-27 units)
  __shared__ float s_lam[4], s_mu[4], s_top[4], s_alpha[4];
  if (tid < 4) s_psum[tid] = 0.0;
  for (int i = tid; i < 4 * 128; i += kThreads) (&s_vsum[0][0])[i] = 0ull;

  // requested in this order: query inputs, every chunk's min / max, then codes
  const QLoad ql = q_load<G, F32>(P, unit, b, h);
  // wave hh < G gathers head hh over chunks lane, lane + 64, ... (branch-free
  // loads, as above; lanes past the last chunk repeat it)
  const int hw = wave < G ? wave : G - 1;
  const float2 mm0 = *reinterpret_cast<const float2*>(P.mm + ((size_t)unit * P.nc + min(lane, P.nc - 1)) * 8 + 2 * hw);
  const float tmx0 = P.tmx[(size_t)unit * 4 + hw];
  const int tile0 = chunk * P.ct + wave;
  uint4 kn0, kn1, vn0, vn1;                    // one tile of look-ahead
  load_key(P.kc, unit, n, P.ncap, tile0, lane, kn0, kn1);
  load_val(P.vc, unit, R, P.ncap >> 5, tile0, lane, vn0, vn1);
  q_prologue<G, F32>(P, ql, qs);
  const KeyOp ko = key_op<G>(qs, lane);

  // g and the softmax reference of every head
  if (wave < G) {
    const int hh = wave;
    float m = mm0.x, M = mm0.y;
    const float tmax = T > 0 ? tmx0 : -INFINITY;
    for (int c = lane + 64; c < P.nc; c += 64) {
      const float2 v = *reinterpret_cast<const float2*>(P.mm + ((size_t)unit * P.nc + c) * 8 + 2 * hh);
      m = fminf(m, v.x);
      M = fmaxf(M, v.y);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      m = fminf(m, __shfl_xor(m, off));
      M = fmaxf(M, __shfl_xor(M, off));
    }
    float lam = 1.f, mu = 0.f, vis_max = M;
    if (P.calib_on) {
      const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
      lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
      mu = t_lo - lam * m;
      // the largest value of g: the larger end of [t_lo, t_hi], or t_lo
      // when every score is the same (g is then the constant t_lo)
      vis_max = M > m ? fmaxf(t_lo, t_hi) : t_lo;
    }
    const float top = fmaxf(vis_max, tmax);
    if (lane == 0) {
      s_lam[hh] = lam * kLog2e;                 // p / p_max = 2^(s lam' + mu')
      s_mu[hh] = (mu - vis_max) * kLog2e;
      s_top[hh] = top;
      s_alpha[hh] = exp2f((vis_max - top) * kLog2e);
    }
  }
  lds_barrier();                                // the first tiles stay in flight

  const float lam2 = s_lam[oh < G ? oh : 0], mu2 = s_mu[oh < G ? oh : 0];
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  double psum = 0.0;                           // sum of this lane's P (exact: integers below 2^53)
  unsigned char* pd = reinterpret_cast<unsigned char*>(&s_pdig[wave][0][0][0]);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tile = tile0 + kWaves * t;
    if (tile >= ntiles) break;
    const uint4 kw0 = kn0, kw1 = kn1, vw0 = vn0, vw1 = vn1;
    if (t + 1 < MT) {
      load_key(P.kc, unit, n, P.ncap, tile + kWaves, lane, kn0, kn1);
      load_val(P.vc, unit, R, P.ncap >> 5, tile + kWaves, lane, vn0, vn1);
    }
    // probabilities of this lane's 8 tokens (head oh), as 22-bit fixed point
    const bool okA = oh < G && tile * kTile + tok_of(i16, 0) < n;
    const bool okB = oh < G && tile * kTile + tok_of(i16, 4) < n;
    float st[8];
    tile_scores(ko, kw0, kw1, st);
    // P = round(p 2^27) as four signed base-256 digits
    uint32_t fb[8], ptile = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float p = 0.f;
      if (m < 4 ? okA : okB) p = exp2f(fmaf(st[m], lam2, mu2));
      const uint32_t Pm = cqm::p_fixed(p);
      ptile += Pm;
      fb[m] = cqm::sdigits(Pm);
    }
    psum += (double)ptile;
    if (oh < G) {
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) {
        // token order within the tile: tokens 4 i16 .. +3, then 64 + 4 i16 .. +3
        *reinterpret_cast<uint32_t*>(pd + (oh * 4 + pl) * 128 + tok_of(i16, 0)) =
            gather_byte(fb[0], fb[1], fb[2], fb[3], pl);
        *reinterpret_cast<uint32_t*>(pd + (oh * 4 + pl) * 128 + tok_of(i16, 4)) =
            gather_byte(fb[4], fb[5], fb[6], fb[7], pl);
      }
    }
    wave_sync_lds();
    v4i av0 = {0, 0, 0, 0}, av1 = {0, 0, 0, 0};
    if (rh < G) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(pd + (rh * 4 + rp) * 128 + 32 * g4);
      const uint4 x1 = *reinterpret_cast<const uint4*>(pd + (rh * 4 + rp) * 128 + 32 * g4 + 16);
      av0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
      av1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
    const uint32_t vwd[8] = {vw0.x, vw0.y, vw0.z, vw0.w, vw1.x, vw1.y, vw1.z, vw1.w};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      vacc[ct] = mfma(av0, spread_lo(vwd[ct]), vacc[ct]);
      vacc[ct] = mfma(av1, spread_hi(vwd[ct]), vacc[ct]);
    }
    wave_sync_lds();                            // digits read before the next tile overwrites them
  }

  // ---- the chunk's record ------------------------------------------------
  // exact integer sums, as in the one-launch kernel: the waves add theirs with
  // 64-bit LDS atomics
  if (oh < G) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const long long sv = (long long)vacc[ct][0] + 256ll * vacc[ct][1] + 65536ll * vacc[ct][2] +
                           16777216ll * vacc[ct][3];
      atomicAdd(&s_vsum[oh][ch_of(i16, ct)], (unsigned long long)sv);
    }
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
  if (i16 == 0 && oh < G) atomicAdd(&s_psum[oh], psum);
  __syncthreads();
  float* rec = P.part + ((size_t)unit * (P.nc + 1) + chunk) * 4 * kPart;
  for (int idx = tid; idx < G * 128; idx += kThreads) {
    const int hh = idx >> 7, j = idx & 127;
    rec[hh * kPart + j] = (float)((double)(long long)s_vsum[hh][j] * (1.0 / 134217728.0) * s_alpha[hh]);
  }
  if (tid < G) rec[tid * kPart + 128] = (float)(s_psum[tid] * (1.0 / 134217728.0) * s_alpha[tid]);
  if (chunk != 0) return;

  // ---- chunk 0: the text tail's record --------------------------------------
  __shared__ float s_pt[4][kMaxTail];
  __shared__ float s_tailred[kThreads / 128][4][128];
  float* trec = P.part + ((size_t)unit * (P.nc + 1) + P.nc) * 4 * kPart;
  if (wave < G) {                               // tail probabilities of head `wave`
    const int hh = wave;
    const float top = s_top[hh];
    float pt = 0.f;
    for (int j = lane; j < T; j += 64) {
      const float pj = exp2f((P.tsc[((size_t)unit * 4 + hh) * T + j] - top) * kLog2e);
      s_pt[hh][j] = pj;
      pt += pj;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pt += __shfl_xor(pt, off);
    if (lane == 0) trec[hh * kPart + 128] = pt;
  }
  __syncthreads();
  {                                             // tail values: channel tid % 128, tokens of one phase
    constexpr int kPh = kThreads / 128;
    const int j = tid & 127, ph = tid >> 7;
    float ta[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int t = ph; t < T; t += kPh) {
      const float v = ld_any(P.vt, ((size_t)unit * T + t) * 128 + j, F32);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) ta[hh] = fmaf(s_pt[hh][t], v, ta[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s_tailred[ph][hh][j] = ta[hh];
  }
  __syncthreads();
  for (int idx = tid; idx < G * 128; idx += kThreads) {
    const int hh = idx >> 7, j = idx & 127;
    float tail = 0.f;
#pragma unroll
    for (int q = 0; q < kThreads / 128; ++q) tail += s_tailred[q][hh][j];
    trec[hh * kPart + j] = tail;
  }
}

// ---- launch 3: the unit's merge ----------------------------------------------
//   out = (tail + v_scale * sum_c sv_c + v_min * sum_c pv_c) / (sum_c pv_c + p_tail)
template <int G>
__global__ void __launch_bounds__(kThreads) ds_merge(SParams P) {
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const float* ru = P.part + (size_t)unit * (P.nc + 1) * 4 * kPart;
  for (int idx = threadIdx.x; idx < G * 128; idx += kThreads) {
    const int hh = idx >> 7, j = idx & 127;
    float sv = 0.f, pv = 0.f;
#pragma unroll 4
    for (int c = 0; c < P.nc; ++c) {
      sv += ru[((size_t)c * 4 + hh) * kPart + j];
      pv += ru[((size_t)c * 4 + hh) * kPart + 128];
    }
    const float* tr = ru + ((size_t)P.nc * 4 + hh) * kPart;
    float o = tr[j] + P.vs[(size_t)unit * 128 + j] * sv + pv * P.vm[(size_t)unit * 128 + j];
    o /= (pv + tr[128]);
    const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
    if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
    else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
  }
}

// Chunking: MT tiles per wave, kWaves * MT tiles per chunk; the largest MT
// (fewest, longest chunks) that still gives kMinBlocks workgroups, so that the
// per-workgroup prologue is paid as few times as possible.
struct Chunking {
  int mt, nc, ct;
};

Chunking chunking(int units, int n, int requested) {
  const int ntiles = (n + kTile - 1) / kTile;
  Chunking c{1, 1, kWaves};
  for (int mt : {8, 4, 2, 1}) {
    c.mt = mt;
    c.ct = kWaves * mt;
    c.nc = (ntiles + c.ct - 1) / c.ct;
    if ((long)units * c.nc >= kMinBlocks) break;
  }
  if (requested > 0) {                          // a caller's chunk count: tiles per wave follow from it
    const int per_wave = (ntiles + (long)requested * kWaves - 1) / ((long)requested * kWaves);
    c.mt = per_wave <= 1 ? 1 : (per_wave <= 2 ? 2 : (per_wave <= 4 ? 4 : 8));
    c.ct = kWaves * c.mt;
    c.nc = (ntiles + c.ct - 1) / c.ct;
  }
  return c;
}

struct WsLayout {
  size_t mm, tsc, tmx, part, total;
};

WsLayout ws_layout(int units, int nc, int T) {
  WsLayout w;
  size_t o = 0;
  w.mm = o;   o = cqi::align_up(o + (size_t)units * nc * 8 * sizeof(float), 256);
  w.tsc = o;  o = cqi::align_up(o + (size_t)units * 4 * T * sizeof(float), 256);
  w.tmx = o;  o = cqi::align_up(o + (size_t)units * 4 * sizeof(float), 256);
  w.part = o; o = cqi::align_up(o + (size_t)units * (nc + 1) * 4 * kPart * sizeof(float), 256);
  w.total = o;
  return w;
}

template <int G, bool F32, int MT>
hipError_t launch_mt(const SParams& p, int units, hipStream_t st) {
  const dim3 grid((unsigned)(units * p.nc));
  CQ_LAUNCH((ds_keys<G, F32, MT>), grid, dim3(kThreads), 0, st, p);
  CQ_LAUNCH((ds_vals<G, F32, MT>), grid, dim3(kThreads), 0, st, p);
  CQ_LAUNCH((ds_merge<G>), dim3((unsigned)units), dim3(kThreads), 0, st, p);
  return hipSuccess;
}

template <int G, bool F32>
hipError_t launch_g(const SParams& p, int mt, int units, hipStream_t st) {
  if (mt == 1) return launch_mt<G, F32, 1>(p, units, st);
  if (mt == 2) return launch_mt<G, F32, 2>(p, units, st);
  if (mt == 4) return launch_mt<G, F32, 4>(p, units, st);
  return launch_mt<G, F32, 8>(p, units, st);
}

template <bool F32>
hipError_t launch_f(const SParams& p, int G, int mt, int units, hipStream_t st) {
  if (G == 1) return launch_g<1, F32>(p, mt, units, st);
  if (G == 2) return launch_g<2, F32>(p, mt, units, st);
  return launch_g<4, F32>(p, mt, units, st);
}

}  // namespace

namespace cqi {

bool decode_split_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n > 0 && a.n % 32 == 0 &&
         a.T <= kMaxTail && (a.T == 0 || a.tail_dtype == a.q_dtype);
}

// The one-launch kernel runs one workgroup per (batch, kv head); with fewer
// units than a quarter of the CUs most of the device would idle, and the
// chunked launches are faster (measured at n = 8192: 8 units 26 vs 32 us,
// 64 units 36 vs 33 us).
bool decode_split_preferred(const DecodeArgs& a, bool one_ok) {
  return decode_split_supported(a) && (!one_ok || (long)a.B * a.Hkv < 64);
}

size_t decode_split_ws(int B, int Hkv, int n, int T, int requested) {
  if (n <= 0) return 0;
  const Chunking c = chunking(B * Hkv, n, requested);
  return ws_layout(B * Hkv, c.nc, T).total;
}

size_t decode_split_ws_max(int B, int Hkv, int n, int T) {
  if (n <= 0) return 0;
  const int ntiles = (n + kTile - 1) / kTile;
  return ws_layout(B * Hkv, (ntiles + kWaves - 1) / kWaves, T).total;   // one tile per wave
}

hipError_t decode_split(const DecodeArgs& a, int requested) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  const Chunking c = chunking(units, a.n, requested);
  const WsLayout w = ws_layout(units, c.nc, a.T);
  char* ws = static_cast<char*>(a.ws);
  SParams p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
            a.Hq, a.Hkv, a.n, a.T, a.out_dtype == CQ_F32, a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi,
            a.c_hi, c.nc, c.ct, reinterpret_cast<float*>(ws + w.mm), reinterpret_cast<float*>(ws + w.tsc),
            reinterpret_cast<float*>(ws + w.tmx), reinterpret_cast<float*>(ws + w.part), a.nc};
  const int G = a.Hq / a.Hkv;
  return a.q_dtype == CQ_F32 ? launch_f<true>(p, G, c.mt, units, a.stream)
                             : launch_f<false>(p, G, c.mt, units, a.stream);
}

}  // namespace cqi
