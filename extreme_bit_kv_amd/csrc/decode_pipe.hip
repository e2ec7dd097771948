// 1-bit post-scaled, calibrated decode attention with the keys read once and
// the visual scores kept on chip (gfx950).
//
// QbitAI article on CalibQuant, "Method" part 2: with per-channel scale and
// minimum, q . k_hat_i = (q * scale_K) . c_i + q . min_K and
// sum_i p_i v_hat_i = scale_V * sum_i p_i c_i + (sum_i p_i) min_V, so only the
// integer codes enter the products; part 3: the visual scores of each query
// head are mapped by the affine g fixed by their min and max before softmax.
//
// Schedule.  One workgroup of 8 waves per CU walks its (batch, kv head)
// units u_0, u_1, ...; a wave owns the 128-token tiles w, w + 8, ... of every
// unit (TPW tiles at most).  The work is a sequence of segments:
//   segment 0:      key tiles of u_0;
//   segment j:      value tile k of u_{j-1}, key tile k of u_j, for each k;
//   last segment:   value tiles of the last unit,
// separated by one workgroup barrier each, where the finished unit's score
// statistics fix g and the unit before it is written out.  A key tile's
// scores stay in the LDS slot of the wave that made them (TPW slots of
// 4 x 128 floats per wave) until the value tile of the same slot consumes
// them, one segment later, and overwrite them with its probability digits;
// so each key tile is read once and no score travels through HBM.
// The code tiles of every step are requested D steps ahead into a ring of
// registers; the ring runs across segment boundaries, so the memory stream
// does not stop at the barriers.  Inputs of the small per-unit work (query,
// scales, text tail) are requested a segment before they are used, ahead of
// that segment's ring loads: vector loads complete in order, so using them
// never waits for the ring.
//
// Key side: C[16 x 16] = A[16 x 128] B[128 x 16] with the 16x16x128
// f8f6f4 product, A in fp6 (e2m3) and B in fp4 (e2m1).  B is a packed key
// word masked in place, one AND per register: bit s of every 4-bit field
// holds a code; fields whose code sits in bit 0, 1 or 2 read 0.5, 1 or 2
// (bit 3 is shifted down to bit 2 first).  Rows of A are (head, digit
// plane): q * scale_K is the integer Q = round(q' 2^F) split into four
// balanced base-31 digits d in [-15, 15], each stored as d / (4 w) for a code
// of weight w, so every product is exactly d c / 4 and every plane sum is
// exact in float32.  s = ((D0 31 + D1) 31 + D2) 31 + D3 = Q . c / 4.
//
// Value side: as in the one-launch kernel, int8 products of the probability
// digits (four signed base-256 digits of P = round(p 2^27), p relative to the
// largest calibrated visual weight) with the masked value words; the planes
// combine into exact integers.
#include "cq_device.h"
#include "cq_internal.h"
#include "cq_mfma.h"

#include <utility>

namespace {

constexpr int kW = 8;                         // waves per workgroup
constexpr int kTh = kW * 64;
constexpr int kTile = 128;
constexpr int kMaxT = 128;                    // text-tail tokens this schedule takes
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQMax = 15 * (31 * 31 * 31 + 31 * 31 + 31 + 1);   // largest |Q| with four digits

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
using cqm::v4i;
using cqm::bits_hi;
using cqm::bits_lo;
using cqm::bit_weight;
using cqm::lds_barrier;
using cqm::transpose_bytes;
using cqm::wave_sync_lds;

// Read in place of a tile past the end of a unit or of the step sequence, so
// that every ring load is unconditional and costs no HBM traffic.
__device__ __align__(16) uint32_t g_zero[512];

struct PP {
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
  int Hq, Hkv, n, T, units;
  int out_f32;
  float sm;
  int calib_on;
  float a_lo, c_lo, a_hi, c_hi;
};

// fp6 e2m3 code of x / 8 for an integer |x| <= 60 that the format holds
// (|x| < 16, even |x| < 32, or a multiple of 4)
__device__ __forceinline__ uint32_t enc6(int x) {
  const uint32_t a = (uint32_t)(x < 0 ? -x : x);
  uint32_t m;
  if (a < 16) m = a;
  else if (a < 32) m = 16 + ((a - 16) >> 1);
  else m = 24 + ((a - 32) >> 2);
  return m | (x < 0 ? 0x20u : 0u);
}

__device__ __forceinline__ int mods31(int x) { return ((x % 31) + 46) % 31 - 15; }

__device__ __forceinline__ float h2f(uint32_t bits16) { return __half2float(__ushort_as_half((unsigned short)bits16)); }

template <int TPW, bool F32>
__global__ void __launch_bounds__(kTh, 1) dp_b1(PP P) {
  constexpr int D = 2 * TPW < 8 ? 2 * TPW : 8;   // ring depth (steps in flight per wave)
  // text tail per round: key rows as (token, channel group), value rows as
  // (token, channel pair); the same bytes per lane for both dtypes
  constexpr int kCpt = F32 ? 8 : 16;              // key-tail channels per lane
  constexpr int kLpt = 128 / kCpt;                 // lanes per key-tail token
  constexpr int kKtw = 64 / kLpt;                  // key-tail tokens per wave and round
  constexpr int kVtw = F32 ? 4 : 8;                // value-tail tokens per wave and round
  constexpr int kKtr = kW * kKtw, kVtr = kW * kVtw;   // tokens per round
  constexpr int kVRounds = kMaxT / kVtr;

  // Per-lane coordinates are formed from an opaque copy of the thread index
  // that is refreshed at every segment: otherwise the compiler hoists every
  // address and constant derived from them out of the unit loop and spills.
  int tid_v = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#define tid (tid_v)
#define lane (tid_v & 63)
#define i16 (tid_v & 15)
#define g4 ((tid_v >> 4) & 3)
  const int n = P.n, T = P.T, G = P.Hq / P.Hkv;
  const int ntiles = (n + kTile - 1) / kTile, R = n >> 5;
  const int ub = blockIdx.x, us = gridDim.x;
  const int U = (P.units - ub + us - 1) / us;     // units of this workgroup, >= 1
  const int last_step = 2 * TPW * U;              // steps of a wave

  // a wave's key-tile slots: the tile's scores [head][128 tokens] (float32)
  // until its value step, which then writes the tile's probability digits
  // [head][plane][128 tokens] (bytes) in their place: 2 KB either way
  __shared__ __align__(16) uint32_t s_sc[kW][TPW][4][128];
  __shared__ __align__(16) uint32_t s_a6[2][4][4][32];       // fp6 key digits: [par][head][plane][128 bytes]
  __shared__ float s_q[2][4][128];                            // sm * q for the key tail
  __shared__ int s_F[2][4];
  __shared__ double s_c0[2][4];
  __shared__ float s_mm[2][kW][4][2];                         // per-wave min / max of the scores
  __shared__ float s_ts[2][4][kMaxT];                         // key-tail scores
  __shared__ float s_ptw[kW][kVRounds][4][kVtw];              // tail weights of the wave's tail tokens
  __shared__ float s_alpha[2][4];
  __shared__ float s_pt[2][kW][4];                            // per-wave sums of the tail weights
  __shared__ unsigned long long s_vsum[2][4][128];            // 2^3 sum P c, 2^-30 units
  __shared__ unsigned long long s_psum[2][kW][4];             // per-wave sums of P, 2^-27 units
  __shared__ float s_tacc[2][4][128];                         // sum_t p_t vt_t

  const uint32_t* zero = g_zero;
  auto unit_of = [&](int j) { return ub + j * us; };

  // ---- ring loads ---------------------------------------------------------
  // step s of a wave: s < TPW: key tile s of u_0; then per segment j >= 1
  // alternately value tile k of u_{j-1} and key tile k of u_j; the last
  // segment: value tile k of u_{U-1}.
  auto step_src = [&](int s) {
    int kind = 0, j = 0, k = s;
    bool past = s >= last_step;
    if (s >= TPW) {
      const int r = s - TPW;
      j = r / (2 * TPW) + 1;
      const int l = r - (j - 1) * 2 * TPW;
      if (j < U) {
        kind = (l & 1) ? 0 : 1;
        k = l >> 1;
        if (kind) j -= 1;
      } else {
        kind = 1;
        k = l;
        j = U - 1;
      }
    }
    const int t = wave + kW * k;
    past = past || t >= ntiles;
    const int u = unit_of(j);
    // 16 bytes per lane and half, the lanes of a plane or row contiguous:
    // the first half holds tokens (channels) 4 i16 .. +3, the second 64 + 4 i16 ..
    const uint32_t* kb = P.kc + ((size_t)u * 4 + g4) * n;
    const uint32_t* key0 = kb + min(t * kTile + 4 * i16, n - 4);
    const uint32_t* key1 = kb + min(t * kTile + 64 + 4 * i16, n - 4);
    const uint32_t* val0 = P.vc + ((size_t)u * R + min(4 * t + g4, R - 1)) * 128 + 4 * i16;
    const uint32_t* p0 = past ? zero : (kind ? val0 : key0);
    const uint32_t* p1 = past ? zero : (kind ? val0 + 64 : key1);
    return std::make_pair(reinterpret_cast<const uint4*>(p0), reinterpret_cast<const uint4*>(p1));
  };
  uint4 ring[D][2];
  auto load_step = [&](int s, uint4 (&slot)[2]) {
    // the lane's address is formed here, not ahead of the loop for every step
    asm volatile("" : "+v"(tid_v));
    const auto pp = step_src(s);
    slot[0] = *pp.first;
    slot[1] = *pp.second;
  };

  // ---- per-unit inputs (requested a segment early) --------------------------
  // prologue inputs: wave h < G handles head h, lane l channels 2l, 2l + 1
  const int ph = min(wave, G - 1);
  uint32_t pq_raw[2];
  float2 pks, pkm;
  auto load_prologue = [&](int j) {
    const int u = unit_of(min(j, U - 1));
    const int b = u / P.Hkv, h = u % P.Hkv;
    const size_t qi = ((size_t)b * P.Hq + h * G + ph) * 128 + 2 * lane;
    if constexpr (F32) {
      const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(P.q) + qi);
      pq_raw[0] = x.x;
      pq_raw[1] = x.y;
    } else {
      pq_raw[0] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(P.q) + qi);
      pq_raw[1] = 0;
    }
    pks = *reinterpret_cast<const float2*>(P.ks + (size_t)u * 128 + 2 * lane);
    pkm = *reinterpret_cast<const float2*>(P.km + (size_t)u * 128 + 2 * lane);
  };
  // output inputs: thread (head tid / 128, channel tid % 128)
  float ovs, ovm;
  auto load_vsvm = [&](int j) {
    const int u = unit_of(min(j, U - 1));
    ovs = P.vs[(size_t)u * 128 + (tid & 127)];
    ovm = P.vm[(size_t)u * 128 + (tid & 127)];
  };
  // key tail, round r: lane (token kKtw * wave + lane / kLpt, channels kCpt * (lane % kLpt) ..)
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(zero);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(zero);
  uint4 ktr[2];
  auto load_ktail = [&](int j, int r, uint4 (&dst)[2]) {
    const int u = unit_of(min(j, U - 1));
    const int tok = r * kKtr + kKtw * wave + lane / kLpt;
    const size_t e = T > 0 ? ((size_t)u * T + min(tok, T - 1)) * 128 + kCpt * (lane % kLpt) : 0;
    const uint4* p = reinterpret_cast<const uint4*>(ktb + e * (F32 ? 4 : 2));
    dst[0] = p[0];
    dst[1] = p[1];
  };
  // value tail, round r: lane = channel pair, tokens kVtw * wave + i
  uint32_t vtr[kVtw * (F32 ? 2 : 1)];
  auto load_vtail = [&](int j, int r, uint32_t (&dst)[kVtw * (F32 ? 2 : 1)]) {
    const int u = unit_of(min(j, U - 1));
#pragma unroll
    for (int i = 0; i < kVtw; ++i) {
      const int tok = r * kVtr + kVtw * wave + i;
      const size_t e = T > 0 ? ((size_t)u * T + min(tok, T - 1)) * 128 + 2 * lane : 0;
      if constexpr (F32) {
        const uint2 x = *reinterpret_cast<const uint2*>(vtb + e * 4);
        dst[2 * i] = x.x;
        dst[2 * i + 1] = x.y;
      } else {
        dst[i] = *reinterpret_cast<const uint32_t*>(vtb + e * 2);
      }
    }
  };

  // ---- prologue of a unit: key digits, sm * q, c0 and F (waves < G) ------------
  auto prologue = [&](int par) {
    if (wave < G) {
      float qv[2];
      if constexpr (F32) {
        qv[0] = P.sm * __uint_as_float(pq_raw[0]);
        qv[1] = P.sm * __uint_as_float(pq_raw[1]);
      } else {
        qv[0] = P.sm * h2f(pq_raw[0] & 0xFFFFu);
        qv[1] = P.sm * h2f(pq_raw[0] >> 16);
      }
      const float qp0 = qv[0] * pks.x, qp1 = qv[1] * pks.y;
      double c0 = (double)qv[0] * (double)pkm.x + (double)qv[1] * (double)pkm.y;
      float mq = fmaxf(fabsf(qp0), fabsf(qp1));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        c0 += __shfl_xor(c0, off);
        mq = fmaxf(mq, __shfl_xor(mq, off));
      }
      int F = 0;
      if (mq > 0.f) {
        const int e = ilogbf(mq);
        F = ldexpf(mq, 18 - e) > (float)kQMax ? 17 - e : 18 - e;
      }
      s_q[par][wave][2 * lane] = qv[0];
      s_q[par][wave][2 * lane + 1] = qv[1];
      if (lane == 0) {
        s_F[par][wave] = F;
        s_c0[par][wave] = c0;
      }
      unsigned char* a6 = reinterpret_cast<unsigned char*>(&s_a6[par][wave][0][0]);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = 2 * lane + c2;
        int x = (int)rintf(ldexpf(c2 ? qp1 : qp0, F));       // |x| <= kQMax
        int d[4];
#pragma unroll
        for (int k = 3; k >= 0; --k) {
          d[k] = mods31(x);
          x = (x - d[k]) / 31;
        }
        // channel c sits at position kk = 8 R + N of its 32-channel group,
        // R = (e / 4) mod 4, N = 2 (e mod 4) + e / 16 for e = c mod 32; its
        // code reads 0.5, 1, 2, 2 for R = 0..3
        const int e = c & 31, R = (e >> 2) & 3, kk = 8 * R + 2 * (e & 3) + (e >> 4);
        const int mult = R == 0 ? 4 : (R == 1 ? 2 : 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) a6[k * 128 + 32 * (c >> 5) + kk] = (unsigned char)enc6(d[k] * mult);
      }
    }
  };
  // key A operand of this lane: row (head i16 / 4, plane i16 % 4), group g4
  v8i kdig;
  auto pack_digits = [&](int par) {
    const uint4* src = reinterpret_cast<const uint4*>(&s_a6[par][i16 >> 2][i16 & 3][8 * g4]);
    const uint4 x0 = src[0], x1 = src[1];
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t o[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = (w[i >> 2] >> (8 * (i & 3))) & 0x3Fu;
      const int bit = 6 * i, wd = bit >> 5, off = bit & 31;
      o[wd] |= c << off;
      if (off > 26) o[wd + 1] |= c >> (32 - off);
    }
    kdig = v8i{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], 0, 0};
  };

  // ---- state --------------------------------------------------------------
  float vmin = INFINITY, vmax = -INFINITY;
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  unsigned long long psum = 0;
  float lamS = 0.f, muS = -INFINITY;             // value side of the unit before: head g4

  auto key_step = [&](int k, const uint4 (&slot)[2]) {
    const int t = wave + kW * k;
    if (t >= ntiles) return;
    // tokens of this lane: 4 i16 + m (m < 4) and 64 + 4 i16 + m - 4 (m >= 4)
    const bool ok0 = t * kTile + 4 * i16 < n, ok1 = t * kTile + 64 + 4 * i16 < n;
    const uint32_t wd[8] = {slot[0].x, slot[0].y, slot[0].z, slot[0].w, slot[1].x, slot[1].y, slot[1].z, slot[1].w};
    float tmin0 = INFINITY, tmax0 = -INFINITY, tmin1 = INFINITY, tmax1 = -INFINITY, st[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t w = wd[m];
      const v8i b{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u),
                  (int)((w >> 1) & 0x44444444u), 0, 0, 0, 0};
      const v4f a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kdig, b, v4f{0.f, 0.f, 0.f, 0.f}, 2, 4, 0,
                                                                      127, 0, 127);
      const float s = fmaf(fmaf(fmaf(a[0], 31.f, a[1]), 31.f, a[2]), 31.f, a[3]);
      st[m] = s;
      if (m < 4) {
        tmin0 = fminf(tmin0, s);
        tmax0 = fmaxf(tmax0, s);
      } else {
        tmin1 = fminf(tmin1, s);
        tmax1 = fmaxf(tmax1, s);
      }
    }
    *reinterpret_cast<float4*>(&s_sc[wave][k][g4][4 * i16]) = make_float4(st[0], st[1], st[2], st[3]);
    *reinterpret_cast<float4*>(&s_sc[wave][k][g4][64 + 4 * i16]) = make_float4(st[4], st[5], st[6], st[7]);
    if (ok0) {
      vmin = fminf(vmin, tmin0);
      vmax = fmaxf(vmax, tmax0);
    }
    if (ok1) {
      vmin = fminf(vmin, tmin1);
      vmax = fmaxf(vmax, tmax1);
    }
  };

  auto value_step = [&](int k, const uint4 (&slot)[2]) {
    const int t = wave + kW * k;
    if (t >= ntiles) return;
    const bool ok0 = g4 < G && t * kTile + 4 * i16 < n, ok1 = g4 < G && t * kTile + 64 + 4 * i16 < n;
    const float mu0 = ok0 ? muS : -INFINITY, mu1 = ok1 ? muS : -INFINITY;
    uint32_t* slot_lds = &s_sc[wave][k][0][0];
    float st[8];
    {
      const float4 a = *reinterpret_cast<const float4*>(slot_lds + g4 * 128 + 4 * i16);
      const float4 c = *reinterpret_cast<const float4*>(slot_lds + g4 * 128 + 64 + 4 * i16);
      st[0] = a.x; st[1] = a.y; st[2] = a.z; st[3] = a.w;
      st[4] = c.x; st[5] = c.y; st[6] = c.z; st[7] = c.w;
    }
    uint32_t fb[8], ptile = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st[m], lamS, m < 4 ? mu0 : mu1));
      const uint32_t Pm = cqm::p_fixed(p);
      ptile += Pm;
      fb[m] = cqm::sdigits(Pm << bit_weight(4 * i16));    // the same weight for all eight tokens
    }
    psum += ptile;
    wave_sync_lds();                               // every lane has read its scores of the slot
    unsigned char* pd = reinterpret_cast<unsigned char*>(slot_lds);
    uint32_t dg[2][4];
    transpose_bytes(fb[0], fb[1], fb[2], fb[3], dg[0][0], dg[0][1], dg[0][2], dg[0][3]);
    transpose_bytes(fb[4], fb[5], fb[6], fb[7], dg[1][0], dg[1][1], dg[1][2], dg[1][3]);
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) {
      *reinterpret_cast<uint32_t*>(pd + (g4 * 4 + pl) * 128 + 4 * i16) = dg[0][pl];
      *reinterpret_cast<uint32_t*>(pd + (g4 * 4 + pl) * 128 + 64 + 4 * i16) = dg[1][pl];
    }
    wave_sync_lds();
    const uint4 x0 = *reinterpret_cast<const uint4*>(pd + i16 * 128 + 32 * g4);
    const uint4 x1 = *reinterpret_cast<const uint4*>(pd + i16 * 128 + 32 * g4 + 16);
    const v4i av0{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w}, av1{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    const uint32_t vw[8] = {slot[0].x, slot[0].y, slot[0].z, slot[0].w, slot[1].x, slot[1].y, slot[1].z, slot[1].w};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      vacc[ct] = cqm::mfma(av0, bits_lo(vw[ct]), vacc[ct]);
      vacc[ct] = cqm::mfma(av1, bits_hi(vw[ct]), vacc[ct]);
    }
  };

  // ---- segment ends --------------------------------------------------------
  // keys of the unit just scored: min / max per head, key-tail scores
  auto finish_keys = [&](int j) {
    const int par = j & 1;
    float a = vmin, b = vmax;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      a = fminf(a, __shfl_xor(a, off));
      b = fmaxf(b, __shfl_xor(b, off));
    }
    if (i16 == 0) {
      s_mm[par][wave][g4][0] = a;
      s_mm[par][wave][g4][1] = b;
    }
    vmin = INFINITY;
    vmax = -INFINITY;
    for (int r = 0; r * kKtr < T; ++r) {
      uint4 kx[2];
      if (r == 0) {
        kx[0] = ktr[0];
        kx[1] = ktr[1];
      } else {
        load_ktail(j, r, kx);
      }
      float kf[kCpt];
      if constexpr (F32) {
        const uint32_t w[8] = {kx[0].x, kx[0].y, kx[0].z, kx[0].w, kx[1].x, kx[1].y, kx[1].z, kx[1].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) kf[c] = __uint_as_float(w[c]);
      } else {
        const uint32_t w[8] = {kx[0].x, kx[0].y, kx[0].z, kx[0].w, kx[1].x, kx[1].y, kx[1].z, kx[1].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          kf[2 * c] = h2f(w[c] & 0xFFFFu);
          kf[2 * c + 1] = h2f(w[c] >> 16);
        }
      }
      const int tok = r * kKtr + kKtw * wave + lane / kLpt, c0 = kCpt * (lane % kLpt);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < G) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < kCpt; c += 4) {
            const float4 qq = *reinterpret_cast<const float4*>(&s_q[par][h][c0 + c]);
            s = fmaf(qq.x, kf[c], s);
            s = fmaf(qq.y, kf[c + 1], s);
            s = fmaf(qq.z, kf[c + 2], s);
            s = fmaf(qq.w, kf[c + 3], s);
          }
#pragma unroll
          for (int off = 1; off < kLpt; off <<= 1) s += __shfl_xor(s, off);
          if (lane % kLpt == 0 && tok < T) s_ts[par][h][tok] = s;
        }
      }
    }
  };
  // values of the unit before: exact sums into LDS, value-tail sums
  auto finish_values = [&](int j) {
    const int par = j & 1;
    if (g4 < G) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const long long sv = (long long)vacc[ct][0] + 256ll * vacc[ct][1] + 65536ll * vacc[ct][2] +
                             16777216ll * vacc[ct][3];
        atomicAdd(&s_vsum[par][g4][ct < 4 ? 4 * i16 + ct : 60 + 4 * i16 + ct], (unsigned long long)sv);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
    unsigned long long ps = psum;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
    if (i16 == 0) s_psum[par][wave][g4] = ps;
    psum = 0;
    for (int r = 0; r * kVtr < T; ++r) {
      uint32_t vx[kVtw * (F32 ? 2 : 1)];
      if (r == 0) {
#pragma unroll
        for (int i = 0; i < kVtw * (F32 ? 2 : 1); ++i) vx[i] = vtr[i];
      } else {
        load_vtail(j, r, vx);
      }
      float acc[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < kVtw; ++i) {
        float v0, v1;
        if constexpr (F32) {
          v0 = __uint_as_float(vx[2 * i]);
          v1 = __uint_as_float(vx[2 * i + 1]);
        } else {
          v0 = h2f(vx[i] & 0xFFFFu);
          v1 = h2f(vx[i] >> 16);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float p = s_ptw[wave][r][h][i];        // 0 past the tail and for heads >= G
          acc[h][0] = fmaf(p, v0, acc[h][0]);
          acc[h][1] = fmaf(p, v1, acc[h][1]);
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < G) {
          atomicAdd(&s_tacc[par][h][2 * lane], acc[h][0]);
          atomicAdd(&s_tacc[par][h][2 * lane + 1], acc[h][1]);
        }
      }
    }
  };
  // after the barrier: g and the softmax reference of the unit just scored
  // (every lane, head g4), and the weights of the wave's tail tokens
  auto stats = [&](int j) {
    const int par = j & 1;
    float m = i16 < kW ? s_mm[par][i16][g4][0] : INFINITY;
    float M = i16 < kW ? s_mm[par][i16][g4][1] : -INFINITY;
    float tm = -INFINITY;
    for (int t = i16; t < T; t += 16) tm = fmaxf(tm, s_ts[par][g4 < G ? g4 : 0][t]);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      m = fminf(m, __shfl_xor(m, off));
      M = fmaxf(M, __shfl_xor(M, off));
      tm = fmaxf(tm, __shfl_xor(tm, off));
    }
    const int hh = g4 < G ? g4 : 0;
    const double scale = ldexp(4.0, -s_F[par][hh]);           // real score per unit of s
    const double c0 = s_c0[par][hh];
    double vis_max, lam, mu;                                   // exponent = lam s + mu (natural log)
    if (P.calib_on) {
      const double mr = (double)m * scale + c0, Mr = (double)M * scale + c0;
      const double t_lo = (double)P.a_lo * mr + (double)P.c_lo, t_hi = (double)P.a_hi * Mr + (double)P.c_hi;
      // g's largest value: the larger end, or t_lo when every score is the same
      vis_max = M > m ? fmax(t_lo, t_hi) : t_lo;
      const double l = M > m ? (t_hi - t_lo) / ((double)(M - m) * scale) : 0.0;
      lam = l * scale;
      mu = t_lo - vis_max - lam * (double)m;
    } else {
      vis_max = (double)M * scale + c0;
      lam = scale;
      mu = -lam * (double)M;
    }
    lamS = (float)(lam * 1.4426950408889634);
    muS = (float)(mu * 1.4426950408889634);
    const float top = fmaxf((float)vis_max, tm);
    const float alpha = exp2f(((float)vis_max - top) * kLog2e);
    if (wave == 0 && i16 == 0 && g4 < G) s_alpha[par][g4] = alpha;
    // tail weights of this wave's value-tail tokens: lane (head lane / 16,
    // token lane % 16 of the wave's rounds)
    const int th = lane >> 4;
    const float top_h = __shfl(top, 16 * min(th, G - 1));
    float pts = 0.f;
    for (int r = 0; r * kVtr < T; ++r) {
      for (int i = i16; i < kVtw; i += 16) {
        const int tok = r * kVtr + kVtw * wave + i;
        float p = 0.f;
        if (th < G && tok < T) p = exp2f((s_ts[par][th][tok] - top_h) * kLog2e);
        s_ptw[wave][r][th][i] = p;
        pts += p;
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) pts += __shfl_xor(pts, off);
    if (i16 == 0) s_pt[par][wave][th] = pts;
  };
  // after the barrier: the unit before is written out and its sums cleared
  auto output = [&](int j) {
    const int par = j & 1;
    if (tid < G * 128) {
      const int h = tid >> 7, c = tid & 127;
      const int u = unit_of(j);
      const int b = u / P.Hkv, hk = u % P.Hkv;
      unsigned long long psm = 0;
      float pt = 0.f;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        psm += s_psum[par][w][h];
        pt += s_pt[par][w][h];
      }
      const float sv = (float)((double)(long long)s_vsum[par][h][c] * (1.0 / 1073741824.0));   // 2^-30
      const float pv = (float)((double)psm * (1.0 / 134217728.0));                             // 2^-27
      const float al = s_alpha[par][h];
      float o = s_tacc[par][h][c] + al * (ovs * sv + pv * ovm);
      o /= al * pv + pt;
      const size_t oi = ((size_t)b * P.Hq + hk * G + h) * 128 + c;
      if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
      else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
      s_vsum[par][h][c] = 0ull;
      s_tacc[par][h][c] = 0.f;
    }
  };

  // ---- run ------------------------------------------------------------------
  for (int i = tid; i < 2 * 4 * 128; i += kTh) {
    (&s_vsum[0][0][0])[i] = 0ull;
    (&s_tacc[0][0][0])[i] = 0.f;
  }
  for (int i = tid; i < 2 * 4 * 4 * 32; i += kTh) (&s_a6[0][0][0][0])[i] = 0u;
  // requested in this order: the first unit's prologue inputs, the ring, the
  // second unit's prologue inputs and the first unit's key tail
  load_prologue(0);
#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, ring[d]);
  int s = D;                                       // next step to request
  lds_barrier();                                   // the LDS is cleared
  prologue(0);
  load_prologue(1);
  load_ktail(0, 0, ktr);
  lds_barrier();
  pack_digits(0);

  // segment 0: key tiles of u_0
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    key_step(k, ring[k % D]);
    load_step(s++, ring[k % D]);
    __builtin_amdgcn_sched_barrier(0);
  }
  finish_keys(0);
  if (U > 1) prologue(1);
  lds_barrier();
  if (U > 1) pack_digits(1);
  stats(0);
  load_prologue(2);
  load_vsvm(0);
  load_ktail(1, 0, ktr);
  load_vtail(0, 0, vtr);

  for (int j = 1; j < U; ++j) {
    asm volatile("" : "+v"(tid_v));
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      value_step(k, ring[(TPW + 2 * k) % D]);
      load_step(s++, ring[(TPW + 2 * k) % D]);
      __builtin_amdgcn_sched_barrier(0);          // steps are scheduled one by one
      key_step(k, ring[(TPW + 2 * k + 1) % D]);
      load_step(s++, ring[(TPW + 2 * k + 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
    }
    finish_keys(j);
    finish_values(j - 1);
    if (j + 1 < U) prologue((j + 1) & 1);
    lds_barrier();
    if (j + 1 < U) pack_digits((j + 1) & 1);
    output(j - 1);
    stats(j);
    load_prologue(j + 2);
    load_vsvm(j);
    load_ktail(j + 1, 0, ktr);
    load_vtail(j, 0, vtr);
  }

  // last segment: value tiles of u_{U-1}
  asm volatile("" : "+v"(tid_v));
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    value_step(k, ring[(TPW + k) % D]);
    __builtin_amdgcn_sched_barrier(0);
  }
  finish_values(U - 1);
  lds_barrier();
  output(U - 1);
}

#undef tid
#undef lane
#undef i16
#undef g4

template <bool F32>
hipError_t launch(const PP& p, int tpw, int grid, hipStream_t st) {
  switch (tpw) {
    case 1: CQ_LAUNCH((dp_b1<1, F32>), dim3(grid), dim3(kTh), 0, st, p); break;
    case 2: CQ_LAUNCH((dp_b1<2, F32>), dim3(grid), dim3(kTh), 0, st, p); break;
    case 4: CQ_LAUNCH((dp_b1<4, F32>), dim3(grid), dim3(kTh), 0, st, p); break;
    default: CQ_LAUNCH((dp_b1<8, F32>), dim3(grid), dim3(kTh), 0, st, p); break;
  }
  return hipSuccess;
}

int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = cus;
  }
  return cache[dev];
}

int tiles_per_wave(int n) {
  const int per = ((n + kTile - 1) / kTile + kW - 1) / kW;
  return per <= 1 ? 1 : (per <= 2 ? 2 : (per <= 4 ? 4 : 8));
}

}  // namespace

namespace cqi {

// b = 1, d = 128, G in {1, 2, 4}, 32 <= n <= 8192, n % 32 == 0, T <= 256,
// q and tails in one dtype
bool decode_pipe_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n >= 32 && a.n <= kW * 8 * kTile &&
         a.n % 32 == 0 && a.T <= kMaxT && (a.T == 0 || a.tail_dtype == a.q_dtype) && (long)a.B * a.Hkv >= 1;
}

hipError_t decode_pipe(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  const int cus = cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  PP p{};
  p.q = a.q;
  p.kc = a.k_codes;
  p.ks = a.k_scale;
  p.km = a.k_min;
  p.vc = a.v_codes;
  p.vs = a.v_scale;
  p.vm = a.v_min;
  p.kt = a.k_tail;
  p.vt = a.v_tail;
  p.out = a.out;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.n = a.n;
  p.T = a.T;
  p.units = units;
  p.out_f32 = a.out_dtype == CQ_F32;
  p.sm = a.sm_scale;
  p.calib_on = a.calib_on;
  p.a_lo = a.a_lo;
  p.c_lo = a.c_lo;
  p.a_hi = a.a_hi;
  p.c_hi = a.c_hi;
  const int grid = units < cus ? units : cus;
  const int tpw = tiles_per_wave(a.n);
  return a.q_dtype == CQ_F32 ? launch<true>(p, tpw, grid, a.stream) : launch<false>(p, tpw, grid, a.stream);
}

}  // namespace cqi
