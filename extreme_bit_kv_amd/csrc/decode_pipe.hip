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
// units u_0, u_1, ...; wave w owns the 128-token tiles w, w + 8, ... of every
// unit (TPW <= 8 tiles).  The work is a sequence of segments:
//   segment 0:      key tiles of u_0;
//   segment j:      value tile k of u_{j-1}, then key tile k of u_j, for each k;
//   last segment:   value tiles of the last unit,
// separated by one workgroup barrier each.  Only what fixes g waits there:
// every wave's min / max of the unit just scored, then g itself.  The rest of
// a unit's work runs as side tasks between the steps of the next segments:
// its key-tail scores (while its keys are scored), its value tail (while its
// values are summed; the tail is weighed against its own largest score and
// the two parts are combined at the output), the digits of the next unit's
// query (one segment ahead) and its output (one segment after its values).  A key tile's
// scores wait in the wave's LDS slot (4 x 128 floats) for the value tile of
// the same slot, one segment later, which overwrites them with its
// probability digits: each key tile is read once and no score goes to HBM.
// Every wave keeps two steps of code tiles in flight; the stream runs across
// segment ends.  Tiles are read with buffer loads: a descriptor per unit and
// tensor, a fixed byte offset per lane, so a step costs one address add per
// load, and a row past the unit's codes reads as zero without any traffic.
//
// Key side: C[16 x 16] = A[16 x 128] B[128 x 16] with the 16x16x128 f8f6f4
// product, A in fp8 (e4m3) and B in fp4 (e2m1) (the two formats spread k
// over a lane's values differently; the digits are read to match).  B is a packed key word
// masked in place, one operation per register: fields whose code sits in
// bit 0, 1 or 2 read 0.5 c, c or 2 c; the bit-3 fields are forced to
// +-1 (1 - 2 c), and the constant part of their products is added back to
// the head's score offset.  Rows of A are (head, digit plane): q * scale_K is
// the integer Q = round(q' 2^F) split into four balanced base-31 digits
// d in [-15, 15], each stored as d / 2, d / 4, d / 8 or -d / 8 for the four
// field kinds, so every product is exactly d c / 4 (up to that constant) and
// every plane sum is exact in float32.  s = ((D0 31 + D1) 31 + D2) 31 + D3.
//
// Value side: as in the one-launch kernel, int8 products of the probability
// digits (four signed base-256 digits of P = round(p 2^27), p relative to the
// largest calibrated visual weight) with the masked value words; the planes
// combine into exact integers.
#include "cq_device.h"
#include "cq_internal.h"
#include "cq_mfma.h"

namespace {

constexpr int kTile = 128;
constexpr int kMaxTiles = 64;                 // tiles per unit: n <= 8192
constexpr int kMaxT = 128;                    // text-tail tokens this schedule takes
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQMax = 15 * (31 * 31 * 31 + 31 * 31 + 31 + 1);   // largest |Q| with four digits
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
using cqm::v4i;
using cqm::bits_hi;
using cqm::bits_lo;
using cqm::bit_weight;
using cqm::lds_barrier;
using cqm::transpose_bytes;
using cqm::wave_sync_lds;

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
  int nc;               // token capacity of the code buffers (their layout is that of nc >= n tokens)
  int out_f32;
  float sm;
  int calib_on;
  float a_lo, c_lo, a_hi, c_hi;
};

__device__ __forceinline__ float h2f(uint32_t bits16) { return __half2float(__ushort_as_half((unsigned short)bits16)); }

// min / max of three floats in one instruction (the operands are finite or
// +-infinity, never NaN, so no quieting is needed)
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint4 ld_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(x.x, x.y, x.z, x.w);
}

// FULL: n = KW TPW 128, so every wave owns TPW whole tiles of every unit
template <int KW, int TPW, bool F32, bool FULL>
__global__ void __launch_bounds__(KW * 64, 1) dp_b1(PP P) {
  constexpr int kW = KW;                         // waves per workgroup
  constexpr int kTh = kW * 64;
  // text tail: key rows as (token, channel chunk of kKl 16-byte pieces),
  // value rows as (token, channel pair), 64 tokens per round; round 0 of each
  // is requested ahead
  constexpr int kKl = 16 / kW;                   // 16-byte key-tail pieces per thread
  constexpr int kCpt = (F32 ? 4 : 8) * kKl;      // key-tail channels per thread
  constexpr int kLpt = 128 / kCpt;               // threads per key-tail token
  constexpr int kKtr = kTh / kLpt;               // key-tail tokens per round
  constexpr int kVtw = 64 / kW;                  // value-tail tokens per wave and round
  constexpr int kVtr = kW * kVtw;                // value-tail tokens per round

  // Per-lane coordinates are formed from an opaque copy of the thread index
  // that is refreshed at every segment: otherwise the compiler keeps every
  // value derived from them alive across the unit loop.
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

  // a wave's key-tile slots: the tile's scores [head][128 tokens] (float32)
  // until its value step, which writes the tile's probability digits
  // [head][plane][128 tokens] (bytes) in their place: 2 KB either way
  __shared__ __align__(16) uint32_t s_sc[kW][TPW][4][128];
  __shared__ __align__(16) unsigned char s_a8[2][4][4][128];   // fp8 key digits [par][head][plane][k slot]
  __shared__ __align__(16) float s_q[2][4][128];               // sm * q, for the key tail
  __shared__ int s_F[3][4];
  __shared__ double s_c0[3][4];                                 // q . min_K plus the bit-3 constant
  __shared__ float s_mm[2][kW][4][2];                           // per-wave min / max of the scores
  __shared__ float s_ts[2][4][kMaxT];                           // key-tail scores
  __shared__ float s_pw[kW][4][kMaxT / kW];                     // tail weights of the wave's tail tokens
  __shared__ float s_vmax[2][4];                                // largest calibrated visual exponent per head
  __shared__ float s_tm[2][4];                                  // largest tail score per head
  __shared__ float s_pt[2][kW][4];                              // per-wave sums of the tail weights
  __shared__ unsigned long long s_vsum[2][4][128];              // 2^3 sum P c, 2^-30 units
  __shared__ unsigned long long s_psum[2][kW][4];               // per-wave sums of P, 2^-27 units
  __shared__ float s_tacc[2][4][128];                           // sum_t p_t vt_t

  auto unit_of = [&](int j) { return ub + j * us; };

  // ---- ring loads -----------------------------------------------------------
  // Byte offsets of this lane's two 16-byte pieces inside a tile (fixed), and
  // of tile t inside a unit's codes.  Keys [4 word rows][n tokens]: the lane
  // reads tokens 4 i16 .. +3 and 64 + 4 i16 .. +3 of word row g4.  Values
  // [n / 32 rows][128 channels]: row 4 t + g4, channels 4 i16 .. +3 and 64 + ...
  const uint32_t koff = (uint32_t)(g4 * P.nc + 4 * i16) * 4u;
  const uint32_t voff = (uint32_t)(g4 * 128 + 4 * i16) * 4u;
  const uint32_t kbytes = (uint32_t)P.nc * 16u, vbytes = (uint32_t)(P.nc >> 5) * 512u;   // per unit
  // key tile k / value tile k of unit j (wave-uniform).  One descriptor per
  // code tensor (each at most 2 GB); the tile's byte offset (unit and tile:
  // wave-uniform) joins the lane's; a tile past the unit or a unit past the
  // workgroup's last gets bit 31 set, out of range: zeros, no traffic.
  const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)P.kc, (short)0, (int)((uint32_t)P.units * kbytes),
                                                    kRsrcFlags);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)P.vc, (short)0, (int)((uint32_t)P.units * vbytes),
                                                    kRsrcFlags);
  auto load_key = [&](int j, int k, uint4 (&slot)[2]) {
    const int t = wave + kW * k;
    const bool past = t >= ntiles || j >= U;
    const uint32_t u = (uint32_t)unit_of(j < U ? j : U - 1);
    const uint32_t off = koff + (past ? 0x80000000u : u * kbytes + (uint32_t)t * 512u);
    slot[0] = ld_buf(rk, off);
    slot[1] = ld_buf(rk, off + 256u);
  };
  auto load_val = [&](int j, int k, uint4 (&slot)[2]) {
    const int t = wave + kW * k;
    const bool past = t >= ntiles || j >= U;
    const uint32_t u = (uint32_t)unit_of(j < U ? j : U - 1);
    const uint32_t off = voff + (past ? 0x80000000u : u * vbytes + (uint32_t)t * 2048u);
    slot[0] = ld_buf(rv, off);
    slot[1] = ld_buf(rv, off + 256u);
  };
  uint4 ring[2][2];

  // ---- per-unit inputs --------------------------------------------------------
  // prologue inputs: wave h < G handles head h, lane l channels 2l, 2l + 1
  const int ph = min(wave, G - 1);
  uint32_t pq_raw[2];
  float2 pks, pkm;
  // Side inputs are requested with unconditional loads at clamped, always
  // valid addresses (their values are simply not used when there is nothing
  // to read), so that the waits for them stay exact.
  constexpr size_t kElt = F32 ? 4 : 2;            // bytes per q / tail element
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
  float ovs = 0.f, ovm = 0.f;
  auto load_vsvm = [&](int j) {
    const int u = unit_of(max(0, min(j, U - 1)));
    ovs = P.vs[(size_t)u * 128 + (tid & 127)];
    ovm = P.vm[(size_t)u * 128 + (tid & 127)];
  };
  // tails: without a text tail the loads read q instead (at least 256 bytes)
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(P.q);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(P.q);
  auto tail_elem = [&](int j, int tok, int c) -> size_t {
    if (T == 0) return 0;
    const int u = unit_of(max(0, min(j, U - 1)));
    return ((size_t)u * T + min(tok, T - 1)) * 128 + c;
  };
  // key tail, round r: thread (token r kKtr + tid / kLpt, channels kCpt (tid % kLpt) ..)
  auto load_ktail = [&](int j, int r, uint4 (&dst)[kKl]) {
    const size_t e = tail_elem(j, r * kKtr + tid / kLpt, kCpt * (tid % kLpt));
#pragma unroll
    for (int i = 0; i < kKl; ++i) dst[i] = reinterpret_cast<const uint4*>(ktb + e * kElt)[i];
  };
  // value tail, round r: lane = channel pair, tokens r kVtr + wave + kW i
  auto load_vtail = [&](int j, int r, uint32_t (&dst)[kVtw * (F32 ? 2 : 1)]) {
#pragma unroll
    for (int i = 0; i < kVtw; ++i) {
      const size_t e = tail_elem(j, r * kVtr + wave + kW * i, 2 * lane);
      if constexpr (F32) {
        const uint2 x = *reinterpret_cast<const uint2*>(vtb + e * 4);
        dst[2 * i] = x.x;
        dst[2 * i + 1] = x.y;
      } else {
        dst[i] = *reinterpret_cast<const uint32_t*>(vtb + e * 2);
      }
    }
  };

  // ---- prologue of unit j: key digits, sm * q, c0 and F (waves < G) ------------
  auto prologue = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int par = j & 1, tri = j % 3;
    if (wave < G) {
      float qv[2];
      if constexpr (F32) {
        qv[0] = P.sm * __uint_as_float(pq_raw[0]);
        qv[1] = P.sm * __uint_as_float(pq_raw[1]);
      } else {
        qv[0] = P.sm * h2f(pq_raw[0] & 0xFFFFu);
        qv[1] = P.sm * h2f(pq_raw[0] >> 16);
      }
      const float qp[2] = {qv[0] * pks.x, qv[1] * pks.y};
      double c0 = (double)qv[0] * (double)pkm.x + (double)qv[1] * (double)pkm.y;
      float mq = fmaxf(fabsf(qp[0]), fabsf(qp[1]));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mq = fmaxf(mq, __shfl_xor(mq, off));
      int F = 0;
      if (mq > 0.f) {
        const int e = ilogbf(mq);
        F = ldexpf(mq, 18 - e) > (float)kQMax ? 17 - e : 18 - e;
      }
      // channel c sits in k slot 32 (c / 32) + 8 R + 2 (e mod 4) + e / 16 of
      // its rows, e = c mod 32, R = (e / 4) mod 4 (the fp4 field that holds
      // its key bit); its digit is stored times 1/2, 1/4, 1/8 or -1/8
      float kconst = 0.f;                          // sum of Q / 8 over the bit-3 channels
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = 2 * lane + c2;
        const float x = rintf(ldexpf(qp[c2], F));  // |x| <= kQMax, exact
        float d[4], r = x;
#pragma unroll
        for (int k = 3; k > 0; --k) {
          const float qk = rintf(r * (1.f / 31.f));   // exact: r / 31 is never near a half
          d[k] = fmaf(-31.f, qk, r);
          r = qk;
        }
        d[0] = r;
        const int e = c & 31, Rf = (e >> 2) & 3, slot = 32 * (c >> 5) + 8 * Rf + 2 * (e & 3) + (e >> 4);
        const float mult = Rf == 0 ? 0.5f : (Rf == 1 ? 0.25f : (Rf == 2 ? 0.125f : -0.125f));
        if (Rf == 3) kconst += 0.125f * x;
        uint32_t b4 = __builtin_amdgcn_cvt_pk_fp8_f32(d[0] * mult, d[1] * mult, 0, false);
        b4 = __builtin_amdgcn_cvt_pk_fp8_f32(d[2] * mult, d[3] * mult, b4, true);
#pragma unroll
        for (int k = 0; k < 4; ++k) s_a8[par][wave][k][slot] = (unsigned char)(b4 >> (8 * k));
      }
      double kc = (double)kconst;                  // multiples of 1 / 8 below 2^24: exact
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        c0 += __shfl_xor(c0, off);
        kc += __shfl_xor(kc, off);
      }
      s_q[par][wave][2 * lane] = qv[0];
      s_q[par][wave][2 * lane + 1] = qv[1];
      if (lane == 0) {
        s_F[tri][wave] = F;
        s_c0[tri][wave] = c0 + kc * ldexp(4.0, -F);
      }
    }
  };
  // key A operand of this lane: row (head i16 / 4, plane i16 % 4).  In fp8
  // the lane's bytes 0..15 meet k = 16 g4 .. +15 and bytes 16..31 meet
  // k = 64 + 16 g4 .. +15, while an fp4 lane's 32 fields meet 32 g4 .. +31, so
  // the digits are kept in fp4 order (k slot) and read as those two pieces.
  v8i kdig;
  auto read_digits = [&](int par) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const unsigned char* row = &s_a8[par][i16 >> 2][i16 & 3][0];
    const uint4 x0 = *reinterpret_cast<const uint4*>(row + 16 * g4);
    const uint4 x1 = *reinterpret_cast<const uint4*>(row + 64 + 16 * g4);
    kdig = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  };

  // ---- state --------------------------------------------------------------
  float vmin = INFINITY, vmax = -INFINITY;
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  unsigned long long psum = 0;
  float lamS = 0.f, muS = -INFINITY;             // value side of the unit before: head g4

  auto key_step = [&](int k, const uint4 (&slot)[2]) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int t = wave + kW * k;
    if (!FULL && t >= ntiles) return;
    const uint32_t wd[8] = {slot[0].x, slot[0].y, slot[0].z, slot[0].w, slot[1].x, slot[1].y, slot[1].z, slot[1].w};
    float st[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t w = wd[m];
      const v8i b{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u),
                  (int)((w & 0x88888888u) | 0x22222222u), 0, 0, 0, 0};
      const v4f a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kdig, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 4, 0,
                                                                      127, 0, 127);
      st[m] = fmaf(fmaf(fmaf(a[0], 31.f, a[1]), 31.f, a[2]), 31.f, a[3]);
      if (m == 3) __builtin_amdgcn_sched_barrier(0);   // four products in flight at most
    }
    // tokens of this lane: 4 i16 + m (m < 4) and 64 + 4 i16 + m - 4 (m >= 4)
    *reinterpret_cast<float4*>(&s_sc[wave][k][g4][4 * i16]) = make_float4(st[0], st[1], st[2], st[3]);
    *reinterpret_cast<float4*>(&s_sc[wave][k][g4][64 + 4 * i16]) = make_float4(st[4], st[5], st[6], st[7]);
    if (FULL || (t + 1) * kTile <= n) {
      vmin = min3f(min3f(vmin, st[0], st[1]), min3f(st[2], st[3], st[4]), min3f(st[5], st[6], st[7]));
      vmax = max3f(max3f(vmax, st[0], st[1]), max3f(st[2], st[3], st[4]), max3f(st[5], st[6], st[7]));
    } else {                                       // the ragged last tile (n is a multiple of 32)
      if (t * kTile + 4 * i16 < n) {
        vmin = min3f(vmin, min3f(st[0], st[1], st[2]), st[3]);
        vmax = max3f(vmax, max3f(st[0], st[1], st[2]), st[3]);
      }
      if (t * kTile + 64 + 4 * i16 < n) {
        vmin = min3f(vmin, min3f(st[4], st[5], st[6]), st[7]);
        vmax = max3f(vmax, max3f(st[4], st[5], st[6]), st[7]);
      }
    }
  };

  auto value_step = [&](int k, const uint4 (&slot)[2]) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int t = wave + kW * k;
    if (!FULL && t >= ntiles) return;
    float mu0 = muS, mu1 = muS;
    if (!FULL && (t + 1) * kTile > n) {
      mu0 = t * kTile + 4 * i16 < n ? muS : -INFINITY;
      mu1 = t * kTile + 64 + 4 * i16 < n ? muS : -INFINITY;
    }
    uint32_t* slot_lds = &s_sc[wave][k][0][0];
    float st[8];
    {
      const float4 a = *reinterpret_cast<const float4*>(slot_lds + g4 * 128 + 4 * i16);
      const float4 c = *reinterpret_cast<const float4*>(slot_lds + g4 * 128 + 64 + 4 * i16);
      st[0] = a.x; st[1] = a.y; st[2] = a.z; st[3] = a.w;
      st[4] = c.x; st[5] = c.y; st[6] = c.z; st[7] = c.w;
    }
    uint32_t fb[8], ptile = 0;
    const int bw = bit_weight(4 * i16);            // the same weight for all eight tokens
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st[m], lamS, m < 4 ? mu0 : mu1));
      const uint32_t Pm = cqm::p_fixed(p);
      ptile += Pm;
      fb[m] = cqm::sdigits(Pm << bw);
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

  // ---- segment ends: only what fixes g waits at the barrier -----------------
  // min / max of this wave's scores of unit j, per head
  auto finish_keys = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
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
  };
  // this wave's value sums of unit j: exact integers into LDS
  auto flush_values = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
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
  };
  // after the barrier: g of unit j (every lane, head g4); the visual weights
  // are taken relative to the largest calibrated visual exponent
  auto stats = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int par = j & 1, tri = j % 3;
    const int hh = g4 < G ? g4 : 0;
    float m = i16 < kW ? s_mm[par][i16][hh][0] : INFINITY;
    float M = i16 < kW ? s_mm[par][i16][hh][1] : -INFINITY;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      m = fminf(m, __shfl_xor(m, off));
      M = fmaxf(M, __shfl_xor(M, off));
    }
    const double scale = ldexp(4.0, -s_F[tri][hh]);          // real score per unit of s
    const double c0 = s_c0[tri][hh];
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
    muS = g4 < G ? (float)(mu * 1.4426950408889634) : -INFINITY;
    if (wave == 0 && i16 == 0 && g4 < G) s_vmax[par][g4] = (float)vis_max;
  };

  // ---- side tasks, run between steps -------------------------------------------
  // key-tail scores of unit j (every thread: token tid / kLpt of a round,
  // channels kCpt (tid % kLpt) ..), from inputs requested a step earlier
  uint4 ktr[kKl];
  auto key_tail = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int par = j & 1;
    for (int r = 0; r * kKtr < T; ++r) {
      uint4 kx[kKl];
      if (r == 0) {
#pragma unroll
        for (int i = 0; i < kKl; ++i) kx[i] = ktr[i];
      } else {
        load_ktail(j, r, kx);
      }
      float kf[kCpt];
#pragma unroll
      for (int i = 0; i < kKl; ++i) {
        const uint32_t w[4] = {kx[i].x, kx[i].y, kx[i].z, kx[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (F32) {
            kf[4 * i + c] = __uint_as_float(w[c]);
          } else {
            kf[8 * i + 2 * c] = h2f(w[c] & 0xFFFFu);
            kf[8 * i + 2 * c + 1] = h2f(w[c] >> 16);
          }
        }
      }
      const int tok = r * kKtr + tid / kLpt, c0 = kCpt * (tid % kLpt);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < G) {
          float sc = 0.f;
#pragma unroll
          for (int c = 0; c < kCpt; c += 4) {
            const float4 qq = *reinterpret_cast<const float4*>(&s_q[par][h][c0 + c]);
            sc = fmaf(qq.x, kf[c], sc);
            sc = fmaf(qq.y, kf[c + 1], sc);
            sc = fmaf(qq.z, kf[c + 2], sc);
            sc = fmaf(qq.w, kf[c + 3], sc);
          }
#pragma unroll
          for (int off = 1; off < kLpt; off <<= 1) sc += __shfl_xor(sc, off);
          if (tid % kLpt == 0 && tok < T) s_ts[par][h][tok] = sc;
        }
      }
    }
  };
  // value tail of unit j: weights exp(s_t - max_t s_t) of the wave's tail
  // tokens, then their value sums (lane = channel pair) into LDS
  uint32_t vtr[kVtw * (F32 ? 2 : 1)];
  auto value_tail = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
    const int par = j & 1;
    float tm = -INFINITY;
    if (g4 < G)
      for (int t = i16; t < T; t += 16) tm = fmaxf(tm, s_ts[par][g4][t]);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
    if (wave == 0 && i16 == 0 && g4 < G) s_tm[par][g4] = tm;
    float pts = 0.f;
    if (i16 < kMaxT / kW) {
      const int tok = (i16 / kVtw) * kVtr + wave + kW * (i16 % kVtw);
      float p = 0.f;
      if (g4 < G && tok < T) p = exp2f((s_ts[par][g4][tok] - tm) * kLog2e);
      s_pw[wave][g4][i16] = p;
      pts = p;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) pts += __shfl_xor(pts, off);
    if (i16 == 0) s_pt[par][wave][g4] = pts;
    wave_sync_lds();
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
          const float p = s_pw[wave][h][r * kVtw + i];   // 0 past the tail and for heads >= G
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
  // unit j written out (thread = head tid / 128, channel tid % 128) and its
  // sums cleared: the visual part weighs exp(vis_max - top), the tail part
  // exp(tail max - top)
  auto output = [&](int j) {
    asm volatile("" : "+v"(tid_v));        // lane coordinates formed here
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
      const float vx = s_vmax[par][h], tx = T > 0 ? s_tm[par][h] : -INFINITY, top = fmaxf(vx, tx);
      const float av = exp2f((vx - top) * kLog2e), at = T > 0 ? exp2f((tx - top) * kLog2e) : 0.f;
      float o = at * s_tacc[par][h][c] + av * (ovs * sv + pv * ovm);
      o /= av * pv + at * pt;
      const size_t oi = ((size_t)b * P.Hq + hk * G + h) * 128 + c;
      if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
      else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
      s_vsum[par][h][c] = 0ull;
      s_tacc[par][h][c] = 0.f;
    }
  };
  // Side tasks of segment j (1 <= j < U, or 0 for the first, U for the last):
  // the key tail of u_j, the value tail of u_{j-1}, the prologue of u_{j+1}
  // and the output of u_{j-2}, each fed by loads requested one key step
  // before it runs (all at the segment start when TPW = 1).
  auto req_kt = [&](int j) { load_ktail(j, 0, ktr); };
  auto req_vt = [&](int j) { load_vtail(j, 0, vtr); };
  auto req_pro = [&](int j) { load_prologue(j); };
  auto req_out = [&](int j) { load_vsvm(j); };
  auto run_kt = [&](int j) { if (j < U) key_tail(j); };
  auto run_vt = [&](int j) { if (j >= 0 && j < U) value_tail(j); };
  auto run_pro = [&](int j) { if (j < U) prologue(j); };
  auto run_out = [&](int j) { if (j >= 0) output(j); };
  // requests at the start of segment j, and tasks after its key / value step k
  auto side_start = [&](int j) {
    req_kt(j);
    if (TPW <= 2) req_vt(j - 1);
    if (TPW == 1) {
      req_pro(j + 1);
      req_out(j - 2);
    }
  };
  auto side_after = [&](int j, int k) {
    if constexpr (TPW >= 4) {
      if (k == 0) { run_kt(j); req_vt(j - 1); }
      if (k == 1) { run_vt(j - 1); req_pro(j + 1); }
      if (k == 2) { run_pro(j + 1); req_out(j - 2); }
      if (k == 3) run_out(j - 2);
    } else if constexpr (TPW == 2) {
      if (k == 0) { run_kt(j); run_vt(j - 1); req_pro(j + 1); req_out(j - 2); }
      if (k == 1) { run_pro(j + 1); run_out(j - 2); }
    } else {
      run_kt(j);
      run_vt(j - 1);
      run_pro(j + 1);
      run_out(j - 2);
    }
  };

  // ---- run ------------------------------------------------------------------
  for (int i = tid; i < 2 * 4 * 128; i += kTh) {
    (&s_vsum[0][0][0])[i] = 0ull;
    (&s_tacc[0][0][0])[i] = 0.f;
  }
  for (int i = tid; i < 2 * 4 * 4 * 128 / 4; i += kTh) reinterpret_cast<uint32_t*>(&s_a8[0][0][0][0])[i] = 0u;
  // Every wave keeps two steps in flight: consuming a step requests the step
  // two places later in the sequence K_0(0..TPW-1), [V_{j-1}(k) K_j(k)] for
  // j = 1 .. U-1, V_{U-1}(0..TPW-1); its ring slot is its position's parity.
  load_prologue(0);
  load_key(0, 0, ring[0]);
  if (TPW > 1) load_key(0, 1, ring[1]);
  else load_val(0, 0, ring[1]);
  lds_barrier();                                   // the LDS is cleared
  prologue(0);
  lds_barrier();
  read_digits(0);

  // segment 0: key tiles of u_0 (side tasks: key tail of u_0, prologue of u_1)
  side_start(0);
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    key_step(k, ring[k & 1]);
    if (k + 2 < TPW) load_key(0, k + 2, ring[k & 1]);
    else if (k + 2 == TPW) load_val(0, 0, ring[k & 1]);             // position 0 after the segment
    else if (U > 1) load_key(1, 0, ring[k & 1]);                     // position 1: K_1(0) ...
    else load_val(0, 1, ring[k & 1]);                                // ... or V_0(1) when u_0 is the last
    __builtin_amdgcn_sched_barrier(0);
    side_after(0, k);
    __builtin_amdgcn_sched_barrier(0);
  }
  finish_keys(0);
  lds_barrier();
  if (U > 1) read_digits(1);
  stats(0);

  // middle segments: positions 2 k (value tile k of u_{j-1}) and 2 k + 1 (key
  // tile k of u_j) after the segment's first, whose parity is that of TPW
  for (int j = 1; j < U; ++j) {
    asm volatile("" : "+v"(tid_v));
    constexpr int p0 = TPW & 1;                    // parity of the segment's first position
    side_start(j);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      uint4 (&sv)[2] = ring[(p0 + 2 * k) & 1];
      uint4 (&sk)[2] = ring[(p0 + 2 * k + 1) & 1];
      // the value step of tile k and the key step of tile k are independent:
      // the compiler may interleave them
      value_step(k, sv);
      if (k + 1 < TPW) load_val(j - 1, k + 1, sv);
      else load_val(j, 0, sv);
      key_step(k, sk);
      if (k + 1 < TPW) load_key(j, k + 1, sk);
      else if (j + 1 < U) load_key(j + 1, 0, sk);
      else load_val(j, 1, sk);
      __builtin_amdgcn_sched_barrier(0);
      side_after(j, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    finish_keys(j);
    flush_values(j - 1);
    lds_barrier();
    if (j + 1 < U) read_digits((j + 1) & 1);
    stats(j);
  }

  // last segment: value tiles of u_{U-1} (side tasks: its value tail, the
  // output of u_{U-2})
  asm volatile("" : "+v"(tid_v));
  {
    constexpr int p0 = TPW & 1;
    side_start(U);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      value_step(k, ring[(p0 + k) & 1]);
      if (k + 2 < TPW) load_val(U - 1, k + 2, ring[(p0 + k) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      side_after(U, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  req_out(U - 1);
  flush_values(U - 1);
  lds_barrier();
  output(U - 1);
}

#undef tid
#undef lane
#undef i16
#undef g4

template <int KW, bool F32>
hipError_t launch_w(const PP& p, int tpw, int grid, hipStream_t st) {
  const bool full = p.n == KW * tpw * kTile;
  const dim3 g(grid), b(KW * 64);
  switch (tpw) {
    case 1:
      if (full) CQ_LAUNCH((dp_b1<KW, 1, F32, true>), g, b, 0, st, p);
      else CQ_LAUNCH((dp_b1<KW, 1, F32, false>), g, b, 0, st, p);
      break;
    case 2:
      if (full) CQ_LAUNCH((dp_b1<KW, 2, F32, true>), g, b, 0, st, p);
      else CQ_LAUNCH((dp_b1<KW, 2, F32, false>), g, b, 0, st, p);
      break;
    case 4:
      if (full) CQ_LAUNCH((dp_b1<KW, 4, F32, true>), g, b, 0, st, p);
      else CQ_LAUNCH((dp_b1<KW, 4, F32, false>), g, b, 0, st, p);
      break;
    default:
      if (full) CQ_LAUNCH((dp_b1<KW, kMaxTiles / KW, F32, true>), g, b, 0, st, p);
      else CQ_LAUNCH((dp_b1<KW, kMaxTiles / KW, F32, false>), g, b, 0, st, p);
      break;
  }
  return hipSuccess;
}

// 8 waves: at 16 (four per SIMD) the kernel needs more than the 128 registers
// a wave may then hold, and its spills (whose reloads wait for every load in
// flight) made it slower (59 against 48.5 us at 64 x 8 units, n = 8192)
constexpr int kWaves = 8;

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

int tiles_per_wave(int n, int waves) {
  const int per = ((n + kTile - 1) / kTile + waves - 1) / waves;
  return per <= 1 ? 1 : (per <= 2 ? 2 : (per <= 4 ? 4 : 8));
}



}  // namespace

namespace cqi {

// b = 1, d = 128, G in {1, 2, 4}, 32 <= n <= 8192, n % 32 == 0, T <= 128,
// q and tails in one dtype, each code tensor at most 2 GB
bool decode_pipe_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n >= 32 &&
         a.n <= kMaxTiles * kTile && a.n % 32 == 0 && a.T <= kMaxT && (a.T == 0 || a.tail_dtype == a.q_dtype) &&
         (long)a.B * a.Hkv >= 1 && (long long)a.B * a.Hkv * a.nc * 16 <= (1ll << 31);
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
  p.nc = a.nc;
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
  const int tpw = tiles_per_wave(a.n, kWaves);
  return a.q_dtype == CQ_F32 ? launch_w<kWaves, true>(p, tpw, grid, a.stream)
                             : launch_w<kWaves, false>(p, tpw, grid, a.stream);
}

}  // namespace cqi
