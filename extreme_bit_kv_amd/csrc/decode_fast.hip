// 1-bit post-scaled, calibrated decode attention on the matrix cores (gfx950).
//
// QbitAI article on CalibQuant, "Method" part 2: with per-channel scale and
// minimum, q . k_hat_i = (q * scale_K) . c_i + q . min_K and
// sum_i p_i v_hat_i = scale_V * sum_i p_i c_i + (sum_i p_i) min_V, so only the
// integer codes enter the products; part 3: the visual scores of each query
// head are mapped by the affine g fixed by their min and max before softmax.
//
// One workgroup (8 waves) per (batch, kv head); its query heads (G <= 4)
// share every code it reads.  The 128-token tiles are dealt to the waves as
// they free up (an LDS counter per pass), so a wave whose loads return late
// does not hold the others at the next barrier.  Two workgroups fit on a CU,
// so a whole decode step (every unit of the batch) is resident at once.
//
// K side, per tile (b = 1): C[16 x 16] = A[16 x 128] B[128 x 16] with the
// 16x16x128 f8f6f4 product, A in fp6 (e2m3), B in fp4 (e2m1).  B is the
// packed key word masked in place, one operation per register: the fields
// whose code sits in bit 0, 1 or 2 read 0.5 c, c or 2 c, the bit-3 fields
// are forced to +-1 (1 - 2 c).  Rows of A are (head, digit plane): each
// head's q * scale_K is the integer Q = round(q' 2^F) (|Q| below 2^18.8, F
// from the largest |q'|) in four balanced base-31 digits d in [-15, 15],
// each stored as d / 2, d / 4, d / 8 or -d / 8 for the four field kinds, so
// every product is exactly d c / 4, every plane sum is exact in float32, and
// the bit-3 fields leave the constant -Q / 8 per channel, added back to the
// head's offset with q . min_K.  Columns are tokens; each lane ends up with
// all four planes of one (head, token) score s = ((D0 31 + D1) 31 + D2) 31 +
// D3, formed by the same operations in both passes and kept in these units
// (the statistics take the scale 4 2^-F and the offset).  The first pass
// over the keys only gathers every head's min and max, which fix g; the
// scores of a unit's first key tiles wait in LDS for the value pass, which
// reads the other key tiles again (partly from the Infinity Cache) and
// recomputes the same scores, since keeping 4 B per head and token for every
// tile would leave room for one workgroup per CU only.  Tiles are read with
// buffer loads: one descriptor per unit
// and tensor, a fixed byte offset per lane, and a tile past the last reads
// out of range (zeros, no traffic).
//
// V side, per tile: C[16 x 16] += A[16 x 64] B[64 x 16], rows again
// (head, plane), columns channels, contraction over tokens; B is the masked
// V word as on the K side.  p = exp(g(s) - max) in (0, 1] becomes
// P = floor(p 2^27); token i's digits are those of P 2^(7 - s(i)), signed
// base 256 (the bytes of x + 0x808080, the low three offset back by 128).
// A lane produces the digits of 8 consecutive tokens of one head, so one LDS
// write / read pair per wave (a 4 x 4 byte transpose in registers) hands
// them to the lanes that feed A.  The planes combine into the exact integer
// 2^7 sum_i P_i c_i, and the normalizer is sum_i P_i (the same weights),
// both summed exactly: the result does not depend on which wave took which
// tile.
//
// The text tail (float K/V) is handled in plain float32 arithmetic.
#include "cq_device.h"
#include "cq_internal.h"
#include "cq_mfma.h"

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 128;
constexpr int kMaxTail = 256;
constexpr int kPreTail = 64;          // tail tokens whose loads are issued early
constexpr int kXRounds = 3;           // later tail-key rounds whose loads are in flight together
constexpr int kXTokens = 8;           // later tail-value tokens per thread whose loads are in flight together
constexpr float kLog2e = 1.4426950408889634f;

using cqm::v4i;
using cqm::ld_any;
using cqm::spread_lo;
using cqm::spread_hi;
using cqm::bits_lo;
using cqm::bits_hi;
using cqm::bit_weight;
using cqm::transpose_bytes;
using cqm::mfma;
using cqm::gather_byte;
using cqm::wave_sync_lds;
using cqm::lds_barrier;

// Every load of the kernels below is issued without a branch: at the join
// of a branch around a load the compiler waits for it (and for everything
// issued before it), which would serialize the prefetches.  Indices are
// clamped into the tensor instead, and what they fetch past its end is
// discarded where it is used.  An empty tensor (n == 0 or T == 0, possibly a
// NULL pointer) is read at this 512-byte block instead: its base pointer is
// selected once, and the clamped offsets of an empty tensor stay below 512 B.
__device__ __align__(16) uint32_t g_pad[128];

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
constexpr int kQMax = 15 * (31 * 31 * 31 + 31 * 31 + 31 + 1);   // largest |Q| with four base-31 digits
constexpr int kRsrcFlags = 0x00020000;                            // raw buffer, 32-bit data format

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

// min / max of three floats in one instruction (never NaN here, so no quieting)
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

// The bit-3 fields of a key word as fp4 +-1: (w & 0x88888888) | 0x22222222
// in one instruction (v_and_or_b32, the mask in a scalar register): c2 holds
// 0x22222222 in a vector register, since a VOP3 instruction takes no literal.
__device__ __forceinline__ uint32_t sign_fields(uint32_t w, uint32_t c2) {
  constexpr uint32_t m = 0x88888888u;
  return (w & m) | (c2 & ~m);
}

__device__ __forceinline__ uint4 ld_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(x.x, x.y, x.z, x.w);
}

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
  int nc;               // token capacity of the code buffers (their layout is that of nc >= n tokens)
};

// The part of a text tail beyond the fused pass's kMaxTail tokens (T >
// kMaxTail), for one unit, run by the 8 waves of its workgroup after its
// visual sums are done, in chunks of kMaxTail tokens with a running reference
// (online softmax):
//   m = max_t s_t so far;  acc = sum_t exp(s_t - m) vt_t;  pt = sum_t exp(s_t - m),
// rescaled by exp(m_old - m_new) when a chunk raises m (the text tail is not
// quantized: "Method" part 2 applies to the visual cache only, per the
// abstract).  It starts from the fused pass's first kMaxTail tokens (their
// sums per (phase, head, channel) in s_tailred, relative to the reference in
// s_tm, their weight in s_ptail) and leaves sum_t exp(s_t - m) vt_t over all
// T tokens in s_tailred, the sums in s_ptail and m in s_tm.  Chunk scores: thread (token
// 4 wave + lane / 16 + 32 r, channels 8 (lane % 16) ..); chunk values: thread
// (channel pair tid % 64, tokens tid / 64 + 8 i).
template <int G, bool F32>
__device__ void long_tail(const Params& P, int unit, const float (&s_q)[4][128], float (&s_ts)[4][kMaxTail],
                          float (&s_tailred)[kThreads / 64][4][128], float* s_ptail, float* s_tm, float* s_cm,
                          float* s_cs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane >> 4, cl = lane & 15, vcp = tid & 63, vph = tid >> 6;
  const int T = P.T;
  constexpr int kRounds = kMaxTail / (4 * kWaves);              // 8 score rounds of 32 tokens
  constexpr int kVals = kMaxTail / kWaves;                      // 32 value tokens per thread
  const char* ktb = reinterpret_cast<const char*>(P.kt);
  const char* vtb = reinterpret_cast<const char*>(P.vt);
  float m_run[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, pt[4] = {0.f, 0.f, 0.f, 0.f};
  float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {                 // the fused pass's first kMaxTail tokens
    m_run[hh] = s_tm[hh];
    pt[hh] = s_ptail[hh];
    ta[hh][0] = s_tailred[vph][hh][2 * vcp];
    ta[hh][1] = s_tailred[vph][hh][2 * vcp + 1];
  }
  for (int c0 = kMaxTail; c0 < T; c0 += kMaxTail) {
    // this chunk's value inputs are requested first, then its keys (rows
    // past T read the last row: clamped, and their weights are 0)
    uint32_t vr[kVals][F32 ? 2 : 1];
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
      const size_t e = ((size_t)unit * T + min(c0 + vph + kWaves * i, T - 1)) * 128 + 2 * vcp;
      if constexpr (F32) {
        const uint2 x = *reinterpret_cast<const uint2*>(vtb + e * 4);
        vr[i][0] = x.x;
        vr[i][F32 ? 1 : 0] = x.y;
      } else {
        vr[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vtb + e * 2));
      }
    }
    // the chunk's key rounds, kLR at a time with their loads in flight
    // together; the heads' sums of a round side by side
    constexpr int kLR = F32 ? 1 : 4;
#pragma unroll
    for (int r0 = 0; r0 < kRounds; r0 += kLR) {
      uint4 kr[kLR][2];
#pragma unroll
      for (int x = 0; x < kLR; ++x) {
        const int j = c0 + 4 * wave + sub + 4 * kWaves * (r0 + x);
        const size_t e = ((size_t)unit * T + min(j, T - 1)) * 128 + 8 * cl;
        if constexpr (F32) {
          const uint4* src = reinterpret_cast<const uint4*>(ktb + e * 4);
          kr[x][0] = cqd::ld_nt(src);
          kr[x][1] = cqd::ld_nt(src + 1);
        } else {
          kr[x][0] = cqd::ld_nt(reinterpret_cast<const __half*>(ktb + e * 2));
          kr[x][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < kLR; ++x) {
        const int j = c0 + 4 * wave + sub + 4 * kWaves * (r0 + x);
        float kf[8];
        if constexpr (F32) {
          const uint32_t w[8] = {kr[x][0].x, kr[x][0].y, kr[x][0].z, kr[x][0].w,
                                 kr[x][1].x, kr[x][1].y, kr[x][1].z, kr[x][1].w};
#pragma unroll
          for (int c = 0; c < 8; ++c) kf[c] = __uint_as_float(w[c]);
        } else {
          const uint32_t w[4] = {kr[x][0].x, kr[x][0].y, kr[x][0].z, kr[x][0].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(w[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(w[c] >> 16)));
          }
        }
        float sc[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          sc[hh] = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) sc[hh] = fmaf(s_q[hh][8 * cl + c], kf[c], sc[hh]);
        }
        cqm::row_sum16x(sc);
        if (cl == 0) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) s_ts[hh][j - c0] = j < T ? sc[hh] : -INFINITY;
        }
      }
    }
    cqm::lds_barrier();
    if (wave < G) {                               // wave hh: the chunk's largest score
      const int hh = wave;
      float cm = -INFINITY;
      for (int t = lane; t < kMaxTail; t += 64) cm = fmaxf(cm, s_ts[hh][t]);
      cm = cqm::wave_max(cm);
      if (lane == 0) s_cm[hh] = cm;
    }
    cqm::lds_barrier();
    float m_new[4], rs[4];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m_new[hh] = fmaxf(m_run[hh], s_cm[hh]);
      rs[hh] = exp2f((m_run[hh] - m_new[hh]) * kLog2e);       // 0 for the first chunk
    }
    if (wave < G) {                               // wave hh: weights in place, their sum
      const int hh = wave;
      float cs = 0.f;
      for (int t = lane; t < kMaxTail; t += 64) {
        const float pw = exp2f((s_ts[hh][t] - m_new[hh]) * kLog2e);   // 0 past T
        s_ts[hh][t] = pw;
        cs += pw;
      }
      cs = cqm::wave_sum(cs);
      if (lane == 0) s_cs[hh] = cs;
    }
    cqm::lds_barrier();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      ta[hh][0] *= rs[hh];
      ta[hh][1] *= rs[hh];
      pt[hh] = pt[hh] * rs[hh] + s_cs[hh];
      m_run[hh] = m_new[hh];
    }
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
      float v0, v1;
      if constexpr (F32) {
        v0 = __uint_as_float(vr[i][0]);
        v1 = __uint_as_float(vr[i][F32 ? 1 : 0]);
      } else {
        v0 = __half2float(__ushort_as_half((unsigned short)(vr[i][0] & 0xFFFF)));
        v1 = __half2float(__ushort_as_half((unsigned short)(vr[i][0] >> 16)));
      }
      const int t = vph + kWaves * i;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
        ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
      }
    }
    cqm::lds_barrier();                           // the chunk's weights are read before the next scores
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    s_tailred[vph][hh][2 * vcp] = ta[hh][0];
    s_tailred[vph][hh][2 * vcp + 1] = ta[hh][1];
  }
  if (tid < G) {
    s_ptail[tid] = pt[tid];
    s_tm[tid] = m_run[tid];
  }
}

// F32: query and text tail are float32 (else float16); the fast path takes
// them in one dtype.
// LT: the text tail is longer than kMaxTail (a separate instance, so that the
// chunked tail's registers do not weigh on the kernel of the common case)
// TPW > 0: every code tile of the unit in flight at once, for launches of at
// most one workgroup per CU.  Wave w owns tiles w, w + 8, ... (at most TPW);
// its key and value tiles, and the text tail, are all requested at the start,
// and the scores stay in registers between the two passes (no second read of
// the keys).  The arithmetic is the same as with dealt tiles (min / max and
// exact integer sums do not depend on which wave took a tile), so the outputs
// are the same bit for bit.  Two waves per SIMD: up to 256 VGPRs.
template <int G, bool F32, bool LT, int TPW = 0>
__global__ void __launch_bounds__(kThreads, TPW > 0 ? 2 : 4) df_b1(Params P) {
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T;
  // the text tail in the fused pass (scores beside the prologue, values
  // beside the value pass), its first kMaxTail tokens when longer: the rest
  // runs in chunks at the end
  const int Tf = LT ? kMaxTail : T;
  const int ntiles = (n + kTile - 1) / kTile;
  const int R = n >> 5;
  const int nc = P.nc, Rc = nc >> 5;           // the code buffers' layout: nc tokens
  // Issue priority: the two workgroups on a CU would otherwise run their key
  // passes unevenly (the older one first), leaving the other's value pass
  // alone at the end.  High through the key pass (latency-bound), low through
  // the value pass (compute-bound), medium for the final reduction.
  __builtin_amdgcn_s_setprio(3);

  __shared__ float s_q[4][128];                 // sm * q, float
  __shared__ double s_c0[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][4][32];   // K-side fp6 digit codes: [head][plane][128 k slots]
  __shared__ float s_kc[4];                              // per head: sum of Q / 8 over the bit-3 channels
  // V-side A digits, [head][plane][128 token bytes] per wave: with dealt
  // tiles they go to the wave's home slot of s_keep instead (below)
  __shared__ __align__(16) uint32_t s_pdig[TPW > 0 ? kWaves : 1][4][4][32];
  __shared__ float s_ts[4][kMaxTail];           // tail scores, then tail probabilities
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4], s_alpha[4];
  __shared__ float s_vmax[4], s_tm[4], s_cm[4], s_cs[4];   // visual max, tail reference; long-tail chunk max / sum
  // dealt tiles, text tail up to kMaxTail: the tail-value sums stay in registers
  // through the value pass (then in the home slots of s_keep), which leaves
  // room for more kept scores
  constexpr bool kRegTail = TPW == 0 && !LT;
  constexpr int kTR = kRegTail ? 1 : kThreads / 64, kTH = kRegTail ? 1 : 4, kTC = kRegTail ? 1 : 128;
  __shared__ float s_tailred[kTR][kTH][kTC];   // tail values per token phase (unused with kRegTail)
  __shared__ unsigned long long s_vsum[4][128];   // sum 2^7 P c per head and channel (2^-29 units)
  __shared__ double s_psum[4];                     // sum P per head (2^-22 units)
  __shared__ int s_next[2];                        // next key tile of each pass
  __shared__ float s_vs[128], s_vm[128];           // scale_V, min_V
  // Dealt tiles: the scores of the unit's first kKeep tiles stay in LDS from
  // the key pass to the value pass ([tile][lane][token], a lane's 8 scores),
  // so those key tiles are read once; the others are read again and their
  // scores recomputed (same operations, so the same values).  kKeep fills
  // the LDS that two workgroups per CU leave.  Slot w (2 KB) is also wave w's
  // home: the value pass deals wave w tile w first, whose scores it reads
  // before anything else, so from then on the slot holds the wave's digits
  // of each tile (its s_pdig), and after the value pass its tail-value sums.
  constexpr int kKeep = TPW == 0 ? (kRegTail ? 33 : 25) : 0;
  static_assert(TPW > 0 || kKeep >= kWaves, "every wave needs a home slot");
  __shared__ __align__(16) float s_keep[kKeep > 0 ? kKeep : 1][64][8];

  // operand coordinates of the 16 x 16 x 64 products
  const int i16 = lane & 15, g4 = lane >> 4;    // A/B operand lane coordinates
  const int rh = i16 >> 2, rp = i16 & 3;        // A row = (head rh, plane rp)
  const int oh = lane >> 4;                     // output lane: head
  const uint32_t* kc = n > 0 ? P.kc : g_pad;
  const uint32_t* vcb = n > 0 ? P.vc : g_pad;
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(g_pad);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(g_pad);
  // The prologue's inputs are requested before any prefetch: vector loads
  // complete in order, so the prologue then waits for these alone.  Wave w < 4
  // takes head w (heads past G read head G - 1, unused) at channels lane and
  // lane + 64, so that each head's statistics and digits stay within one wave;
  // waves 4 and 5 stage scale_V and min_V.  Every lane loads all of it (no
  // load under a branch); an empty cache's scales and minima are read at the
  // zero block.
  const float* ksb = n > 0 ? P.ks : reinterpret_cast<const float*>(g_pad);
  const float* kmb = n > 0 ? P.km : reinterpret_cast<const float*>(g_pad);
  const float* vsb = n > 0 ? P.vs : reinterpret_cast<const float*>(g_pad);
  const float* vmb = n > 0 ? P.vm : reinterpret_cast<const float*>(g_pad);
  const size_t prm = n > 0 ? (size_t)unit * 128 : 0;
  const size_t qrow = ((size_t)b * P.Hq + h * G + min(wave & 3, G - 1)) * 128;
  const float q_lo = ld_any(P.q, qrow + lane, F32), q_hi = ld_any(P.q, qrow + lane + 64, F32);
  const float ks_lo = ksb[prm + lane], ks_hi = ksb[prm + lane + 64];
  const float km_lo = kmb[prm + lane], km_hi = kmb[prm + lane + 64];
  const int vj = lane + 64 * (wave & 1);
  const float vs_in = vsb[prm + vj], vm_in = vmb[prm + vj];
  // Code tiles are read with buffer loads: one descriptor per unit and tensor,
  // a fixed byte offset per lane plus the tile's (wave-uniform); a tile past
  // the last reads out of range, which returns zeros without any traffic.
  const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + (n > 0 ? (size_t)unit * 4 * nc : 0)), (short)0,
                                                    n > 0 ? nc * 16 : 0, kRsrcFlags);
  const uint32_t koff = (uint32_t)(g4 * nc + 8 * i16) * 4u;
  auto load_k = [&](int tile, uint4& w0, uint4& w1) {   // tokens past n: scores not used
    const uint32_t off = koff + (tile < ntiles ? (uint32_t)tile * 512u : 0x80000000u);
    w0 = ld_buf(rk, off);
    w1 = ld_buf(rk, off + 16u);
  };
  // The first kPreTail tail keys, as (token 4 wave + lane/16 + 32 r, channels
  // 8 (lane%16) ..+7), are requested first: their scores are formed right
  // after the prologue, while the first key tiles are still in flight.  The
  // tail is read once and, unlike the codes, is not in the cache from a
  // producer just before, so its loads are non-temporal.
  const int tsub = lane >> 4, tcl = lane & 15;
  constexpr int kKtRounds = kPreTail / (4 * kWaves);
  uint4 ktp[kKtRounds][2];
#pragma unroll
  for (int r = 0; r < kKtRounds; ++r) {
    const int j = 4 * wave + tsub + 4 * kWaves * r;   // rows past T: scores not stored
    const size_t e = ((size_t)unit * T + max(min(j, T - 1), 0)) * 128 + 8 * tcl;
    if constexpr (F32) {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
      ktp[r][0] = cqd::ld_nt(src);
      ktp[r][1] = cqd::ld_nt(src + 1);
    } else {
      ktp[r][0] = cqd::ld_nt(reinterpret_cast<const __half*>(ktb) + e);
      ktp[r][1] = make_uint4(0, 0, 0, 0);
    }
  }
  // V word row of this lane, channels 8*i16 .. +7.  Rows past the last hold
  // tokens whose p is 0: whatever codes they read, their digits are 0.
  const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vcb + (n > 0 ? (size_t)unit * Rc * 128 : 0)), (short)0,
                                                    R * 512, kRsrcFlags);
  const uint32_t voff = (uint32_t)(g4 * 128 + 8 * i16) * 4u;
  auto load_v = [&](int tile, uint4& w0, uint4& w1) {
    const uint32_t off = voff + (tile < ntiles ? (uint32_t)tile * 2048u : 0x80000000u);
    w0 = ld_buf(rv, off);
    w1 = ld_buf(rv, off + 16u);
  };
  // tail values: thread (channel pair vcp, phase vph) holds channels 2 vcp,
  // 2 vcp + 1 of tokens vph + kPhases i, as raw bits converted where used
  constexpr int kPhases = kThreads / 64;
  const int vcp = tid & 63, vph = tid >> 6;
  uint32_t vtr[kPreTail / kPhases][F32 ? 2 : 1];
  auto load_vtail = [&]() {
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      const size_t e = ((size_t)unit * T + max(min(vph + kPhases * i, T - 1), 0)) * 128 + 2 * vcp;
      if constexpr (F32) {
        const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
        vtr[i][0] = x.x;
        vtr[i][F32 ? 1 : 0] = x.y;
      } else {
        vtr[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e));
      }
    }
  };
  // the key pass keeps two tiles of look-ahead per wave (a ring of three
  // tile slots: kn, km, kx), the value pass one (kn, vn); the first two are
  // requested under the prologue.  With
  // TPW > 0 every key tile of the wave is requested here, and the tail values
  // and value tiles right after the prologue (issued together with these, they
  // would delay the prologue's own inputs, which queue behind every CU's
  // requests).
  uint4 kn0, kn1, km0, km1, kx0, kx1;
  constexpr int kSlots = TPW > 0 ? TPW : 1;
  uint4 kwide[kSlots][2], vwide[kSlots][2];
  if constexpr (TPW > 0) {
#pragma unroll
    for (int k = 0; k < TPW; ++k) load_k(wave + kWaves * k, kwide[k][0], kwide[k][1]);
  } else {
    load_k(wave, kn0, kn1);
    load_k(wave + kWaves, km0, km1);
  }
  // Tiles are dealt dynamically: wave w starts with tile w and then takes the
  // next untaken one, so that a wave whose loads come back late does not hold
  // up the workgroup at the next barrier.  (Results do not depend on which
  // wave took which tile: min / max, and exact integer sums below.)
  if (tid == 0) {
    s_next[0] = 2 * kWaves;
    s_next[1] = kWaves;
  }
  if (tid < 4) s_psum[tid] = 0.0;
  for (int i = tid; i < 4 * 128; i += kThreads) (&s_vsum[0][0])[i] = 0ull;

  // ---- prologue: post-scaled query, fixed-point digits -------------------
  // Wave hh < 4 settles head hh alone (one barrier in all): sm q and
  // q' = sm q * scale_K, the offset c0 = sm q . min_K (the sums of channels
  // 0..63 and 64..127, each over the wave, then added), F from max |q'|, and
  // Q = round(q' 2^F) in four balanced base-31 digits.  Channel j sits in k
  // slot 32 (j / 32) + 8 R + 2 (e mod 4) + e / 16 of its row, e = j mod 32,
  // R = (e / 4) mod 4, the fp4 field of its key bit; its digit is stored as
  // d / 2, d / 4, d / 8 or -d / 8 (the bit-3 fields read +-1: 1 - 2 c), so
  // that every product is d c / 4 and the bit-3 channels leave a constant
  // sum of -Q / 8, added back to the head's offset.
  if (wave < 4) {
    const int hh = wave;
    float qv[2] = {0.f, 0.f}, qp[2] = {0.f, 0.f};
    double pr[2] = {0.0, 0.0};
    if (hh < G) {
      qv[0] = P.sm * q_lo;
      qv[1] = P.sm * q_hi;
      qp[0] = qv[0] * ks_lo;
      qp[1] = qv[1] * ks_hi;
      pr[0] = (double)qv[0] * (double)km_lo;
      pr[1] = (double)qv[1] * (double)km_hi;
    }
    s_q[hh][lane] = qv[0];
    s_q[hh][lane + 64] = qv[1];
    const double c0 = cqm::wave_sum(pr[0]) + cqm::wave_sum(pr[1]);
    const float mq = cqm::wave_max(fmaxf(fabsf(qp[0]), fabsf(qp[1])));
    int F = 0;
    if (mq > 0.f) {
      const int e = ilogbf(mq);
      F = ldexpf(mq, 18 - e) > (float)kQMax ? 17 - e : 18 - e;
    }
    unsigned char* ad = reinterpret_cast<unsigned char*>(&s_adig[hh][0][0]);
    float kcs = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int j = lane + 64 * c;
      const float x = rintf(ldexpf(qp[c], F));                       // |x| <= kQMax, exact
      float d[4], r = x;
#pragma unroll
      for (int k = 3; k > 0; --k) {
        const float qk = rintf(r * (1.f / 31.f));                    // exact: r / 31 is never near a half
        d[k] = fmaf(-31.f, qk, r);
        r = qk;
      }
      d[0] = r;
      const int e = j & 31, Rf = (e >> 2) & 3, slot = 32 * (j >> 5) + 8 * Rf + 2 * (e & 3) + (e >> 4);
      const int mult = Rf == 0 ? 4 : (Rf == 1 ? 2 : (Rf == 2 ? 1 : -1));
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) ad[pl * 128 + slot] = (unsigned char)enc6((int)d[pl] * mult);
      kcs += Rf == 3 ? 0.125f * x : 0.f;                             // multiples of 1/8 below 2^21: exact
    }
    kcs = cqm::wave_sum(kcs);
    if (lane == 0) {
      s_F[hh] = F;
      s_c0[hh] = c0;
      s_kc[hh] = hh < G ? kcs : 0.f;
    }
  } else if (wave < 6) {
    s_vs[vj] = vs_in;
    s_vm[vj] = vm_in;
  }
  lds_barrier();
  if constexpr (TPW > 0) {
    load_vtail();
#pragma unroll
    for (int k = 0; k < TPW; ++k) load_v(wave + kWaves * k, vwide[k][0], vwide[k][1]);
  }

  // ---- text tail scores ---------------------------------------------------
  // The prefetched rounds run straight (no early exit: every lane's rows were
  // loaded, in bounds, and rows past T are not stored); rounds past kPreTail
  // tokens load as they go.
  {
    const int sub = tsub, cl = tcl;
    auto tail_scores = [&](int j, const float (&kf)[8]) {
      float sc[G];                                   // the heads' sums side by side
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        sc[hh] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) sc[hh] = fmaf(s_q[hh][8 * cl + c], kf[c], sc[hh]);
      }
      cqm::row_sum16x(sc);
      if (cl == 0 && j < Tf) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s_ts[hh][j] = sc[hh];
      }
    };
#pragma unroll
    for (int r = 0; r < kKtRounds; ++r) {
      float kf[8];
      if constexpr (F32) {
        kf[0] = __uint_as_float(ktp[r][0].x); kf[1] = __uint_as_float(ktp[r][0].y);
        kf[2] = __uint_as_float(ktp[r][0].z); kf[3] = __uint_as_float(ktp[r][0].w);
        kf[4] = __uint_as_float(ktp[r][1].x); kf[5] = __uint_as_float(ktp[r][1].y);
        kf[6] = __uint_as_float(ktp[r][1].z); kf[7] = __uint_as_float(ktp[r][1].w);
      } else {
        const uint32_t hw[4] = {ktp[r][0].x, ktp[r][0].y, ktp[r][0].z, ktp[r][0].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
          kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
        }
      }
      tail_scores(4 * wave + 4 * kWaves * r + sub, kf);
    }
    constexpr int kXR = F32 ? 1 : kXRounds;
    // rounds past kPreTail tokens, kXR at a time: their keys are read as
    // the prefetched ones (clamped rows, whole 16-byte pieces, no branch), the
    // rounds' loads in flight together
    for (int j0 = 4 * wave + 4 * kWaves * kKtRounds; j0 < Tf; j0 += 4 * kWaves * kXR) {
      uint4 kr[kXR][2];
#pragma unroll
      for (int x = 0; x < kXR; ++x) {
        const size_t e = ((size_t)unit * T + max(min(j0 + 4 * kWaves * x + sub, T - 1), 0)) * 128 + 8 * cl;
        if constexpr (F32) {
          const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
          kr[x][0] = cqd::ld_nt(src);
          kr[x][1] = cqd::ld_nt(src + 1);
        } else {
          kr[x][0] = cqd::ld_nt(reinterpret_cast<const __half*>(ktb) + e);
          kr[x][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < kXR; ++x) {
        float kf[8];
        if constexpr (F32) {
          kf[0] = __uint_as_float(kr[x][0].x); kf[1] = __uint_as_float(kr[x][0].y);
          kf[2] = __uint_as_float(kr[x][0].z); kf[3] = __uint_as_float(kr[x][0].w);
          kf[4] = __uint_as_float(kr[x][1].x); kf[5] = __uint_as_float(kr[x][1].y);
          kf[6] = __uint_as_float(kr[x][1].z); kf[7] = __uint_as_float(kr[x][1].w);
        } else {
          const uint32_t hw[4] = {kr[x][0].x, kr[x][0].y, kr[x][0].z, kr[x][0].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
          }
        }
        tail_scores(j0 + 4 * kWaves * x + sub, kf);          // rows past T: scores not stored
      }
    }
  }
  // ---- phase 1: visual scores, their min and max -------------------------
  // K-side A operand of this lane: row (head rh, plane rp), k slots 32 g4 ..
  // +31 as 32 dense 6-bit fields in 6 registers (zero rows past G)
  v8i kdig = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  {
    const uint4* src = reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
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
    if (rh < G) kdig = v8i{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], 0, 0};
  }
  // scores of this lane's 8 tokens (head oh) from one key tile, in units of
  // s = Q . c / 4 less the bit-3 constant: C[16 x 16] = A[16 x 128] B[128 x 16]
  // with the 16x16x128 f8f6f4 product, A fp6 (e2m3) digits, B the key word
  // masked in place into fp4 (e2m1) fields; the plane sums are exact and the
  // same operations give the same scores in both passes
  uint32_t kc2 = 0x22222222u;                  // in a register for sign_fields
  asm volatile("" : "+v"(kc2));
  auto scores = [&](const uint4& w0, const uint4& w1, float (&st)[8]) {
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t w = wd[m];
      const v8i bq{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u),
                   (int)sign_fields(w, kc2), 0, 0, 0, 0};
      const v4f a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kdig, bq, v4f{0.f, 0.f, 0.f, 0.f}, 2, 4, 0,
                                                                      127, 0, 127);
      st[m] = fmaf(fmaf(fmaf(a[0], 31.f, a[1]), 31.f, a[2]), 31.f, a[3]);
      // pin the finished score: otherwise the compiler may keep the four
      // accumulator registers alive in its place
      asm volatile("" : "+v"(st[m]));
    }
  };
  float vmin = INFINITY, vmax = -INFINITY;
  float swide[kSlots][8];                       // TPW > 0: the wave's scores, kept for the value pass
  if constexpr (TPW > 0) {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave + kWaves * k;
      if (tile < ntiles) {
        scores(kwide[k][0], kwide[k][1], swide[k]);
        const float* st = swide[k];
        if ((tile + 1) * kTile <= n || tile * kTile + 8 * i16 < n) {
          vmin = min3f(min3f(vmin, st[0], st[1]), min3f(st[2], st[3], st[4]), min3f(st[5], st[6], st[7]));
          vmax = max3f(max3f(vmax, st[0], st[1]), max3f(st[2], st[3], st[4]), max3f(st[5], st[6], st[7]));
        }
      }
    }
  }
  // a wave's tiles come in increasing order.  The ring's slots keep their
  // roles through an unrolled round of three steps: a step requests the next
  // tile into the free slot and scores the oldest one, so two tiles stay in
  // flight while one is scored.  (Copying a slot into another would wait for
  // the load still in flight into it: one tile of look-ahead.)
  auto key_step = [&](const uint4& w0, const uint4& w1, int tile, uint4& f0, uint4& f1, int& tf)
                      __attribute__((always_inline)) {
    int nxt = 0;
    if (lane == 0) nxt = atomicAdd(&s_next[0], 1);
    nxt = __builtin_amdgcn_readfirstlane(nxt);
    load_k(nxt, f0, f1);                        // past the last tile: an out-of-range read, unused
    tf = nxt;
    // n % 32 == 0, so this lane's 8 tokens tile*128 + 8 i16 + m are all valid or none
    float st[8];
    scores(w0, w1, st);
    if ((tile + 1) * kTile <= n || tile * kTile + 8 * i16 < n) {
      vmin = min3f(min3f(vmin, st[0], st[1]), min3f(st[2], st[3], st[4]), min3f(st[5], st[6], st[7]));
      vmax = max3f(max3f(vmax, st[0], st[1]), max3f(st[2], st[3], st[4]), max3f(st[5], st[6], st[7]));
    }
    if (tile < kKeep) {
      float4* kp = reinterpret_cast<float4*>(&s_keep[tile][lane][0]);
      kp[0] = make_float4(st[0], st[1], st[2], st[3]);
      kp[1] = make_float4(st[4], st[5], st[6], st[7]);
    }
    // fold tile by tile: left free, the compiler sinks these updates past the
    // loop and keeps every tile's scores alive
    asm volatile("" : "+v"(vmin), "+v"(vmax));
  };
  if constexpr (TPW == 0) {
    int ta = wave, tb = wave + kWaves, tx = ntiles;
    while (ta < ntiles) {
      key_step(kn0, kn1, ta, kx0, kx1, tx);
      if (tb >= ntiles) break;
      key_step(km0, km1, tb, kn0, kn1, ta);
      if (tx >= ntiles) break;
      key_step(kx0, kx1, tx, km0, km1, tb);
    }
  }
  // the first key and value tiles of the second pass, then the first
  // kPreTail tail values, are requested before the score statistics settle.
  // (The key base goes through an opaque copy: otherwise the compiler proves
  // the second pass's loads equal the first's and keeps every first-pass score
  // alive instead of recomputing it.)
  asm("" : "+s"(kc));
  uint4 vn0, vn1;
  if constexpr (TPW == 0) {                     // the tail values first: they are used first
    load_vtail();
    load_k(wave < kKeep ? ntiles : wave, kn0, kn1);   // a kept tile: an out-of-range read, no traffic
    load_v(wave, vn0, vn1);
  }
  // ---- min / max of every head's visual scores ---------------------------
  vmin = cqm::row_min16(vmin);
  vmax = cqm::row_max16(vmax);
  if ((lane & 15) == 0) {
    s_red[wave][oh][0] = vmin;
    s_red[wave][oh][1] = vmax;
  }
  lds_barrier();
  if (wave < G) {                               // wave hh settles head hh
    const int hh = wave;
    float m = lane < kWaves ? s_red[lane][hh][0] : INFINITY;
    float M = lane < kWaves ? s_red[lane][hh][1] : -INFINITY;
    float tmax = -INFINITY;
    for (int j = lane; j < Tf; j += 64) tmax = fmaxf(tmax, s_ts[hh][j]);
    m = cqm::wave_min(m);
    M = cqm::wave_max(M);
    tmax = cqm::wave_max(tmax);
    // scores are in units of scale = 4 2^-F, offset by q . min_K plus the
    // bit-3 constant; the exponent of a visual weight is lam s + mu
    const double scale = ldexp(4.0, -s_F[hh]);
    const double c0 = s_c0[hh] + (double)s_kc[hh] * scale;
    double lam = scale, mu = -scale * (double)M, vis_max = (double)M * scale + c0;
    if (P.calib_on && n > 0) {
      const double mr = (double)m * scale + c0, Mr = (double)M * scale + c0;
      const double t_lo = (double)P.a_lo * mr + (double)P.c_lo, t_hi = (double)P.a_hi * Mr + (double)P.c_hi;
      // the largest value of g: the larger end of [t_lo, t_hi], or t_lo
      // when every score is the same (g is then the constant t_lo)
      vis_max = M > m ? fmax(t_lo, t_hi) : t_lo;
      lam = M > m ? (t_hi - t_lo) / ((double)(M - m) * scale) * scale : 0.0;
      mu = t_lo - vis_max - lam * (double)m;
    }
    const float top = fmaxf(n > 0 ? (float)vis_max : -INFINITY, tmax);
    if (lane == 0) {
      // visual weights relative to the largest one: p = 2^(s * lam' + mu');
      // alpha = its weight relative to the softmax reference
      s_lam[hh] = (float)(lam * 1.4426950408889634);
      s_mu[hh] = (float)(mu * 1.4426950408889634);
      s_alpha[hh] = n > 0 ? exp2f(((float)vis_max - top) * kLog2e) : 0.f;
      s_vmax[hh] = n > 0 ? (float)vis_max : -INFINITY;
      s_tm[hh] = top;                           // the fused tail's weights are taken relative to top
    }
    // tail probabilities (in place) and their sum
    float pt = 0.f;
    for (int j = lane; j < Tf; j += 64) {
      const float pj = exp2f((s_ts[hh][j] - top) * kLog2e);
      s_ts[hh][j] = pj;
      pt += pj;
    }
    pt = cqm::wave_sum(pt);
    if (lane == 0) s_ptail[hh] = pt;
  }
  lds_barrier();
  // text-tail values: thread (channel pair vcp, phase vph) sums the tail
  // tokens vph + kPhases i for every head, the first kPreTail from the loads above
  float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  {
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      // (a select, not a branch: a token past T weighs 0, and the heads'
      // weights of every token are read together)
      const int t = vph + kPhases * i;
      const bool tok = t < Tf;
      float v0, v1;
      if constexpr (F32) {
        v0 = __uint_as_float(vtr[i][0]);
        v1 = __uint_as_float(vtr[i][F32 ? 1 : 0]);
      } else {
        v0 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] & 0xFFFF)));
        v1 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] >> 16)));
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float w = tok ? s_ts[hh][t] : 0.f;
        ta[hh][0] = fmaf(w, v0, ta[hh][0]);
        ta[hh][1] = fmaf(w, v1, ta[hh][1]);
      }
    }
    constexpr int kXT = F32 ? 4 : kXTokens;
    // tokens past kPreTail, kXT at a time: loads in flight together
    // (clamped rows, no branch); a token past T weighs 0
    for (int t0 = kPreTail + vph; t0 < Tf; t0 += kPhases * kXT) {
      uint32_t vx[kXT][F32 ? 2 : 1];
#pragma unroll
      for (int x = 0; x < kXT; ++x) {
        const size_t e = ((size_t)unit * T + max(min(t0 + kPhases * x, T - 1), 0)) * 128 + 2 * vcp;
        if constexpr (F32) {
          const uint2 w2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
          vx[x][0] = w2.x;
          vx[x][F32 ? 1 : 0] = w2.y;
        } else {
          vx[x][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e));
        }
      }
#pragma unroll
      for (int x = 0; x < kXT; ++x) {
        const int t = t0 + kPhases * x;
        const bool tok = t < Tf;
        float v0, v1;
        if constexpr (F32) {
          v0 = __uint_as_float(vx[x][0]);
          v1 = __uint_as_float(vx[x][F32 ? 1 : 0]);
        } else {
          v0 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] & 0xFFFF)));
          v1 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] >> 16)));
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float w = tok ? s_ts[hh][min(t, kMaxTail - 1)] : 0.f;
          ta[hh][0] = fmaf(w, v0, ta[hh][0]);
          ta[hh][1] = fmaf(w, v1, ta[hh][1]);
        }
      }
    }
    if constexpr (!kRegTail) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        s_tailred[vph][hh][2 * vcp] = ta[hh][0];
        s_tailred[vph][hh][2 * vcp + 1] = ta[hh][1];
      }
    }
  }

  // ---- phase 2: values ------------------------------------------------------
  __builtin_amdgcn_s_setprio(0);
  const float lam2 = s_lam[oh < G ? oh : 0], mu2 = s_mu[oh < G ? oh : 0];
  // compensating factors of this lane's tokens 8 i16 + m (bits_lo / bits_hi):
  // 2^wt0 for m < 4, 2^wt1 for m >= 4
  const int wt0 = bit_weight(8 * i16), wt1 = bit_weight(8 * i16 + 4);
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  // the wave's int32 plane sums grow by at most 2^17 per tile (128 tokens x
  // |digit| <= 128 x code byte <= 8); they are moved into the exact 64-bit
  // LDS sums every kFlushTiles tiles, far below 2^31
  constexpr int kFlushTiles = 256;
  auto flush = [&]() {
    if (oh < G) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const long long sv = (long long)vacc[ct][0] + 256ll * vacc[ct][1] + 65536ll * vacc[ct][2] +
                             16777216ll * vacc[ct][3];
        atomicAdd(&s_vsum[oh][8 * i16 + ct], (unsigned long long)sv);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  };
  int wtiles = 0;
  double psum = 0.0;                            // sum of this lane's P (exact: integers below 2^53)
  unsigned char* pd = TPW > 0 ? reinterpret_cast<unsigned char*>(&s_pdig[wave][0][0][0])
                               : reinterpret_cast<unsigned char*>(&s_keep[wave][0][0]);
  // one value tile: probabilities of this lane's 8 tokens (head oh),
  // relative to the largest calibrated visual score, as fixed point
  // P = floor(p 2^27) (tokens that do not count get exponent -inf, so p = 0),
  // their digits through LDS to the A lanes, the products with the V words
  auto value_tile = [&](int tile, const float (&st)[8], const uint4& vw0, const uint4& vw1)
                        __attribute__((always_inline)) {
    const bool ok = oh < G && tile * kTile + 8 * i16 < n;
    const float mu_t = ok ? mu2 + 27.f : -INFINITY;   // the exponent of p 2^27
    uint32_t fb[8], ptile = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t Pm = cqm::p_fixed_exp2(fmaf(st[m], lam2, mu_t));   // exponent <= 27 (up to rounding)
      ptile += Pm;
      fb[m] = cqm::sdigits(Pm << (m < 4 ? wt0 : wt1));   // digits of P 2^wt, |P 2^wt| <= 2^30
    }
    psum += (double)ptile;
    if (oh < G) {
      uint32_t d[2][4];
      transpose_bytes(fb[0], fb[1], fb[2], fb[3], d[0][0], d[0][1], d[0][2], d[0][3]);
      transpose_bytes(fb[4], fb[5], fb[6], fb[7], d[1][0], d[1][1], d[1][2], d[1][3]);
#pragma unroll
      for (int pl = 0; pl < 4; ++pl)
        *reinterpret_cast<uint2*>(pd + (oh * 4 + pl) * 128 + 8 * i16) = make_uint2(d[0][pl], d[1][pl]);
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
      vacc[ct] = mfma(av0, bits_lo(vwd[ct]), vacc[ct]);
      vacc[ct] = mfma(av1, bits_hi(vwd[ct]), vacc[ct]);
    }
    wave_sync_lds();                       // digits read before the next tile overwrites them
  };
  if constexpr (TPW > 0) {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave + kWaves * k;
      if (tile < ntiles) value_tile(tile, swide[k], vwide[k][0], vwide[k][1]);
    }
  }
  for (int tile = wave; TPW == 0 && tile < ntiles;) {
    int nxt = 0;
    if (lane == 0) nxt = atomicAdd(&s_next[1], 1);
    nxt = __builtin_amdgcn_readfirstlane(nxt);
    const uint4 kw0 = kn0, kw1 = kn1, vw0 = vn0, vw1 = vn1;
    load_k(nxt < kKeep ? ntiles : nxt, kn0, kn1);
    load_v(nxt, vn0, vn1);
    float st[8];
    if (tile < kKeep) {
      const float4* kp = reinterpret_cast<const float4*>(&s_keep[tile][lane][0]);
      const float4 a = kp[0], c = kp[1];
      st[0] = a.x; st[1] = a.y; st[2] = a.z; st[3] = a.w;
      st[4] = c.x; st[5] = c.y; st[6] = c.z; st[7] = c.w;
    } else {
      scores(kw0, kw1, st);
    }
    value_tile(tile, st, vw0, vw1);
    if (++wtiles == kFlushTiles) {
      flush();
      wtiles = 0;
    }
    tile = nxt;
  }

  // ---- combine planes, reduce over waves --------------------------------
  __builtin_amdgcn_s_setprio(1);
  // lane (head oh, column i16): channels 8*i16 + ct.  The planes combine into
  // the exact integer 2^7 sum_i P_i c_i, and the waves add theirs with 64-bit
  // LDS atomics: exact, so the order in which waves arrive does not matter.
  flush();
  psum = cqm::row_sum16(psum);
  if ((lane & 15) == 0 && oh < G) atomicAdd(&s_psum[oh], psum);
  // [phase][head][channel] once the values are done: the eight home slots
  float* tr = reinterpret_cast<float*>(&s_keep[0][0][0]);
  if constexpr (kRegTail) {
    // phase vph is this wave: its home slot, which no other wave uses
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      tr[(vph * 4 + hh) * 128 + 2 * vcp] = ta[hh][0];
      tr[(vph * 4 + hh) * 128 + 2 * vcp + 1] = ta[hh][1];
    }
  }
  lds_barrier();
  if constexpr (LT) {
    long_tail<G, F32>(P, unit, s_q, s_ts, s_tailred, s_ptail, s_tm, s_cm, s_cs);
    lds_barrier();
  }
  if (tid < G * 128) {
    const int hh = tid >> 7, j = tid & 127;
    const float sv = (float)((double)(long long)s_vsum[hh][j] * (1.0 / 1073741824.0));   // 2^-30
    const float pv = (float)(s_psum[hh] * (1.0 / 134217728.0));                       // 2^-27
    float tail = 0.f;
#pragma unroll
    for (int q = 0; q < kPhases; ++q) {
      if constexpr (kRegTail) tail += tr[(q * 4 + hh) * 128 + j];
      else tail += s_tailred[q][hh][j];
    }
    const float pt = s_ptail[hh];
    // the visual sums are relative to the largest visual weight, the tail's
    // to its reference (top in the fused pass, the tail's own largest score
    // in the chunked one): each part is weighed by exp(its reference - top),
    // top the larger of the two (in the fused pass the tail's factor is 1 and
    // the visual one alpha)
    const float vx = s_vmax[hh], tx = s_tm[hh], top = fmaxf(vx, tx);
    const float al = n > 0 ? exp2f((vx - top) * kLog2e) : 0.f;
    const float at = exp2f((tx - top) * kLog2e);
    // (the tail terms are pinned, so that the fused multiply-adds are the
    // LDS-score kernel's, whose results equal these bit for bit)
    float o = at * tail, ptw = at * pt;
    asm volatile("" : "+v"(o), "+v"(ptw));
    if (n > 0) o += al * (s_vs[j] * sv + pv * s_vm[j]);
    o /= (al * pv + ptw);
    const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
    if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
    else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
  }
}

// ---------------------------------------------------------------------------
// b = 1 with the visual scores kept in LDS: no second read of the keys.
//
// The key tiles are read once.  Every head's scores (float32, the same values
// as in df_b1) wait in LDS for the value pass, which turns them into
// probabilities and digits in place: a tile's G x 128 scores and its G x 4 x
// 128 digit bytes take the same G x 512 bytes.  An Infinity-Cache re-read of
// a key tile costs nearly as much as the first read, so the saved re-read is
// about a third of the decode's traffic, and the value pass no longer
// recomputes scores (about 130 fewer VALU instructions per tile).
//
// One workgroup of 16 waves per CU (the scores of a 8192-token unit at G = 4
// take 128 KB of the 160 KB LDS) walks its units in turn; the first key
// tiles of its next unit are requested before the current unit's reduction.
// Arithmetic, operand layouts and summation order are those of df_b1, so the
// outputs equal df_b1's bit for bit.
constexpr int kWavesL = 16;
constexpr int kThreadsL = kWavesL * 64;
constexpr int kScoreBytes = 128 * 1024;       // G * n * 4 bytes at most

constexpr int kAheadK = 2;                   // key tiles in flight per wave
constexpr int kAheadV = 2;                   // value tiles in flight per wave

template <int G, bool F32>
__global__ void __launch_bounds__(kThreadsL, 1) dl_b1(Params P, int units) {
  const int n = P.n, T = P.T;
  const int ntiles = (n + kTile - 1) / kTile;
  const int R = n >> 5;
  const int nc = P.nc, Rc = nc >> 5;           // the code buffers' layout: nc tokens
  constexpr int kRegion = G * 128;            // words per tile: G x 128 scores, then G x 4 x 128 digit bytes

  __shared__ float s_q[4][128];
  __shared__ float s_qp[4][128];
  __shared__ double s_c0[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][4][32];   // fp6 digit codes: [head][plane][128 k slots]
  __shared__ float s_kc[4];                              // per head: sum of Q / 8 over the bit-3 channels
  __shared__ float s_ts[4][kMaxTail];
  __shared__ float s_red[kWavesL][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4], s_alpha[4];
  __shared__ float s_tailred[kThreads / 64][4][128];   // df_b1's eight token phases
  __shared__ unsigned long long s_vsum[4][128];
  __shared__ double s_psum[4];
  __shared__ int s_next[2];
  __shared__ float s_vs[128], s_vm[128];
  __shared__ double s_c0p[8];
  __shared__ float s_mqp[8];
  __shared__ __align__(16) uint32_t s_sc[kScoreBytes / 4];

  constexpr int kKtRounds = kPreTail / (4 * kWavesL);
  constexpr int kPhases = kThreads / 64;       // tail-value phases (threads < 512)

  int unit = blockIdx.x;
  const uint32_t* kc = n > 0 ? P.kc : g_pad;
  const uint32_t* vcb = n > 0 ? P.vc : g_pad;
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(g_pad);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(g_pad);
  // The helpers take the thread index: inside the unit loop it is an opaque
  // copy, so that per-lane constants are formed where they are used instead
  // of being hoisted out of the loop (and spilled).
  auto load_k = [&](int u, int tile, int t, uint4& w0, uint4& w1) {   // tokens past n: scores not used
    const int tok = max(min(tile * kTile + 8 * (t & 15), n - 8), 0);
    const uint4* src = reinterpret_cast<const uint4*>(kc + ((size_t)u * 4 + ((t & 63) >> 4)) * nc + tok);
    w0 = src[0];
    w1 = src[1];
  };
  auto load_v = [&](int u, int tile, int t, uint4& w0, uint4& w1) {
    const int row = max(min(tile * 4 + ((t & 63) >> 4), R - 1), 0);
    const uint4* src = reinterpret_cast<const uint4*>(vcb + ((size_t)u * Rc + row) * 128 + 8 * (t & 15));
    w0 = src[0];
    w1 = src[1];
  };
  // A unit's own inputs are requested before its first key tiles (vector
  // loads complete in order): at the start for the first unit, after the
  // value pass of the previous one for the others.  Threads >= 512 load a
  // copy they do not use.
  const float* ksb = n > 0 ? P.ks : reinterpret_cast<const float*>(g_pad);
  const float* kmb = n > 0 ? P.km : reinterpret_cast<const float*>(g_pad);
  const float* vsb = n > 0 ? P.vs : reinterpret_cast<const float*>(g_pad);
  const float* vmb = n > 0 ? P.vm : reinterpret_cast<const float*>(g_pad);
  float q_in, ks_in, km_in, vs_in, vm_in;
  uint4 ktp[kKtRounds][2];
  auto load_inputs = [&](int u, int t) {
    const int ub = u / P.Hkv, uh = u % P.Hkv;
    const int pj = t & 127, wv = t >> 6, tsub = (t & 63) >> 4, tcl = t & 15;
    const size_t prm = n > 0 ? (size_t)u * 128 + pj : (size_t)pj;
    q_in = ld_any(P.q, ((size_t)ub * P.Hq + uh * G + min((t & 511) >> 7, G - 1)) * 128 + pj, F32);
    ks_in = ksb[prm];
    km_in = kmb[prm];
    vs_in = vsb[prm];
    vm_in = vmb[prm];
#pragma unroll
    for (int r = 0; r < kKtRounds; ++r) {
      const int j = 4 * wv + tsub + 4 * kWavesL * r;
      const size_t e = ((size_t)u * T + max(min(j, T - 1), 0)) * 128 + 8 * tcl;
      if constexpr (F32) {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
        ktp[r][0] = src[0];
        ktp[r][1] = src[1];
      } else {
        ktp[r][0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(ktb) + e);
        ktp[r][1] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // key tiles in flight: kq[j] holds this wave's j-th next tile
  uint4 kq[kAheadK][2];
  {
    const int t = threadIdx.x;
    load_inputs(unit, t);
#pragma unroll
    for (int j = 0; j < kAheadK; ++j) load_k(unit, (t >> 6) + j * kWavesL, t, kq[j][0], kq[j][1]);
  }

  for (; unit < units; unit += gridDim.x) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, g4 = lane >> 4;
    const int rh = i16 >> 2, rp = i16 & 3;
    const int oh = lane >> 4;
    const int ph = tid >> 7, pj = tid & 127;   // prologue thread (tid < 512): head, channel
    const int tsub = lane >> 4, tcl = lane & 15;
    const int vcp = tid & 63, vph = wave;
    __builtin_amdgcn_s_setprio(3);
    const int b = unit / P.Hkv, h = unit % P.Hkv;
    if (tid == 0) {
      s_next[0] = kAheadK * kWavesL;
      s_next[1] = kAheadV * kWavesL;
    }
    if (tid < 4) {
      s_psum[tid] = 0.0;
      s_kc[tid] = 0.f;
    }
    for (int i = tid; i < 4 * 128; i += kThreadsL) (&s_vsum[0][0])[i] = 0ull;

    // ---- prologue (threads < 512: head ph, channel pj) ----------------------
    if (tid < 512) {
      const int hh = ph, j = pj;
      float qv = 0.f, qp = 0.f;
      double pr = 0.0;
      if (hh < G) {
        qv = P.sm * q_in;
        qp = qv * ks_in;
        pr = (double)qv * (double)km_in;
      }
      s_q[hh][j] = qv;
      s_qp[hh][j] = qp;
      if (hh == 0) {
        s_vs[j] = vs_in;
        s_vm[j] = vm_in;
      }
      float aq = fabsf(qp);
      pr = cqm::wave_sum(pr);
      aq = cqm::wave_max(aq);
      if (lane == 0) {
        s_c0p[wave] = pr;
        s_mqp[wave] = aq;
      }
    }
    lds_barrier();
    if (tid < 4) {
      const double c0 = s_c0p[2 * tid] + s_c0p[2 * tid + 1];
      const float mq = fmaxf(s_mqp[2 * tid], s_mqp[2 * tid + 1]);
      int F = 0;
      if (mq > 0.f) {
        const int e = ilogbf(mq);
        F = ldexpf(mq, 18 - e) > (float)kQMax ? 17 - e : 18 - e;
      }
      s_F[tid] = F;
      s_c0[tid] = c0;
    }
    lds_barrier();
    if (tid < 512) {                            // the digits of df_b1, formed the same way
      const int hh = tid >> 7, j = tid & 127;
      const float x = rintf(ldexpf(s_qp[hh][j], s_F[hh]));
      float d[4], r = x;
#pragma unroll
      for (int k = 3; k > 0; --k) {
        const float qk = rintf(r * (1.f / 31.f));
        d[k] = fmaf(-31.f, qk, r);
        r = qk;
      }
      d[0] = r;
      const int e = j & 31, Rf = (e >> 2) & 3, slot = 32 * (j >> 5) + 8 * Rf + 2 * (e & 3) + (e >> 4);
      const int mult = Rf == 0 ? 4 : (Rf == 1 ? 2 : (Rf == 2 ? 1 : -1));
      unsigned char* ad = reinterpret_cast<unsigned char*>(&s_adig[hh][0][0]);
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) ad[pl * 128 + slot] = (unsigned char)enc6((int)d[pl] * mult);
      float kcs = Rf == 3 ? 0.125f * x : 0.f;
      kcs = cqm::wave_sum(kcs);
      if (lane == 0 && hh < G) atomicAdd(&s_kc[hh], kcs);
    }
    lds_barrier();

    // ---- text tail scores -----------------------------------------------------
    {
      const int sub = tsub, cl = tcl;
      auto tail_scores = [&](int j, const float (&kf)[8]) {
        float sc[G];                                   // the heads' sums side by side
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          sc[hh] = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) sc[hh] = fmaf(s_q[hh][8 * cl + c], kf[c], sc[hh]);
        }
        cqm::row_sum16x(sc);
        if (cl == 0 && j < T) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) s_ts[hh][j] = sc[hh];
        }
      };
#pragma unroll
      for (int r = 0; r < kKtRounds; ++r) {
        float kf[8];
        if constexpr (F32) {
          kf[0] = __uint_as_float(ktp[r][0].x); kf[1] = __uint_as_float(ktp[r][0].y);
          kf[2] = __uint_as_float(ktp[r][0].z); kf[3] = __uint_as_float(ktp[r][0].w);
          kf[4] = __uint_as_float(ktp[r][1].x); kf[5] = __uint_as_float(ktp[r][1].y);
          kf[6] = __uint_as_float(ktp[r][1].z); kf[7] = __uint_as_float(ktp[r][1].w);
        } else {
          const uint32_t hw[4] = {ktp[r][0].x, ktp[r][0].y, ktp[r][0].z, ktp[r][0].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
          }
        }
        tail_scores(4 * wave + 4 * kWavesL * r + sub, kf);
      }
      constexpr int kXR = F32 ? 1 : kXRounds;
    // rounds past kPreTail tokens, kXR at a time: their keys are read as
      // the prefetched ones (clamped rows, whole 16-byte pieces, no branch), the
      // rounds' loads in flight together
      for (int j0 = 4 * wave + 4 * kWavesL * kKtRounds; j0 < T; j0 += 4 * kWavesL * kXR) {
        uint4 kr[kXR][2];
#pragma unroll
        for (int x = 0; x < kXR; ++x) {
          const size_t e = ((size_t)unit * T + max(min(j0 + 4 * kWavesL * x + sub, T - 1), 0)) * 128 + 8 * cl;
          if constexpr (F32) {
            const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
            kr[x][0] = cqd::ld_nt(src);
            kr[x][1] = cqd::ld_nt(src + 1);
          } else {
            kr[x][0] = cqd::ld_nt(reinterpret_cast<const __half*>(ktb) + e);
            kr[x][1] = make_uint4(0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int x = 0; x < kXR; ++x) {
          float kf[8];
          if constexpr (F32) {
            kf[0] = __uint_as_float(kr[x][0].x); kf[1] = __uint_as_float(kr[x][0].y);
            kf[2] = __uint_as_float(kr[x][0].z); kf[3] = __uint_as_float(kr[x][0].w);
            kf[4] = __uint_as_float(kr[x][1].x); kf[5] = __uint_as_float(kr[x][1].y);
            kf[6] = __uint_as_float(kr[x][1].z); kf[7] = __uint_as_float(kr[x][1].w);
          } else {
            const uint32_t hw[4] = {kr[x][0].x, kr[x][0].y, kr[x][0].z, kr[x][0].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
              kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
            }
          }
          tail_scores(j0 + 4 * kWavesL * x + sub, kf);          // rows past T: scores not stored
        }
      }
    }

    // ---- key pass: scores into LDS, their min and max --------------------------
    v8i kdig = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    {
      const uint4* src = reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
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
      if (rh < G) kdig = v8i{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], 0, 0};
    }
    float vmin = INFINITY, vmax = -INFINITY;
    // Slot j of the ring holds the key tile tq[j]; the slots are used in
    // turn, and a used slot is refilled in place with the next dealt tile.
    // (Rotating the registers instead would move a tile whose load is still
    // in flight, and the move waits for it: no look-ahead would be left.)
    int tq[kAheadK];
#pragma unroll
    for (int j = 0; j < kAheadK; ++j) tq[j] = wave + j * kWavesL;
    uint32_t kc2 = 0x22222222u;                // in a register for sign_fields
    asm volatile("" : "+v"(kc2));
    auto key_tile = [&](uint4& s0, uint4& s1, int& slot_tile) {
      const int tile = slot_tile;
      int nxt = 0;
      if (lane == 0) nxt = atomicAdd(&s_next[0], 1);
      nxt = __builtin_amdgcn_readfirstlane(nxt);
      const bool ok = tile * kTile + 8 * i16 < n;
      const uint32_t wd[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float st[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {            // df_b1's scores, formed the same way
        const uint32_t w = wd[m];
        const v8i bq{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u),
                     (int)sign_fields(w, kc2), 0, 0, 0, 0};
        const v4f a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kdig, bq, v4f{0.f, 0.f, 0.f, 0.f}, 2, 4, 0,
                                                                        127, 0, 127);
        st[m] = fmaf(fmaf(fmaf(a[0], 31.f, a[1]), 31.f, a[2]), 31.f, a[3]);
      }
      if (oh < G) {
        float4* dst = reinterpret_cast<float4*>(&s_sc[tile * kRegion + oh * 128 + 8 * i16]);
        dst[0] = make_float4(st[0], st[1], st[2], st[3]);
        dst[1] = make_float4(st[4], st[5], st[6], st[7]);
      }
      float tmin = st[0], tmax = st[0];
#pragma unroll
      for (int m = 1; m < 8; ++m) {
        tmin = fminf(tmin, st[m]);
        tmax = fmaxf(tmax, st[m]);
      }
      if (ok) {
        vmin = fminf(vmin, tmin);
        vmax = fmaxf(vmax, tmax);
      }
      asm volatile("" : "+v"(vmin), "+v"(vmax));
      // the slot is refilled once its tile is used: no register copy of a tile in flight
      slot_tile = nxt;
      load_k(unit, nxt, tid, s0, s1);
    };
    for (;;) {
#pragma unroll
      for (int j = 0; j < kAheadK; ++j) {
        if (tq[j] >= ntiles) goto keys_done;
        key_tile(kq[j][0], kq[j][1], tq[j]);
      }
    }
  keys_done:
    // value tiles and the first tail values, before the statistics
    uint4 vq[kAheadV][2];
#pragma unroll
    for (int j = 0; j < kAheadV; ++j) load_v(unit, wave + j * kWavesL, tid, vq[j][0], vq[j][1]);
    uint32_t vtr[kPreTail / kPhases][F32 ? 2 : 1];
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      const size_t e = ((size_t)unit * T + max(min((vph & 7) + kPhases * i, T - 1), 0)) * 128 + 2 * vcp;
      if constexpr (F32) {
        const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
        vtr[i][0] = x.x;
        vtr[i][F32 ? 1 : 0] = x.y;
      } else {
        vtr[i][0] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e);
      }
    }
    // ---- statistics ---------------------------------------------------------
    vmin = cqm::row_min16(vmin);
    vmax = cqm::row_max16(vmax);
    if ((lane & 15) == 0) {
      s_red[wave][oh][0] = vmin;
      s_red[wave][oh][1] = vmax;
    }
    lds_barrier();
    if (wave < G) {
      const int hh = wave;
      float m = lane < kWavesL ? s_red[lane][hh][0] : INFINITY;
      float M = lane < kWavesL ? s_red[lane][hh][1] : -INFINITY;
      float tmax = -INFINITY;
      for (int j = lane; j < T; j += 64) tmax = fmaxf(tmax, s_ts[hh][j]);
      m = cqm::wave_min(m);
      M = cqm::wave_max(M);
      tmax = cqm::wave_max(tmax);
      const double scale = ldexp(4.0, -s_F[hh]);   // the statistics of df_b1, computed the same way
      const double c0 = s_c0[hh] + (double)s_kc[hh] * scale;
      double lam = scale, mu = -scale * (double)M, vis_max = (double)M * scale + c0;
      if (P.calib_on && n > 0) {
        // (the parameters pass through opaque copies: converted here rather
        // than held in registers across the unit loop)
        float alo = P.a_lo, clo = P.c_lo, ahi = P.a_hi, chi = P.c_hi;
        asm volatile("" : "+s"(alo), "+s"(clo), "+s"(ahi), "+s"(chi));
        const double mr = (double)m * scale + c0, Mr = (double)M * scale + c0;
        const double t_lo = (double)alo * mr + (double)clo, t_hi = (double)ahi * Mr + (double)chi;
        vis_max = M > m ? fmax(t_lo, t_hi) : t_lo;
        lam = M > m ? (t_hi - t_lo) / ((double)(M - m) * scale) * scale : 0.0;
        mu = t_lo - vis_max - lam * (double)m;
      }
      const float top = fmaxf(n > 0 ? (float)vis_max : -INFINITY, tmax);
      if (lane == 0) {
        s_lam[hh] = (float)(lam * 1.4426950408889634);
        s_mu[hh] = (float)(mu * 1.4426950408889634);
        s_alpha[hh] = n > 0 ? exp2f(((float)vis_max - top) * kLog2e) : 0.f;
      }
      float ptl = 0.f;
      for (int j = lane; j < T; j += 64) {
        const float pj2 = exp2f((s_ts[hh][j] - top) * kLog2e);
        s_ts[hh][j] = pj2;
        ptl += pj2;
      }
      ptl = cqm::wave_sum(ptl);
      if (lane == 0) s_ptail[hh] = ptl;
    }
    lds_barrier();
    if (tid < kThreads) {                       // text-tail values, df_b1's phases
      float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < kPreTail / kPhases; ++i) {
        // (a select, not a branch: a token past T weighs 0, and the heads'
        // weights of every token are read together)
        const int t = vph + kPhases * i;
        const bool tok = t < T;
        float v0, v1;
        if constexpr (F32) {
          v0 = __uint_as_float(vtr[i][0]);
          v1 = __uint_as_float(vtr[i][F32 ? 1 : 0]);
        } else {
          v0 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] & 0xFFFF)));
          v1 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] >> 16)));
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float w = tok ? s_ts[hh][t] : 0.f;
          ta[hh][0] = fmaf(w, v0, ta[hh][0]);
          ta[hh][1] = fmaf(w, v1, ta[hh][1]);
        }
      }
      constexpr int kXT = F32 ? 4 : kXTokens;
    // tokens past kPreTail, kXT at a time: loads in flight together
      // (clamped rows, no branch); a token past T weighs 0
      for (int t0 = kPreTail + vph; t0 < T; t0 += kPhases * kXT) {
        uint32_t vx[kXT][F32 ? 2 : 1];
#pragma unroll
        for (int x = 0; x < kXT; ++x) {
          const size_t e = ((size_t)unit * T + max(min(t0 + kPhases * x, T - 1), 0)) * 128 + 2 * vcp;
          if constexpr (F32) {
            const uint2 w2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
            vx[x][0] = w2.x;
            vx[x][F32 ? 1 : 0] = w2.y;
          } else {
            vx[x][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e));
          }
        }
#pragma unroll
        for (int x = 0; x < kXT; ++x) {
          const int t = t0 + kPhases * x;
          const bool tok = t < T;
          float v0, v1;
          if constexpr (F32) {
            v0 = __uint_as_float(vx[x][0]);
            v1 = __uint_as_float(vx[x][F32 ? 1 : 0]);
          } else {
            v0 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] & 0xFFFF)));
            v1 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] >> 16)));
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const float w = tok ? s_ts[hh][min(t, kMaxTail - 1)] : 0.f;
            ta[hh][0] = fmaf(w, v0, ta[hh][0]);
            ta[hh][1] = fmaf(w, v1, ta[hh][1]);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        s_tailred[vph][hh][2 * vcp] = ta[hh][0];
        s_tailred[vph][hh][2 * vcp + 1] = ta[hh][1];
      }
    }

    // ---- value pass -------------------------------------------------------------
    __builtin_amdgcn_s_setprio(0);
    const float lam2 = s_lam[oh < G ? oh : 0], mu2 = s_mu[oh < G ? oh : 0];
    const int wt0 = bit_weight(8 * i16), wt1 = bit_weight(8 * i16 + 4);
    v4i vacc[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
    constexpr int kFlushTiles = 256;
    auto flush = [&]() {
      if (oh < G) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const long long sv = (long long)vacc[ct][0] + 256ll * vacc[ct][1] + 65536ll * vacc[ct][2] +
                               16777216ll * vacc[ct][3];
          atomicAdd(&s_vsum[oh][8 * i16 + ct], (unsigned long long)sv);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
    };
    int wtiles = 0;
    double psum = 0.0;
    int tv[kAheadV];
#pragma unroll
    for (int j = 0; j < kAheadV; ++j) tv[j] = wave + j * kWavesL;
    auto value_tile = [&](uint4& s0, uint4& s1, int& slot_tile) {
      const int tile = slot_tile;
      int nxt = 0;
      if (lane == 0) nxt = atomicAdd(&s_next[1], 1);
      nxt = __builtin_amdgcn_readfirstlane(nxt);

      uint32_t* reg = &s_sc[tile * kRegion];
      const bool ok = oh < G && tile * kTile + 8 * i16 < n;
      const float mu_t = ok ? mu2 + 27.f : -INFINITY;   // the exponent of p 2^27, as in df_b1
      float st[8];
      {
        const float4* src = reinterpret_cast<const float4*>(reg + (oh < G ? oh : 0) * 128 + 8 * i16);
        const float4 a = src[0], c = src[1];
        st[0] = a.x; st[1] = a.y; st[2] = a.z; st[3] = a.w;
        st[4] = c.x; st[5] = c.y; st[6] = c.z; st[7] = c.w;
      }
      uint32_t fb[8], ptile = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t Pm = cqm::p_fixed_exp2(fmaf(st[m], lam2, mu_t));
        ptile += Pm;
        fb[m] = cqm::sdigits(Pm << (m < 4 ? wt0 : wt1));
      }
      psum += (double)ptile;
      wave_sync_lds();                          // every lane has read its scores of the tile
      unsigned char* pd = reinterpret_cast<unsigned char*>(reg);
      if (oh < G) {
        uint32_t d[2][4];
        transpose_bytes(fb[0], fb[1], fb[2], fb[3], d[0][0], d[0][1], d[0][2], d[0][3]);
        transpose_bytes(fb[4], fb[5], fb[6], fb[7], d[1][0], d[1][1], d[1][2], d[1][3]);
#pragma unroll
        for (int pl = 0; pl < 4; ++pl)
          *reinterpret_cast<uint2*>(pd + (oh * 4 + pl) * 128 + 8 * i16) = make_uint2(d[0][pl], d[1][pl]);
      }
      wave_sync_lds();
      v4i av0 = {0, 0, 0, 0}, av1 = {0, 0, 0, 0};
      if (rh < G) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(pd + (rh * 4 + rp) * 128 + 32 * g4);
        const uint4 x1 = *reinterpret_cast<const uint4*>(pd + (rh * 4 + rp) * 128 + 32 * g4 + 16);
        av0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
        av1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
      const uint32_t vwd[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        vacc[ct] = mfma(av0, bits_lo(vwd[ct]), vacc[ct]);
        vacc[ct] = mfma(av1, bits_hi(vwd[ct]), vacc[ct]);
      }
      slot_tile = nxt;
      load_v(unit, nxt, tid, s0, s1);
      if (++wtiles == kFlushTiles) {
        flush();
        wtiles = 0;
      }
    };
    for (;;) {
#pragma unroll
      for (int j = 0; j < kAheadV; ++j) {
        if (tv[j] >= ntiles) goto values_done;
        value_tile(vq[j][0], vq[j][1], tv[j]);
      }
    }
  values_done:
    // the next unit's inputs and first key tiles, requested before this
    // unit's reduction (past the last unit: the last one again, unused)
    {
      const int un = min(unit + (int)gridDim.x, units - 1);
      load_inputs(un, tid);
#pragma unroll
      for (int j = 0; j < kAheadK; ++j) load_k(un, wave + j * kWavesL, tid, kq[j][0], kq[j][1]);
    }

    // ---- combine planes, reduce over waves --------------------------------------
    __builtin_amdgcn_s_setprio(1);
    flush();
    psum = cqm::row_sum16(psum);
    if ((lane & 15) == 0 && oh < G) atomicAdd(&s_psum[oh], psum);
    lds_barrier();
    if (tid < G * 128) {
      const int hh = tid >> 7, j = tid & 127;
      const float sv = (float)((double)(long long)s_vsum[hh][j] * (1.0 / 1073741824.0));
      const float pv = (float)(s_psum[hh] * (1.0 / 134217728.0));
      float tail = 0.f;
#pragma unroll
      for (int q = 0; q < kPhases; ++q) tail += s_tailred[q][hh][j];
      const float ptt = s_ptail[hh];
      const float al = s_alpha[hh];
      float o = tail;
      if (n > 0) o += al * (s_vs[j] * sv + pv * s_vm[j]);
      o /= (al * pv + ptt);
      const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
      if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
      else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
    }
    lds_barrier();                              // LDS is reused by the next unit
  }
}

// b in {2, 4, 8}: the same two passes over b-bit codes.  A tile is 128/b
// tokens, so that on either side a lane reads 8 words per tile:
//   keys: lane (i16, g4) holds word planes b g4 .. b g4 + b - 1 (channels
//     32 g4 .. +31, the A digits of the 1-bit kernel unchanged) of tokens
//     TPL i16 .. +TPL-1, TPL = 8/b; a plane word spreads into byte-sized codes
//     with one shift and mask per 4 codes;
//   values: lane (i16, g4) holds V word row 4 tile + g4 (E = 32/b tokens) of
//     channels 8 i16 .. +7; for b = 4 and 8 a lane's 16 contraction bytes are
//     only half / a quarter used (the matrix cores have the headroom).
// For b = 8 a code (0..255) is not a signed byte: it enters as its low nibble
// plus twice (8 x high nibble), three products into the same accumulator.
// The key dot product can exceed 32 bits for b >= 4 and is summed in 64 bits.
// the key tiles whose scores stay in LDS: as many as two workgroups per CU
// leave room for, or (ALL, for launches of at most one workgroup per CU) the
// first kAllKeepTokens tokens' (108 KB of scores: with the kernel's other
// LDS, 152 to 158 KB of the CU's 160 KB)
constexpr int kAllKeepTokens = 6912;
template <int BITS, bool ALL>
constexpr int keep_tiles() {
  return ALL ? kAllKeepTokens / (128 / BITS) : (BITS == 2 ? 28 : (BITS == 4 ? 66 : 140));
}

template <int BITS, int G, bool F32, bool LT, bool ALL = false>
__global__ void __launch_bounds__(kThreads, ALL ? 2 : 4) df_bn(Params P) {
  constexpr int E = 32 / BITS;                  // codes per word
  constexpr int TB = 4 * E;                     // tokens per tile
  constexpr int TPL = TB / 16;                  // key tokens per lane per tile
  constexpr int W = 4 * BITS;                   // key word planes per token
  constexpr uint32_t kNib = 0x0F0F0F0Fu;
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T;
  const int Tf = LT ? kMaxTail : T;            // the text tail in the fused pass (the rest chunked at the end)
  const int tiles = (n + TB - 1) / TB;
  const int R = n / E;
  const int nc = P.nc, Rc = nc / E;            // the code buffers' layout: nc tokens

  __shared__ float s_q[4][128];
  __shared__ float s_qp[4][128];
  __shared__ double s_c0[4];
  __shared__ float s_inv2f[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][3][32];
  __shared__ __align__(16) uint32_t s_pdig[kWaves][4][4][TB / 4];   // V-side A digits: [head][plane][TB bytes]
  __shared__ float s_ts[4][kMaxTail];
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4], s_alpha[4];
  __shared__ float s_vmax[4], s_tm[4], s_cm[4], s_cs[4];
  __shared__ float s_tailred[kThreads / 64][4][128];
  __shared__ float s_vred[kWaves][4][128];
  __shared__ float s_psum[kWaves][4];
  // the scores of the unit's first kKeepN tiles stay in LDS from the key pass
  // to the value pass ([tile][lane][token]), so those key tiles are read once
  // (as in df_b1; the rest of the LDS two workgroups per CU leave, or with
  // ALL the tiles of the first kAllKeepTokens tokens)
  constexpr int kKeepN = keep_tiles<BITS, ALL>();
  __shared__ __align__(16) float s_keepn[kKeepN][64][TPL];

  const int i16 = lane & 15, g4 = lane >> 4;
  const int rh = i16 >> 2, rp = i16 & 3;
  const int oh = lane >> 4;
  const uint32_t* kc = n > 0 ? P.kc : g_pad;
  const uint32_t* vcb = n > 0 ? P.vc : g_pad;
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(g_pad);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(g_pad);
  // Key tiles are read with buffer loads (one descriptor per unit): a tile
  // past the last, or a kept one in the value pass, reads out of range, which
  // returns zeros without any traffic.  Tokens past n: scores not used.
  const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + (n > 0 ? (size_t)unit * W * nc : 0)), (short)0,
                                                    n > 0 ? W * nc * 4 : 0, kRsrcFlags);
  auto load_k = [&](int tile, uint32_t (&w)[8]) {
    const uint32_t toff = tile < tiles ? (uint32_t)(tile * TB) * 4u : 0x80000000u;
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = 0u;
#pragma unroll
    for (int p = 0; p < BITS; ++p) {
      const uint32_t off = (uint32_t)((BITS * g4 + p) * nc + TPL * i16) * 4u + toff;
      if constexpr (TPL == 4) {
        const uint4 x = ld_buf(rk, off);
        w[4 * p] = x.x; w[4 * p + 1] = x.y; w[4 * p + 2] = x.z; w[4 * p + 3] = x.w;
      } else if constexpr (TPL == 2) {
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)off, 0, 0);
        w[2 * p] = x.x; w[2 * p + 1] = x.y;
      } else {
        w[p] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)off, 0, 0);
      }
    }
  };
  uint32_t kn[8];
  load_k(wave, kn);

  // ---- prologue: post-scaled query, fixed-point digits -------------------
  __shared__ double s_c0p[8];
  __shared__ float s_mqp[8];
  {                                             // thread: head tid / 128, channel tid % 128
    const int hh = tid >> 7, j = tid & 127;
    float qv = 0.f, qp = 0.f;
    double pr = 0.0;
    if (hh < G) {
      qv = P.sm * ld_any(P.q, ((size_t)b * P.Hq + h * G + hh) * 128 + j, F32);
      qp = qv * P.ks[(size_t)unit * 128 + j];
      pr = (double)qv * (double)P.km[(size_t)unit * 128 + j];
    }
    s_q[hh][j] = qv;
    s_qp[hh][j] = qp;
    float aq = fabsf(qp);
    pr = cqm::wave_sum(pr);
    aq = cqm::wave_max(aq);
    if (lane == 0) {
      s_c0p[wave] = pr;
      s_mqp[wave] = aq;
    }
  }
  lds_barrier();
  if (tid < 4) {
    const double c0 = s_c0p[2 * tid] + s_c0p[2 * tid + 1];
    const float mq = fmaxf(s_mqp[2 * tid], s_mqp[2 * tid + 1]);
    int F = 0;
    if (mq > 0.f) F = 21 - ilogbf(mq);
    s_F[tid] = F;
    s_inv2f[tid] = ldexpf(1.f, -F);
    s_c0[tid] = c0;
  }
  lds_barrier();
  {
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
  lds_barrier();

  // ---- pass 1: visual scores, their min and max --------------------------
  v4i ak0 = {0, 0, 0, 0}, ak1 = {0, 0, 0, 0};
  if (rp < 3 && rh < G) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
    const uint4 x1 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4 + 4]);
    ak0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
    ak1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  const float inv2f = s_inv2f[oh < G ? oh : 0];
  const float c0f = (float)s_c0[oh < G ? oh : 0];
  // score of key token m of this lane's TPL tokens (head oh)
  auto score = [&](const uint32_t (&w)[8], int m) -> float {
    v4i acc = {0, 0, 0, 0};
    if constexpr (BITS == 2) {
      const uint32_t w0 = w[m], w1 = w[TPL + m];
      acc = mfma(ak0, v4i{(int)(w0 & 0x03030303u), (int)((w0 >> 2) & 0x03030303u), (int)((w0 >> 4) & 0x03030303u),
                          (int)((w0 >> 6) & 0x03030303u)}, acc);
      acc = mfma(ak1, v4i{(int)(w1 & 0x03030303u), (int)((w1 >> 2) & 0x03030303u), (int)((w1 >> 4) & 0x03030303u),
                          (int)((w1 >> 6) & 0x03030303u)}, acc);
    } else if constexpr (BITS == 4) {
      const uint32_t w0 = w[m], w1 = w[TPL + m], w2 = w[2 * TPL + m], w3 = w[3 * TPL + m];
      acc = mfma(ak0, v4i{(int)(w0 & kNib), (int)((w0 >> 4) & kNib), (int)(w1 & kNib), (int)((w1 >> 4) & kNib)}, acc);
      acc = mfma(ak1, v4i{(int)(w2 & kNib), (int)((w2 >> 4) & kNib), (int)(w3 & kNib), (int)((w3 >> 4) & kNib)}, acc);
    } else {
      const v4i lo0{(int)(w[0] & kNib), (int)(w[1] & kNib), (int)(w[2] & kNib), (int)(w[3] & kNib)};
      const v4i hi0{(int)((w[0] >> 1) & 0x78787878u), (int)((w[1] >> 1) & 0x78787878u),
                    (int)((w[2] >> 1) & 0x78787878u), (int)((w[3] >> 1) & 0x78787878u)};
      const v4i lo1{(int)(w[4] & kNib), (int)(w[5] & kNib), (int)(w[6] & kNib), (int)(w[7] & kNib)};
      const v4i hi1{(int)((w[4] >> 1) & 0x78787878u), (int)((w[5] >> 1) & 0x78787878u),
                    (int)((w[6] >> 1) & 0x78787878u), (int)((w[7] >> 1) & 0x78787878u)};
      acc = mfma(ak0, lo0, acc);
      acc = mfma(ak0, hi0, acc);
      acc = mfma(ak0, hi0, acc);
      acc = mfma(ak1, lo1, acc);
      acc = mfma(ak1, hi1, acc);
      acc = mfma(ak1, hi1, acc);
    }
    const long long dot = (long long)acc[0] + 256LL * acc[1] + 65536LL * acc[2];
    float s = fmaf((float)dot, inv2f, c0f);
    asm volatile("" : "+v"(s));
    return s;
  };
  float vmin = INFINITY, vmax = -INFINITY;
  for (int tile = wave; tile < tiles; tile += kWaves) {
    uint32_t kw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) kw[q] = kn[q];
    load_k(tile + kWaves, kn);
    // n % 32 == 0: this lane's TPL tokens are all valid or none
    const bool ok = tile * TB + TPL * i16 < n;
    float sk[TPL];
#pragma unroll
    for (int m = 0; m < TPL; ++m) {
      const float s = score(kw, m);
      sk[m] = s;
      if (ok) {
        vmin = fminf(vmin, s);
        vmax = fmaxf(vmax, s);
      }
    }
    if (tile < kKeepN) {
#pragma unroll
      for (int m = 0; m < TPL; ++m) s_keepn[tile][lane][m] = sk[m];
    }
  }
  // second pass: first key and value tiles requested now (the key base goes
  // through an opaque copy so that the compiler re-reads instead of keeping
  // first-pass values alive)
  // tail keys, then the first key and value tiles of the second pass, then
  // tail values, in the order they are needed (loads complete in order)
  const int tsub = lane >> 4, tcl = lane & 15;
  constexpr int kKtRounds = kPreTail / (4 * kWaves);
  uint4 ktp[kKtRounds][2];
#pragma unroll
  for (int r = 0; r < kKtRounds; ++r) {
    const int j = 4 * wave + tsub + 4 * kWaves * r;   // rows past T: scores not stored
    const size_t e = ((size_t)unit * T + max(min(j, T - 1), 0)) * 128 + 8 * tcl;
    if constexpr (F32) {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
      ktp[r][0] = src[0];
      ktp[r][1] = src[1];
    } else {
      ktp[r][0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(ktb) + e);
      ktp[r][1] = make_uint4(0, 0, 0, 0);
    }
  }
  asm("" : "+s"(kc));
  load_k(wave < kKeepN ? tiles : wave, kn);     // a kept tile: an out-of-range read, no traffic
  auto load_v = [&](int tile, uint32_t (&w)[8]) {   // rows past the last: p = 0 (as in df_b1)
    const int row = max(min(tile * 4 + g4, R - 1), 0);
    const uint4* src = reinterpret_cast<const uint4*>(vcb + ((size_t)unit * Rc + row) * 128 + 8 * i16);
    const uint4 x0 = src[0], x1 = src[1];
    w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
    w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
  };
  uint32_t vn[8];
  load_v(wave, vn);
  // tail values: thread (channel pair vcp, phase vph) holds channels 2 vcp,
  // 2 vcp + 1 of tokens vph + kPhases i, as raw bits converted where used
  constexpr int kPhases = kThreads / 64;
  const int vcp = tid & 63, vph = tid >> 6;
  uint32_t vtr[kPreTail / kPhases][F32 ? 2 : 1];
#pragma unroll
  for (int i = 0; i < kPreTail / kPhases; ++i) {
    const size_t e = ((size_t)unit * T + max(min(vph + kPhases * i, T - 1), 0)) * 128 + 2 * vcp;
    if constexpr (F32) {
      const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
      vtr[i][0] = x.x;
      vtr[i][F32 ? 1 : 0] = x.y;
    } else {
      vtr[i][0] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e);
    }
  }
  // ---- text tail scores ---------------------------------------------------
  // The prefetched rounds run straight (no early exit: every lane's rows were
  // loaded, in bounds, and rows past T are not stored); rounds past kPreTail
  // tokens load as they go.
  {
    const int sub = tsub, cl = tcl;
    auto tail_scores = [&](int j, const float (&kf)[8]) {
      float sc[G];                                   // the heads' sums side by side
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        sc[hh] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) sc[hh] = fmaf(s_q[hh][8 * cl + c], kf[c], sc[hh]);
      }
      cqm::row_sum16x(sc);
      if (cl == 0 && j < Tf) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s_ts[hh][j] = sc[hh];
      }
    };
#pragma unroll
    for (int r = 0; r < kKtRounds; ++r) {
      float kf[8];
      if constexpr (F32) {
        kf[0] = __uint_as_float(ktp[r][0].x); kf[1] = __uint_as_float(ktp[r][0].y);
        kf[2] = __uint_as_float(ktp[r][0].z); kf[3] = __uint_as_float(ktp[r][0].w);
        kf[4] = __uint_as_float(ktp[r][1].x); kf[5] = __uint_as_float(ktp[r][1].y);
        kf[6] = __uint_as_float(ktp[r][1].z); kf[7] = __uint_as_float(ktp[r][1].w);
      } else {
        const uint32_t hw[4] = {ktp[r][0].x, ktp[r][0].y, ktp[r][0].z, ktp[r][0].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
          kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
        }
      }
      tail_scores(4 * wave + 4 * kWaves * r + sub, kf);
    }
    constexpr int kXR = F32 ? 1 : kXRounds;
    // rounds past kPreTail tokens, kXR at a time: their keys are read as
    // the prefetched ones (clamped rows, whole 16-byte pieces, no branch), the
    // rounds' loads in flight together
    for (int j0 = 4 * wave + 4 * kWaves * kKtRounds; j0 < Tf; j0 += 4 * kWaves * kXR) {
      uint4 kr[kXR][2];
#pragma unroll
      for (int x = 0; x < kXR; ++x) {
        const size_t e = ((size_t)unit * T + max(min(j0 + 4 * kWaves * x + sub, T - 1), 0)) * 128 + 8 * cl;
        if constexpr (F32) {
          const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(ktb) + e);
          kr[x][0] = cqd::ld_nt(src);
          kr[x][1] = cqd::ld_nt(src + 1);
        } else {
          kr[x][0] = cqd::ld_nt(reinterpret_cast<const __half*>(ktb) + e);
          kr[x][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < kXR; ++x) {
        float kf[8];
        if constexpr (F32) {
          kf[0] = __uint_as_float(kr[x][0].x); kf[1] = __uint_as_float(kr[x][0].y);
          kf[2] = __uint_as_float(kr[x][0].z); kf[3] = __uint_as_float(kr[x][0].w);
          kf[4] = __uint_as_float(kr[x][1].x); kf[5] = __uint_as_float(kr[x][1].y);
          kf[6] = __uint_as_float(kr[x][1].z); kf[7] = __uint_as_float(kr[x][1].w);
        } else {
          const uint32_t hw[4] = {kr[x][0].x, kr[x][0].y, kr[x][0].z, kr[x][0].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = __half2float(__ushort_as_half((unsigned short)(hw[c] & 0xFFFF)));
            kf[2 * c + 1] = __half2float(__ushort_as_half((unsigned short)(hw[c] >> 16)));
          }
        }
        tail_scores(j0 + 4 * kWaves * x + sub, kf);          // rows past T: scores not stored
      }
    }
  }
  // ---- min / max of every head's visual scores ---------------------------
  vmin = cqm::row_min16(vmin);
  vmax = cqm::row_max16(vmax);
  if ((lane & 15) == 0) {
    s_red[wave][oh][0] = vmin;
    s_red[wave][oh][1] = vmax;
  }
  lds_barrier();
  if (wave < G) {                               // wave hh settles head hh
    const int hh = wave;
    float m = lane < kWaves ? s_red[lane][hh][0] : INFINITY;
    float M = lane < kWaves ? s_red[lane][hh][1] : -INFINITY;
    float tmax = -INFINITY;
    for (int j = lane; j < Tf; j += 64) tmax = fmaxf(tmax, s_ts[hh][j]);
    m = cqm::wave_min(m);
    M = cqm::wave_max(M);
    tmax = cqm::wave_max(tmax);
    float lam = 1.f, mu = 0.f, vis_max = M;
    if (P.calib_on && n > 0) {
      const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
      lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
      mu = t_lo - lam * m;
      // the largest value of g: the larger end of [t_lo, t_hi], or t_lo
      // when every score is the same (g is then the constant t_lo)
      vis_max = M > m ? fmaxf(t_lo, t_hi) : t_lo;
    }
    const float top = fmaxf(n > 0 ? vis_max : -INFINITY, tmax);
    if (lane == 0) {
      // visual weights relative to the largest one: p = 2^(s * lam' + mu');
      // alpha = its weight relative to the softmax reference
      s_lam[hh] = lam * kLog2e;
      s_mu[hh] = (mu - vis_max) * kLog2e;
      s_alpha[hh] = n > 0 ? exp2f((vis_max - top) * kLog2e) : 0.f;
      s_vmax[hh] = n > 0 ? vis_max : -INFINITY;
      s_tm[hh] = top;
    }
    // tail probabilities (in place) and their sum
    float pt = 0.f;
    for (int j = lane; j < Tf; j += 64) {
      const float pj = exp2f((s_ts[hh][j] - top) * kLog2e);
      s_ts[hh][j] = pj;
      pt += pj;
    }
    pt = cqm::wave_sum(pt);
    if (lane == 0) s_ptail[hh] = pt;
  }
  lds_barrier();
  // text-tail values: thread (channel pair vcp, phase vph) sums the tail
  // tokens vph + kPhases i for every head, the first kPreTail from the loads above
  {
    float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      // (a select, not a branch: a token past T weighs 0, and the heads'
      // weights of every token are read together)
      const int t = vph + kPhases * i;
      const bool tok = t < Tf;
      float v0, v1;
      if constexpr (F32) {
        v0 = __uint_as_float(vtr[i][0]);
        v1 = __uint_as_float(vtr[i][F32 ? 1 : 0]);
      } else {
        v0 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] & 0xFFFF)));
        v1 = __half2float(__ushort_as_half((unsigned short)(vtr[i][0] >> 16)));
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float w = tok ? s_ts[hh][t] : 0.f;
        ta[hh][0] = fmaf(w, v0, ta[hh][0]);
        ta[hh][1] = fmaf(w, v1, ta[hh][1]);
      }
    }
    constexpr int kXT = F32 ? 4 : kXTokens;
    // tokens past kPreTail, kXT at a time: loads in flight together
    // (clamped rows, no branch); a token past T weighs 0
    for (int t0 = kPreTail + vph; t0 < Tf; t0 += kPhases * kXT) {
      uint32_t vx[kXT][F32 ? 2 : 1];
#pragma unroll
      for (int x = 0; x < kXT; ++x) {
        const size_t e = ((size_t)unit * T + max(min(t0 + kPhases * x, T - 1), 0)) * 128 + 2 * vcp;
        if constexpr (F32) {
          const uint2 w2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(vtb) + e);
          vx[x][0] = w2.x;
          vx[x][F32 ? 1 : 0] = w2.y;
        } else {
          vx[x][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e));
        }
      }
#pragma unroll
      for (int x = 0; x < kXT; ++x) {
        const int t = t0 + kPhases * x;
        const bool tok = t < Tf;
        float v0, v1;
        if constexpr (F32) {
          v0 = __uint_as_float(vx[x][0]);
          v1 = __uint_as_float(vx[x][F32 ? 1 : 0]);
        } else {
          v0 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] & 0xFFFF)));
          v1 = __half2float(__ushort_as_half((unsigned short)(vx[x][0] >> 16)));
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float w = tok ? s_ts[hh][min(t, kMaxTail - 1)] : 0.f;
          ta[hh][0] = fmaf(w, v0, ta[hh][0]);
          ta[hh][1] = fmaf(w, v1, ta[hh][1]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_tailred[vph][hh][2 * vcp] = ta[hh][0];
      s_tailred[vph][hh][2 * vcp + 1] = ta[hh][1];
    }
  }

  // ---- pass 2: values ------------------------------------------------------
  const float lam2 = s_lam[oh < G ? oh : 0], mu2 = s_mu[oh < G ? oh : 0];
  v4i vacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vacc[ct] = v4i{0, 0, 0, 0};
  float psum = 0.f;
  unsigned char* pd = reinterpret_cast<unsigned char*>(&s_pdig[wave][0][0][0]);
  for (int tile = wave; tile < tiles; tile += kWaves) {
    uint32_t kw[8], vw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      kw[q] = kn[q];
      vw[q] = vn[q];
    }
    // (b = 8: the next key tile is requested once this one's scores are done,
    // which keeps both key tiles from being live at once)
    const int knext = tile + kWaves < kKeepN ? tiles : tile + kWaves;   // kept: no traffic
    if constexpr (BITS < 8) load_k(knext, kn);
    load_v(tile + kWaves, vn);
    const bool ok = oh < G && tile * TB + TPL * i16 < n;
    // p relative to the largest visual probability, as four signed digits of
    // P = round(p 2^27)
    uint32_t fb[TPL];
#pragma unroll
    for (int m = 0; m < TPL; ++m) {
      const float s = tile < kKeepN ? s_keepn[tile][lane][m] : score(kw, m);
      float p = 0.f;
      if (ok) p = exp2f(fmaf(s, lam2, mu2));
      psum += p;
      fb[m] = cqm::sdigits(cqm::p_fixed(p));
    }
    if constexpr (BITS == 8) load_k(knext, kn);
    if (oh < G) {
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) {
        unsigned char* dst = pd + (oh * 4 + pl) * TB + TPL * i16;
        if constexpr (TPL == 4) {
          *reinterpret_cast<uint32_t*>(dst) = gather_byte(fb[0], fb[1], fb[2], fb[3], pl);
        } else {
#pragma unroll
          for (int m = 0; m < TPL; ++m) dst[m] = (unsigned char)(fb[m] >> (8 * pl));
        }
      }
    }
    wave_sync_lds();
    v4i av = {0, 0, 0, 0};
    if (rh < G) {
      const unsigned char* src = pd + (rh * 4 + rp) * TB + E * g4;
      if constexpr (E == 16) {
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        av = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
      } else if constexpr (E == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        av = v4i{(int)x.x, (int)x.y, 0, 0};
      } else {
        av = v4i{(int)*reinterpret_cast<const uint32_t*>(src), 0, 0, 0};
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint32_t w = vw[ct];
      if constexpr (BITS == 2) {
        vacc[ct] = mfma(av, v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)}, vacc[ct]);
      } else if constexpr (BITS == 4) {
        vacc[ct] = mfma(av, v4i{(int)(w & kNib), (int)((w >> 4) & kNib), 0, 0}, vacc[ct]);
      } else {
        const v4i lo{(int)(w & kNib), 0, 0, 0}, hi{(int)((w >> 1) & 0x78787878u), 0, 0, 0};
        vacc[ct] = mfma(av, lo, vacc[ct]);
        vacc[ct] = mfma(av, hi, vacc[ct]);
        vacc[ct] = mfma(av, hi, vacc[ct]);
      }
    }
    wave_sync_lds();                       // digits read before the next tile overwrites them
  }

  // ---- combine planes, reduce over waves --------------------------------
  // lane (head oh, column i16): channels 8*i16 + ct
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const long long sv = (long long)vacc[ct][0] + 256ll * vacc[ct][1] + 65536ll * vacc[ct][2] +
                         16777216ll * vacc[ct][3];
    s_vred[wave][oh][8 * i16 + ct] = (float)((double)sv * (1.0 / 134217728.0));   // 2^-27
  }
  psum = cqm::row_sum16(psum);
  if ((lane & 15) == 0) s_psum[wave][oh] = psum;
  lds_barrier();
  if constexpr (LT) {
    long_tail<G, F32>(P, unit, s_q, s_ts, s_tailred, s_ptail, s_tm, s_cm, s_cs);
    lds_barrier();
  }
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
    for (int q = 0; q < kPhases; ++q) tail += s_tailred[q][hh][j];
    // each part weighed by exp(its reference - top), as in the 1-bit kernel
    const float pt = s_ptail[hh];
    const float vx = s_vmax[hh], tx = s_tm[hh], top = fmaxf(vx, tx);
    const float al = n > 0 ? exp2f((vx - top) * kLog2e) : 0.f, at = exp2f((tx - top) * kLog2e);
    float o = at * tail;
    if (n > 0) o += al * (P.vs[(size_t)unit * 128 + j] * sv + pv * P.vm[(size_t)unit * 128 + j]);
    o /= (al * pv + at * pt);
    const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
    if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
    else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
  }
}



template <bool F32, bool LT>
hipError_t launch_f1(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) { CQ_LAUNCH((df_b1<1, F32, LT>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  if (G == 2) { CQ_LAUNCH((df_b1<2, F32, LT>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  CQ_LAUNCH((df_b1<4, F32, LT>), dim3(units), dim3(kThreads), 0, st, p);
  return hipSuccess;
}

template <bool F32>
hipError_t launch_f(const Params& p, int G, int units, hipStream_t st) {
  return p.T > kMaxTail ? launch_f1<F32, true>(p, G, units, st) : launch_f1<F32, false>(p, G, units, st);
}

template <bool F32, int TPW>
hipError_t launch_w1(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) { CQ_LAUNCH((df_b1<1, F32, false, TPW>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  if (G == 2) { CQ_LAUNCH((df_b1<2, F32, false, TPW>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  CQ_LAUNCH((df_b1<4, F32, false, TPW>), dim3(units), dim3(kThreads), 0, st, p);
  return hipSuccess;
}

// tiles per wave of the all-in-flight instance: 2 or 4 (n <= 4096; with 8,
// the key, score and value registers of a wave exceed its 256 VGPRs)
constexpr int kWideTiles = 4;
int wide_tpw(int n) {
  const int per_wave = ((n + kTile - 1) / kTile + kWaves - 1) / kWaves;
  return per_wave <= 2 ? 2 : 4;
}

template <bool F32>
hipError_t launch_w(const Params& p, int G, int units, hipStream_t st) {
  if (wide_tpw(p.n) == 2) return launch_w1<F32, 2>(p, G, units, st);
  return launch_w1<F32, 4>(p, G, units, st);
}

// CUs of the current device (0 if unknown)
long device_cus() {
  static long cache[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] > 0) return cache[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev] = cus;
  return cache[dev];
}

// Co-resident workgroups of an LDS-score kernel on the current device.
long lds_capacity(const void* fn, int slot) {
  static long cache[64][6];
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev][slot] > 0) return cache[dev][slot];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreadsL, 0) != hipSuccess) return 0;
  cache[dev][slot] = (long)cus * per_cu;
  return cache[dev][slot];
}

template <int G, bool F32>
hipError_t launch_l1(const Params& p, int units, hipStream_t st) {
  const void* fn = (const void*)dl_b1<G, F32>;
  const long cap = lds_capacity(fn, (G == 1 ? 0 : G == 2 ? 1 : 2) + (F32 ? 3 : 0));
  if (cap < 1) return hipErrorInvalidConfiguration;
  const int grid = (int)(units < cap ? units : cap);
  CQ_LAUNCH((dl_b1<G, F32>), dim3(grid), dim3(kThreadsL), 0, st, p, units);
  return hipSuccess;
}

template <bool F32>
hipError_t launch_l(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) return launch_l1<1, F32>(p, units, st);
  if (G == 2) return launch_l1<2, F32>(p, units, st);
  return launch_l1<4, F32>(p, units, st);
}

template <int BITS, bool F32, bool LT, bool ALL>
hipError_t launch_bn1(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) { CQ_LAUNCH((df_bn<BITS, 1, F32, LT, ALL>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  if (G == 2) { CQ_LAUNCH((df_bn<BITS, 2, F32, LT, ALL>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  CQ_LAUNCH((df_bn<BITS, 4, F32, LT, ALL>), dim3(units), dim3(kThreads), 0, st, p);
  return hipSuccess;
}

// The instance that keeps the scores of the first kAllKeepTokens tokens (its
// LDS allows one workgroup per CU) reads only the key tiles past them twice.
// It is the faster one at most one unit per CU, which is all such a launch
// has, and, although it then runs the units in rounds, on long caches, where
// the two-per-CU instance would read most key tiles twice (measured on
// MI355X, 32q/8kv, 512 to 1024 units: 8 to 19 % faster from 4096 tokens at
// b = 4 and 8, 1 to 4 % from 6144 at b = 2; 7 to 13 % slower at 3328).  The
// scores are the same values either way, so are the outputs.
template <int BITS, bool F32>
hipError_t launch_bn(const Params& p, int G, int units, hipStream_t st) {
  if (p.T > kMaxTail) return launch_bn1<BITS, F32, true, false>(p, G, units, st);
  const long cus = device_cus();
  if ((cus > 0 && units <= cus) || p.n >= (BITS == 2 ? 6144 : 4096))
    return launch_bn1<BITS, F32, false, true>(p, G, units, st);
  return launch_bn1<BITS, F32, false, false>(p, G, units, st);
}

template <bool F32>
hipError_t launch_b(const Params& p, int bits, int G, int units, hipStream_t st) {
  if (bits == 2) return launch_bn<2, F32>(p, G, units, st);
  if (bits == 4) return launch_bn<4, F32>(p, G, units, st);
  return launch_bn<8, F32>(p, G, units, st);
}

}  // namespace

namespace cqi {

size_t decode_fast_ws(int, int, int, int, int, int) { return 0; }

bool decode_fast_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return (a.bits == 1 || a.bits == 2 || a.bits == 4 || a.bits == 8) && a.d == 128 &&
         (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 && (a.T == 0 || a.tail_dtype == a.q_dtype);
}

bool decode_wide_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 && a.n <= kWaves * kWideTiles * kTile &&
         a.T <= kMaxTail && (a.T == 0 || a.tail_dtype == a.q_dtype);
}

// The all-in-flight instance needs a CU of its own per (batch, kv head)
// unit: its workgroups hold half of a CU's registers, and with more units
// than CUs the second round of workgroups would start only after the first.
// It is chosen while at least half the CUs stay free: with a unit on nearly
// every CU the one-launch kernel is faster (B = 32, 32q/8kv, n = 3328 on
// MI355X: 15.7 vs 16.3 us; B = 16: 15.0 vs 14.6 us).
bool decode_wide_preferred(const DecodeArgs& a) {
  if (!decode_wide_supported(a)) return false;
  const long cus = device_cus();
  return cus > 0 && 2L * a.B * a.Hkv <= cus;
}

hipError_t decode_wide(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi, a.nc};
  const int G = a.Hq / a.Hkv;
  return a.q_dtype == CQ_F32 ? launch_w<true>(p, G, units, a.stream) : launch_w<false>(p, G, units, a.stream);
}

bool decode_lds_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 && a.T <= kMaxTail &&
         (a.T == 0 || a.tail_dtype == a.q_dtype) && (long)G * ((a.n + kTile - 1) / kTile) * 512 <= kScoreBytes;
}

// The automatic choice: every (batch, kv head) unit gets a workgroup, and so
// a CU, of its own, and at least half the CUs stay free.  Measured on MI355X
// (b = 1, 32q/8kv, n = 8192): 8 to 64 units are 1 to 3 % faster than the
// one-launch kernel and up to 35 % faster than the split schedule, 128 units
// equal; at 256 units (one per CU) the one-launch kernel, whose dealt tiles
// balance the waves, is 5 % faster (24.2 vs 25.4 us), and with two or more
// units per CU its two workgroups per CU overlap each other's phases.
bool decode_lds_preferred(const DecodeArgs& a) {
  if (!decode_lds_supported(a)) return false;
  const long cap = lds_capacity((const void*)dl_b1<4, false>, 2);
  return cap > 0 && 2L * a.B * a.Hkv <= cap;
}

hipError_t decode_lds(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi, a.nc};
  const int G = a.Hq / a.Hkv;
  return a.q_dtype == CQ_F32 ? launch_l<true>(p, G, units, a.stream) : launch_l<false>(p, G, units, a.stream);
}

hipError_t decode_fast(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi, a.nc};
  const int G = a.Hq / a.Hkv;
  if (a.bits > 1)
    return a.q_dtype == CQ_F32 ? launch_b<true>(p, a.bits, G, units, a.stream)
                               : launch_b<false>(p, a.bits, G, units, a.stream);
  return a.q_dtype == CQ_F32 ? launch_f<true>(p, G, units, a.stream)
                             : launch_f<false>(p, G, units, a.stream);
}

}  // namespace cqi
