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
// K side, per tile: C[16 x 16] += A[16 x 64] B[64 x 16] with
// v_mfma_i32_16x16x64_i8, twice (128 channels).  B bytes are code bits left
// in place in the packed word, one AND per register (bits_lo / bits_hi):
// channel j's bit sits in its byte with weight 2^s(j), s(j) =
// min(floor((j mod 32) / 4), 6).  Rows of A are (head, digit plane): each
// head's q * scale_K is a 22-bit fixed-point integer Q (q' 2^F, rounded),
// multiplied by 2^(7 - s(j)) for channel j and split into four signed
// base-256 digits, so every product is 2^7 Q_j c_j and the int32 plane sums
// are exact.  Columns are tokens.  Each lane ends up holding all planes of
// one (head, token) score: s = ((a0 + 2^8 a1) + 2^16 (a2 + 2^8 a3)) 2^-(F+7)
// + c0, the two halves exact in int32 and their sum rounded to float the same
// way in both passes.  The first pass over the keys only gathers every
// head's min and max, which fix g; the value pass reads the key tiles again
// (they are still in the Infinity Cache) and recomputes the same scores,
// instead of keeping 4 B per head and token on chip.
//
// V side, per tile: C[16 x 16] += A[16 x 64] B[64 x 16], rows again
// (head, plane), columns channels, contraction over tokens; B is the masked
// V word as on the K side.  p = exp(g(s) - max) in (0, 1] becomes
// P = round(p 2^22); token i's digits are those of P 2^(7 - s(i)), signed
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

// F32: query and text tail are float32 (else float16); the fast path takes
// them in one dtype.
template <int G, bool F32>
__global__ void __launch_bounds__(kThreads, 4) df_b1(Params P) {
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T;
  const int ntiles = (n + kTile - 1) / kTile;
  const int R = n >> 5;
  // Issue priority: the two workgroups on a CU would otherwise run their key
  // passes unevenly (the older one first), leaving the other's value pass
  // alone at the end.  High through the key pass (latency-bound), low through
  // the value pass (compute-bound), medium for the final reduction.
  __builtin_amdgcn_s_setprio(3);

  __shared__ float s_q[4][128];                 // sm * q, float
  __shared__ float s_qp[4][128];                // sm * q * scale_K
  __shared__ double s_c0[4];
  __shared__ float s_inv2f[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][4][32];   // K-side A digits: [head][plane][128 channel bytes]
  __shared__ __align__(16) uint32_t s_pdig[kWaves][4][4][32];   // V-side A digits: [head][plane][128 token bytes]
  __shared__ float s_ts[4][kMaxTail];           // tail scores, then tail probabilities
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4];
  __shared__ float s_tailred[kThreads / 64][4][128];   // tail values per token phase
  __shared__ unsigned long long s_vsum[4][128];   // sum 2^7 P c per head and channel (2^-29 units)
  __shared__ double s_psum[4];                     // sum P per head (2^-22 units)
  __shared__ int s_next[2];                        // next key tile of each pass
  __shared__ float s_vs[128], s_vm[128];           // scale_V, min_V

  // operand coordinates of the 16 x 16 x 64 products
  const int i16 = lane & 15, g4 = lane >> 4;    // A/B operand lane coordinates
  const int rh = i16 >> 2, rp = i16 & 3;        // A row = (head rh, plane rp)
  const int oh = lane >> 4;                     // output lane: head
  const uint32_t* kc = n > 0 ? P.kc : g_pad;
  const uint32_t* vcb = n > 0 ? P.vc : g_pad;
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(g_pad);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(g_pad);
  // The prologue's inputs are requested before any prefetch: vector loads
  // complete in order, so the prologue then waits for these alone.  Thread:
  // head ph (heads past G read head G - 1, unused), channel pj; the scales and
  // minima of an empty cache are read at the zero block.
  const int ph = tid >> 7, pj = tid & 127;
  const float* ksb = n > 0 ? P.ks : reinterpret_cast<const float*>(g_pad);
  const float* kmb = n > 0 ? P.km : reinterpret_cast<const float*>(g_pad);
  const float* vsb = n > 0 ? P.vs : reinterpret_cast<const float*>(g_pad);
  const float* vmb = n > 0 ? P.vm : reinterpret_cast<const float*>(g_pad);
  const size_t prm = n > 0 ? (size_t)unit * 128 + pj : (size_t)pj;
  const float q_in = ld_any(P.q, ((size_t)b * P.Hq + h * G + min(ph, G - 1)) * 128 + pj, F32);
  const float ks_in = ksb[prm], km_in = kmb[prm], vs_in = vsb[prm], vm_in = vmb[prm];
  auto load_k = [&](int tile, uint4& w0, uint4& w1) {   // tokens past n: scores not used
    const int tok = max(min(tile * kTile + 8 * i16, n - 8), 0);
    const uint4* src = reinterpret_cast<const uint4*>(kc + ((size_t)unit * 4 + g4) * n + tok);
    w0 = src[0];
    w1 = src[1];
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
  // the key pass keeps two tiles of look-ahead per wave (kn, km), the value
  // pass one (kn, vn); the first two are requested under the prologue
  uint4 kn0, kn1, km0, km1;
  load_k(wave, kn0, kn1);
  load_k(wave + kWaves, km0, km1);
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
  __shared__ double s_c0p[8];
  __shared__ float s_mqp[8];
  {                                             // thread: head ph, channel pj
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
  lds_barrier();
  if (tid < 4) {
    const double c0 = s_c0p[2 * tid] + s_c0p[2 * tid + 1];
    const float mq = fmaxf(s_mqp[2 * tid], s_mqp[2 * tid + 1]);
    int F = 0;
    if (mq > 0.f) F = 21 - ilogbf(mq);
    s_F[tid] = F;
    s_inv2f[tid] = ldexpf(1.f, -F - 7);         // products carry 2^7 (bits_lo / bits_hi)
    s_c0[tid] = c0;
  }
  lds_barrier();
  {
    // channel j's factor 2^bit_weight(j mod 32) makes up for the place its
    // code bit keeps in the masked word; the digits are the bytes of
    // Qs + 0x808080 with the low three offset back by 128 (signed base-256)
    const int hh = tid >> 7, j = tid & 127;
    const int Q = (int)rintf(ldexpf(s_qp[hh][j], s_F[hh]));        // |Q| <= 2^22
    const uint32_t dig = ((uint32_t)(Q * (1 << bit_weight(j & 31))) + 0x00808080u) ^ 0x00808080u;   // |Qs| <= 2^29
    unsigned char* ad = reinterpret_cast<unsigned char*>(&s_adig[hh][0][0]);
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) ad[pl * 128 + j] = (unsigned char)(dig >> (8 * pl));
  }
  lds_barrier();

  // ---- text tail scores ---------------------------------------------------
  // The prefetched rounds run straight (no early exit: every lane's rows were
  // loaded, in bounds, and rows past T are not stored); rounds past kPreTail
  // tokens load as they go.
  {
    const int sub = tsub, cl = tcl;
    auto tail_scores = [&](int j, const float (&kf)[8]) {
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
    for (int j0 = 4 * wave + 4 * kWaves * kKtRounds; j0 < T; j0 += 4 * kWaves) {
      const int j = j0 + sub;
      float kf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kf[c] = j < T ? ld_any(P.kt, ((size_t)unit * T + j) * 128 + 8 * cl + c, F32) : 0.f;
      tail_scores(j, kf);
    }
  }
  // ---- phase 1: visual scores, their min and max -------------------------
  v4i ak0 = {0, 0, 0, 0}, ak1 = {0, 0, 0, 0};
  if (rh < G) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
    const uint4 x1 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4 + 4]);
    ak0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
    ak1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  const float inv2f = s_inv2f[oh < G ? oh : 0];
  const float c0f = (float)s_c0[oh < G ? oh : 0];
  // scores of this lane's 8 tokens (head oh) from one key tile; the same
  // integer products and the same rounding in both passes
  auto scores = [&](const uint4& w0, const uint4& w1, float (&st)[8]) {
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      v4i acc = {0, 0, 0, 0};
      acc = mfma(ak0, bits_lo(wd[m]), acc);
      acc = mfma(ak1, bits_hi(wd[m]), acc);
      // 2^7 Q . c = lo + 2^16 hi; both halves fit 31 bits, the sum is
      // rounded to float (the same operations in both passes)
      const int lo = acc[0] + (acc[1] << 8), hi = acc[2] + (acc[3] << 8);
      st[m] = fmaf(fmaf((float)hi, 65536.f, (float)lo), inv2f, c0f);
      // pin the finished score: otherwise the compiler may keep the four
      // accumulator registers alive in its place
      asm volatile("" : "+v"(st[m]));
    }
  };
  float vmin = INFINITY, vmax = -INFINITY;
  // a wave's tiles come in increasing order: tile, then tnext (loading into
  // km), then nxt
  for (int tile = wave, tnext = wave + kWaves; tile < ntiles;) {
    int nxt = 0;
    if (lane == 0) nxt = atomicAdd(&s_next[0], 1);
    nxt = __builtin_amdgcn_readfirstlane(nxt);
    const uint4 kw0 = kn0, kw1 = kn1;
    kn0 = km0;
    kn1 = km1;
    load_k(nxt, km0, km1);                      // past the last tile: an in-bounds reread, unused
    // n % 32 == 0, so this lane's 8 tokens tile*128 + 8 i16 + m are all valid or none
    const bool ok = tile * kTile + 8 * i16 < n;
    float st[8];
    scores(kw0, kw1, st);
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
    // fold tile by tile: left free, the compiler sinks these updates past the
    // loop and keeps every tile's scores alive
    asm volatile("" : "+v"(vmin), "+v"(vmax));
    tile = tnext;
    tnext = nxt;
  }
  // the first key and value tiles of the second pass, then the first
  // kPreTail tail values, are requested before the score statistics settle.
  // (The key base goes through an opaque copy: otherwise the compiler proves
  // the second pass's loads equal the first's and keeps every first-pass score
  // alive instead of recomputing it.)
  asm("" : "+s"(kc));
  load_k(wave, kn0, kn1);
  // V word row of this lane, channels 8*i16 .. +7.  Rows past the last hold
  // tokens whose p is 0: whatever codes they read, their digits are 0.
  auto load_v = [&](int tile, uint4& w0, uint4& w1) {
    const int row = max(min(tile * 4 + g4, R - 1), 0);
    const uint4* src = reinterpret_cast<const uint4*>(vcb + ((size_t)unit * R + row) * 128 + 8 * i16);
    w0 = src[0];
    w1 = src[1];
  };
  uint4 vn0, vn1;
  load_v(wave, vn0, vn1);
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
      vtr[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(vtb) + e));
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
  lds_barrier();
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
    float lam = 1.f, mu = 0.f, vis_max = M;
    if (P.calib_on && n > 0) {
      const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
      lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
      mu = t_lo - lam * m;
      vis_max = fmaxf(t_lo, t_hi);
    }
    const float top = fmaxf(n > 0 ? vis_max : -INFINITY, tmax);
    if (lane == 0) {
      s_lam[hh] = lam * kLog2e;                 // p = 2^(s * lam' + mu')
      s_mu[hh] = (mu - top) * kLog2e;
    }
    // tail probabilities (in place) and their sum
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
  lds_barrier();
  // text-tail values: thread (channel pair vcp, phase vph) sums the tail
  // tokens vph + kPhases i for every head, the first kPreTail from the loads above
  {
    float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      const int t = vph + kPhases * i;
      if (t < T) {
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
          ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
          ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
        }
      }
    }
    for (int t = kPreTail + vph; t < T; t += kPhases) {
      const float v0 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp, F32);
      const float v1 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp + 1, F32);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
        ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_tailred[vph][hh][2 * vcp] = ta[hh][0];
      s_tailred[vph][hh][2 * vcp + 1] = ta[hh][1];
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
  // the wave's int32 plane sums grow by at most 2^20 per tile (128 tokens x
  // |digit| <= 128 x code byte <= 64); they are moved into the exact 64-bit
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
  unsigned char* pd = reinterpret_cast<unsigned char*>(&s_pdig[wave][0][0][0]);
  for (int tile = wave; tile < ntiles;) {
    int nxt = 0;
    if (lane == 0) nxt = atomicAdd(&s_next[1], 1);
    nxt = __builtin_amdgcn_readfirstlane(nxt);
    const uint4 kw0 = kn0, kw1 = kn1, vw0 = vn0, vw1 = vn1;
    load_k(nxt, kn0, kn1);
    load_v(nxt, vn0, vn1);
    // probabilities of this lane's 8 tokens (head oh) as 22-bit fixed point
    // P = round(p 2^22), the mantissa of p 2^22 + 2^23; tokens that do not
    // count get exponent -inf, so p = 0
    const bool ok = oh < G && tile * kTile + 8 * i16 < n;
    const float mu_t = ok ? mu2 : -INFINITY;
    float st[8];
    scores(kw0, kw1, st);
    uint32_t fb[8], ptile = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st[m], lam2, mu_t));   // argument <= 0 (up to rounding)
      const uint32_t Pm = __float_as_uint(fmaf(p, 4194304.f, 8388608.f)) & 0x007FFFFFu;
      ptile += Pm;
      // digits of P 2^wt: bytes of P 2^wt + 0x808080, the low three offset back by 128
      fb[m] = ((Pm << (m < 4 ? wt0 : wt1)) + 0x00808080u) ^ 0x00808080u;
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
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
  if ((lane & 15) == 0 && oh < G) atomicAdd(&s_psum[oh], psum);
  lds_barrier();
  if (tid < G * 128) {
    const int hh = tid >> 7, j = tid & 127;
    const float sv = (float)((double)(long long)s_vsum[hh][j] * (1.0 / 536870912.0));   // 2^-29
    const float pv = (float)(s_psum[hh] * (1.0 / 4194304.0));
    float tail = 0.f;
#pragma unroll
    for (int q = 0; q < kPhases; ++q) tail += s_tailred[q][hh][j];
    const float pt = s_ptail[hh];
    float o = tail;
    if (n > 0) o += s_vs[j] * sv + pv * s_vm[j];
    o /= (pv + pt);
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
  constexpr int kRegion = G * 128;            // words per tile: G x 128 scores, then G x 4 x 128 digit bytes

  __shared__ float s_q[4][128];
  __shared__ float s_qp[4][128];
  __shared__ double s_c0[4];
  __shared__ float s_inv2f[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][4][32];
  __shared__ float s_ts[4][kMaxTail];
  __shared__ float s_red[kWavesL][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4];
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
    const uint4* src = reinterpret_cast<const uint4*>(kc + ((size_t)u * 4 + ((t & 63) >> 4)) * n + tok);
    w0 = src[0];
    w1 = src[1];
  };
  auto load_v = [&](int u, int tile, int t, uint4& w0, uint4& w1) {
    const int row = max(min(tile * 4 + ((t & 63) >> 4), R - 1), 0);
    const uint4* src = reinterpret_cast<const uint4*>(vcb + ((size_t)u * R + row) * 128 + 8 * (t & 15));
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
    if (tid < 4) s_psum[tid] = 0.0;
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
    lds_barrier();
    if (tid < 4) {
      const double c0 = s_c0p[2 * tid] + s_c0p[2 * tid + 1];
      const float mq = fmaxf(s_mqp[2 * tid], s_mqp[2 * tid + 1]);
      int F = 0;
      if (mq > 0.f) F = 21 - ilogbf(mq);
      s_F[tid] = F;
      s_inv2f[tid] = ldexpf(1.f, -F - 7);
      s_c0[tid] = c0;
    }
    lds_barrier();
    if (tid < 512) {
      const int hh = tid >> 7, j = tid & 127;
      const int Q = (int)rintf(ldexpf(s_qp[hh][j], s_F[hh]));
      const uint32_t dig = ((uint32_t)(Q * (1 << bit_weight(j & 31))) + 0x00808080u) ^ 0x00808080u;
      unsigned char* ad = reinterpret_cast<unsigned char*>(&s_adig[hh][0][0]);
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) ad[pl * 128 + j] = (unsigned char)(dig >> (8 * pl));
    }
    lds_barrier();

    // ---- text tail scores -----------------------------------------------------
    {
      const int sub = tsub, cl = tcl;
      auto tail_scores = [&](int j, const float (&kf)[8]) {
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
      for (int j0 = 4 * wave + 4 * kWavesL * kKtRounds; j0 < T; j0 += 4 * kWavesL) {
        const int j = j0 + sub;
        float kf[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          kf[c] = j < T ? ld_any(P.kt, ((size_t)unit * T + j) * 128 + 8 * cl + c, F32) : 0.f;
        tail_scores(j, kf);
      }
    }

    // ---- key pass: scores into LDS, their min and max --------------------------
    v4i ak0 = {0, 0, 0, 0}, ak1 = {0, 0, 0, 0};
    if (rh < G) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4]);
      const uint4 x1 = *reinterpret_cast<const uint4*>(&s_adig[rh][rp][8 * g4 + 4]);
      ak0 = v4i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
      ak1 = v4i{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
    const float inv2f = s_inv2f[oh < G ? oh : 0];
    const float c0f = (float)s_c0[oh < G ? oh : 0];
    float vmin = INFINITY, vmax = -INFINITY;
    // Slot j of the ring holds the key tile tq[j]; the slots are used in
    // turn, and a used slot is refilled in place with the next dealt tile.
    // (Rotating the registers instead would move a tile whose load is still
    // in flight, and the move waits for it: no look-ahead would be left.)
    int tq[kAheadK];
#pragma unroll
    for (int j = 0; j < kAheadK; ++j) tq[j] = wave + j * kWavesL;
    auto key_tile = [&](uint4& s0, uint4& s1, int& slot_tile) {
      const int tile = slot_tile;
      int nxt = 0;
      if (lane == 0) nxt = atomicAdd(&s_next[0], 1);
      nxt = __builtin_amdgcn_readfirstlane(nxt);
      const bool ok = tile * kTile + 8 * i16 < n;
      const uint32_t wd[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float st[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        v4i acc = {0, 0, 0, 0};
        acc = mfma(ak0, bits_lo(wd[m]), acc);
        acc = mfma(ak1, bits_hi(wd[m]), acc);
        const int lo = acc[0] + (acc[1] << 8), hi = acc[2] + (acc[3] << 8);
        st[m] = fmaf(fmaf((float)hi, 65536.f, (float)lo), inv2f, c0f);
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
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      vmin = fminf(vmin, __shfl_xor(vmin, off));
      vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
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
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        m = fminf(m, __shfl_xor(m, off));
        M = fmaxf(M, __shfl_xor(M, off));
        tmax = fmaxf(tmax, __shfl_xor(tmax, off));
      }
      float lam = 1.f, mu = 0.f, vis_max = M;
      if (P.calib_on && n > 0) {
        const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
        lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
        mu = t_lo - lam * m;
        vis_max = fmaxf(t_lo, t_hi);
      }
      const float top = fmaxf(n > 0 ? vis_max : -INFINITY, tmax);
      if (lane == 0) {
        s_lam[hh] = lam * kLog2e;
        s_mu[hh] = (mu - top) * kLog2e;
      }
      float ptl = 0.f;
      for (int j = lane; j < T; j += 64) {
        const float pj2 = exp2f((s_ts[hh][j] - top) * kLog2e);
        s_ts[hh][j] = pj2;
        ptl += pj2;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ptl += __shfl_xor(ptl, off);
      if (lane == 0) s_ptail[hh] = ptl;
    }
    lds_barrier();
    if (tid < kThreads) {                       // text-tail values, df_b1's phases
      float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < kPreTail / kPhases; ++i) {
        const int t = vph + kPhases * i;
        if (t < T) {
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
            ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
            ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
          }
        }
      }
      for (int t = kPreTail + vph; t < T; t += kPhases) {
        const float v0 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp, F32);
        const float v1 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp + 1, F32);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
          ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
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
      const float mu_t = ok ? mu2 : -INFINITY;
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
        const float p = __builtin_amdgcn_exp2f(fmaf(st[m], lam2, mu_t));
        const uint32_t Pm = __float_as_uint(fmaf(p, 4194304.f, 8388608.f)) & 0x007FFFFFu;
        ptile += Pm;
        fb[m] = ((Pm << (m < 4 ? wt0 : wt1)) + 0x00808080u) ^ 0x00808080u;
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
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
    if ((lane & 15) == 0 && oh < G) atomicAdd(&s_psum[oh], psum);
    lds_barrier();
    if (tid < G * 128) {
      const int hh = tid >> 7, j = tid & 127;
      const float sv = (float)((double)(long long)s_vsum[hh][j] * (1.0 / 536870912.0));
      const float pv = (float)(s_psum[hh] * (1.0 / 4194304.0));
      float tail = 0.f;
#pragma unroll
      for (int q = 0; q < kPhases; ++q) tail += s_tailred[q][hh][j];
      const float ptt = s_ptail[hh];
      float o = tail;
      if (n > 0) o += s_vs[j] * sv + pv * s_vm[j];
      o /= (pv + ptt);
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
template <int BITS, int G, bool F32>
__global__ void __launch_bounds__(kThreads, 4) df_bn(Params P) {
  constexpr int E = 32 / BITS;                  // codes per word
  constexpr int TB = 4 * E;                     // tokens per tile
  constexpr int TPL = TB / 16;                  // key tokens per lane per tile
  constexpr int W = 4 * BITS;                   // key word planes per token
  constexpr uint32_t kNib = 0x0F0F0F0Fu;
  const int unit = blockIdx.x;
  const int b = unit / P.Hkv, h = unit % P.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = P.n, T = P.T;
  const int tiles = (n + TB - 1) / TB;
  const int R = n / E;

  __shared__ float s_q[4][128];
  __shared__ float s_qp[4][128];
  __shared__ double s_c0[4];
  __shared__ float s_inv2f[4];
  __shared__ int s_F[4];
  __shared__ __align__(16) uint32_t s_adig[4][3][32];
  __shared__ __align__(16) uint32_t s_pdig[kWaves][4][3][TB / 4];   // V-side A digits: [head][plane][TB bytes]
  __shared__ float s_ts[4][kMaxTail];
  __shared__ float s_red[kWaves][4][2];
  __shared__ float s_lam[4], s_mu[4], s_ptail[4];
  __shared__ float s_tailred[kThreads / 64][4][128];
  __shared__ float s_vred[kWaves][4][128];
  __shared__ float s_psum[kWaves][4];

  const int i16 = lane & 15, g4 = lane >> 4;
  const int rh = i16 >> 2, rp = i16 & 3;
  const int oh = lane >> 4;
  const uint32_t* kc = n > 0 ? P.kc : g_pad;
  const uint32_t* vcb = n > 0 ? P.vc : g_pad;
  const char* ktb = T > 0 ? reinterpret_cast<const char*>(P.kt) : reinterpret_cast<const char*>(g_pad);
  const char* vtb = T > 0 ? reinterpret_cast<const char*>(P.vt) : reinterpret_cast<const char*>(g_pad);
  auto load_k = [&](int tile, uint32_t (&w)[8]) {   // tokens past n: scores not used
    const int tok0 = max(min(tile * TB + TPL * i16, n - TPL), 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = 0u;
    {
#pragma unroll
      for (int p = 0; p < BITS; ++p) {
        const uint32_t* src = kc + ((size_t)unit * W + BITS * g4 + p) * n + tok0;
        if constexpr (TPL == 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(src);
          w[4 * p] = x.x; w[4 * p + 1] = x.y; w[4 * p + 2] = x.z; w[4 * p + 3] = x.w;
        } else if constexpr (TPL == 2) {
          const uint2 x = *reinterpret_cast<const uint2*>(src);
          w[2 * p] = x.x; w[2 * p + 1] = x.y;
        } else {
          w[p] = src[0];
        }
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
#pragma unroll
    for (int m = 0; m < TPL; ++m) {
      const float s = score(kw, m);
      if (ok) {
        vmin = fminf(vmin, s);
        vmax = fmaxf(vmax, s);
      }
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
  load_k(wave, kn);
  auto load_v = [&](int tile, uint32_t (&w)[8]) {   // rows past the last: p = 0 (as in df_b1)
    const int row = max(min(tile * 4 + g4, R - 1), 0);
    const uint4* src = reinterpret_cast<const uint4*>(vcb + ((size_t)unit * R + row) * 128 + 8 * i16);
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
    for (int j0 = 4 * wave + 4 * kWaves * kKtRounds; j0 < T; j0 += 4 * kWaves) {
      const int j = j0 + sub;
      float kf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kf[c] = j < T ? ld_any(P.kt, ((size_t)unit * T + j) * 128 + 8 * cl + c, F32) : 0.f;
      tail_scores(j, kf);
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
  lds_barrier();
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
    float lam = 1.f, mu = 0.f, vis_max = M;
    if (P.calib_on && n > 0) {
      const float t_lo = P.a_lo * m + P.c_lo, t_hi = P.a_hi * M + P.c_hi;
      lam = M > m ? (t_hi - t_lo) / (M - m) : 0.f;
      mu = t_lo - lam * m;
      vis_max = fmaxf(t_lo, t_hi);
    }
    const float top = fmaxf(n > 0 ? vis_max : -INFINITY, tmax);
    if (lane == 0) {
      s_lam[hh] = lam * kLog2e;                 // p = 2^(s * lam' + mu')
      s_mu[hh] = (mu - top) * kLog2e;
    }
    // tail probabilities (in place) and their sum
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
  lds_barrier();
  // text-tail values: thread (channel pair vcp, phase vph) sums the tail
  // tokens vph + kPhases i for every head, the first kPreTail from the loads above
  {
    float ta[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < kPreTail / kPhases; ++i) {
      const int t = vph + kPhases * i;
      if (t < T) {
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
          ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
          ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
        }
      }
    }
    for (int t = kPreTail + vph; t < T; t += kPhases) {
      const float v0 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp, F32);
      const float v1 = ld_any(P.vt, ((size_t)unit * T + t) * 128 + 2 * vcp + 1, F32);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        ta[hh][0] = fmaf(s_ts[hh][t], v0, ta[hh][0]);
        ta[hh][1] = fmaf(s_ts[hh][t], v1, ta[hh][1]);
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
    if constexpr (BITS < 8) load_k(tile + kWaves, kn);
    load_v(tile + kWaves, vn);
    const bool ok = oh < G && tile * TB + TPL * i16 < n;
    uint32_t fb[TPL];
#pragma unroll
    for (int m = 0; m < TPL; ++m) {
      const float s = score(kw, m);
      float p = 0.f;
      if (ok) p = exp2f(fmaf(s, lam2, mu2));
      psum += p;
      fb[m] = __float_as_uint(fmaf(p, 4194304.f, 8388608.f)) ^ 0x00008080u;   // bytes: P^0x80, (P>>8)^0x80, P>>16
    }
    if constexpr (BITS == 8) load_k(tile + kWaves, kn);
    if (oh < G) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        unsigned char* dst = pd + (oh * 3 + pl) * TB + TPL * i16;
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
    if (rp == 3) {
      av = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    } else if (rh < G) {
      const unsigned char* src = pd + (rh * 3 + rp) * TB + E * g4;
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
    const float cnt128 = 128.f * (float)vacc[ct][3];
    const float sv = ((float)vacc[ct][0] + cnt128) + 256.f * ((float)vacc[ct][1] + cnt128) +
                     65536.f * (float)vacc[ct][2];
    s_vred[wave][oh][8 * i16 + ct] = sv * (1.f / 4194304.f);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
  if ((lane & 15) == 0) s_psum[wave][oh] = psum;
  lds_barrier();
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
    const float pt = s_ptail[hh];
    float o = tail;
    if (n > 0) o += P.vs[(size_t)unit * 128 + j] * sv + pv * P.vm[(size_t)unit * 128 + j];
    o /= (pv + pt);
    const size_t oi = ((size_t)b * P.Hq + h * G + hh) * 128 + j;
    if (P.out_f32) reinterpret_cast<float*>(P.out)[oi] = o;
    else reinterpret_cast<__half*>(P.out)[oi] = __float2half_rn(o);
  }
}



template <bool F32>
hipError_t launch_f(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) { CQ_LAUNCH((df_b1<1, F32>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  if (G == 2) { CQ_LAUNCH((df_b1<2, F32>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  CQ_LAUNCH((df_b1<4, F32>), dim3(units), dim3(kThreads), 0, st, p);
  return hipSuccess;
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

template <int BITS, bool F32>
hipError_t launch_bn(const Params& p, int G, int units, hipStream_t st) {
  if (G == 1) { CQ_LAUNCH((df_bn<BITS, 1, F32>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  if (G == 2) { CQ_LAUNCH((df_bn<BITS, 2, F32>), dim3(units), dim3(kThreads), 0, st, p); return hipSuccess; }
  CQ_LAUNCH((df_bn<BITS, 4, F32>), dim3(units), dim3(kThreads), 0, st, p);
  return hipSuccess;
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
         (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 && a.T <= kMaxTail &&
         (a.T == 0 || a.tail_dtype == a.q_dtype);
}

bool decode_lds_supported(const DecodeArgs& a) {
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  return a.bits == 1 && a.d == 128 && (G == 1 || G == 2 || G == 4) && a.n % 32 == 0 && a.T <= kMaxTail &&
         (a.T == 0 || a.tail_dtype == a.q_dtype) && (long)G * ((a.n + kTile - 1) / kTile) * 512 <= kScoreBytes;
}

// The automatic choice: every (batch, kv head) unit gets a workgroup, and so
// a CU, of its own.  Measured on MI355X (b = 1, 32q/8kv): 8 to 256 units at
// n = 3328 and 8192 are 7 to 16 % faster than the one-launch kernel and up to
// 35 % faster than the split schedule; with two or more units per workgroup
// the one-launch kernel, whose two workgroups per CU overlap each other's
// phases, is faster.
bool decode_lds_preferred(const DecodeArgs& a) {
  if (!decode_lds_supported(a)) return false;
  const long cap = lds_capacity((const void*)dl_b1<4, false>, 2);
  return cap > 0 && (long)a.B * a.Hkv <= cap;
}

hipError_t decode_lds(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi};
  const int G = a.Hq / a.Hkv;
  return a.q_dtype == CQ_F32 ? launch_l<true>(p, G, units, a.stream) : launch_l<false>(p, G, units, a.stream);
}

hipError_t decode_fast(const DecodeArgs& a) {
  const int units = a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  Params p{a.q, a.k_codes, a.k_scale, a.k_min, a.v_codes, a.v_scale, a.v_min, a.k_tail, a.v_tail, a.out,
           a.Hq, a.Hkv, a.n, a.T, a.q_dtype == CQ_F32, a.tail_dtype == CQ_F32, a.out_dtype == CQ_F32,
           a.sm_scale, a.calib_on, a.a_lo, a.c_lo, a.a_hi, a.c_hi};
  const int G = a.Hq / a.Hkv;
  if (a.bits > 1)
    return a.q_dtype == CQ_F32 ? launch_b<true>(p, a.bits, G, units, a.stream)
                               : launch_b<false>(p, a.bits, G, units, a.stream);
  return a.q_dtype == CQ_F32 ? launch_f<true>(p, G, units, a.stream)
                             : launch_f<false>(p, G, units, a.stream);
}

}  // namespace cqi
