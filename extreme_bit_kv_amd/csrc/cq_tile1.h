// The 1-bit float16 register tile shared by the fused quantizer
// (quantize_fused.hip) and the streaming row quantizer (quantize_rows.hip):
// packed float16 helpers, the float16 threshold of a channel's midpoint, and
// the stage that turns a tile held in registers into stored code words.
//
// QbitAI article on CalibQuant, "Method" part 1: with b = 1 a value becomes 1
// exactly when it lies above the midpoint of its channel's range
// (round-half-to-even sends the midpoint itself to 0).  For float16 x,
// x > mid  <=>  x > t  with t the largest float16 not above mid, so the code
// is the sign bit of the packed float16 difference t - x (exact: a non-zero
// difference of two float16 values never rounds to zero, an overflow keeps
// its sign, and t is never -0).
//
// Tile (8 waves, 16 rows per thread): thread (wave w, lane l) with r = l/16
// and k = l%16 holds channels 8k..8k+7 of tokens base + 16(4w + r) + it,
// it < 16, as 16 uint4; each load instruction of a wave reads four whole
// 256-byte rows.
#pragma once

#include "cq_device.h"

namespace cqt {

// The code words are written once and read by a later launch: their stores
// are non-temporal, so that they do not fill the caches with dirty lines
// (the fused quantize of K and V was 1.5 % faster with them).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                    // waves per workgroup
constexpr int kRows = 16;                    // consecutive tokens per thread
constexpr int kTile = 4 * kWaves * kRows;    // tokens per tile (512)

typedef _Float16 h2v __attribute__((ext_vector_type(2)));   // one packed float16 pair

__device__ __forceinline__ h2v as_h2(uint32_t a) { return __builtin_bit_cast(h2v, a); }
__device__ __forceinline__ uint32_t as_u(h2v a) { return __builtin_bit_cast(uint32_t, a); }
__device__ __forceinline__ uint32_t hmin2u(uint32_t a, uint32_t b) {
  return as_u(__builtin_elementwise_min(as_h2(a), as_h2(b)));     // v_pk_min_f16
}
__device__ __forceinline__ uint32_t hmax2u(uint32_t a, uint32_t b) {
  return as_u(__builtin_elementwise_max(as_h2(a), as_h2(b)));     // v_pk_max_f16
}
__device__ __forceinline__ uint32_t hsub2u(uint32_t a, uint32_t b) {
  return as_u(as_h2(a) - as_h2(b));                                // v_pk_add_f16 with neg
}
__device__ __forceinline__ float lo_f(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v & 0xFFFF))); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v >> 16))); }

__device__ __forceinline__ unsigned short half_pred(unsigned short b) {     // next float16 down
  if (b == 0x0000 || b == 0x8000) return 0x8001;                          // below zero: -smallest subnormal
  return (b & 0x8000) ? (unsigned short)(b + 1) : (unsigned short)(b - 1);
}
__device__ __forceinline__ unsigned short half_succ(unsigned short b) {     // next float16 up
  if (b == 0x8000 || b == 0x0000) return 0x0001;
  return (b & 0x8000) ? (unsigned short)(b - 1) : (unsigned short)(b + 1);
}

// Largest float16 t with t <= v (v exact in float64), never -0.
__device__ inline unsigned short rd_half(double v) {
  unsigned short h = __half_as_ushort(__float2half_rn((float)v));
  auto val = [](unsigned short b) { return (double)__half2float(__ushort_as_half(b)); };
  for (int i = 0; i < 3 && val(h) > v; ++i) h = half_pred(h);
  for (int i = 0; i < 3 && val(half_succ(h)) <= v; ++i) h = half_succ(h);
  if (h == 0x8000) h = 0x0000;
  return h;
}

// Threshold of a channel with float32 range [mn, mx]: the largest float16 t
// (possibly -inf) with 2t <= mn + mx, decided exactly for any float32 pair
// (their sum need not be exact in float64); +inf when mx <= mn, so that
// every finite value gets code 0.  Never -0.
__device__ inline unsigned short mid_threshold(float mn, float mx) {
  if (!(mx > mn)) return 0x7C00;
  const double a = mn, b = mx;
  auto le = [&](unsigned short h) -> bool {             // value(h) <= (a + b) / 2, exactly
    const float f = __half2float(__ushort_as_half(h));
    if (__builtin_isinf(f)) return f < 0.0f;
    return cqd::exact_sign3(2.0 * (double)f, -a, -b) <= 0;
  };
  unsigned short h = __half_as_ushort(__float2half_rn((float)(0.5 * a + 0.5 * b)));
  for (int i = 0; i < 4 && h != 0xFC00 && !le(h); ++i) h = half_pred(h);
  for (int i = 0; i < 4 && h != 0x7C00 && le(half_succ(h)); ++i) h = half_succ(h);
  if (h == 0x8000) h = 0x0000;
  return h;
}

// Codes of the tile `v` from the per-channel thresholds of this thread's
// channels 8k..8k+7 (t0..t3: float16 pairs), stored into the words of one
// (batch, head): `cu` is its first code word, laid out for `n_codes` tokens;
// `base` is the tile's first token, tokens >= n_end are not coded.
template <int LAYOUT>
__device__ __forceinline__ void store_tile_codes(const uint4 (&v)[kRows], uint32_t t0, uint32_t t1, uint32_t t2,
                                                 uint32_t t3, uint32_t* __restrict__ cu, int base, int n_end,
                                                 int n_codes, int pair, int k) {
  constexpr int IT = kRows;
  if (LAYOUT == CQ_LAYOUT_K) {
    // token word w holds channels 32w..32w+31; channel j at bit 8(j%4) + (j%32)/4.
    // This thread's channels 8k+e land at 8(e%4) + 2(k%4) + e/4.
    const int sh = 2 * (k & 3);
    uint32_t words[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      uint32_t d0 = hsub2u(t0, v[it].x), d1 = hsub2u(t1, v[it].y);
      uint32_t d2 = hsub2u(t2, v[it].z), d3 = hsub2u(t3, v[it].w);
      uint32_t a = __builtin_amdgcn_perm(d1, d0, 0x07050301u);   // sign bytes of e = 0..3
      uint32_t b = __builtin_amdgcn_perm(d3, d2, 0x07050301u);   // sign bytes of e = 4..7
      uint32_t wd = ((a >> 7) & 0x01010101u) | ((b >> 6) & 0x02020202u);
      wd <<= sh;
      wd |= __builtin_amdgcn_update_dpp(0u, wd, 0xB1, 0xF, 0xF, false);   // xor lane 1
      wd |= __builtin_amdgcn_update_dpp(0u, wd, 0x4E, 0xF, 0xF, false);   // xor lane 2
      words[it] = wd;
    }
    // every lane of the quad holds the combined words; lane k%4 = q stores
    // the 16-byte pieces q, q+4, ... of the run, so each store instruction
    // writes whole 64-byte stretches
    const int g = k >> 2, q = k & 3;
    const int tok0 = base + IT * pair;
    uint32_t* dst = cu + (size_t)g * n_codes + tok0;
    if (tok0 + IT <= n_end && (n_codes & 3) == 0) {
#pragma unroll
      for (int q4 = 0; q4 < IT / 4; q4 += 4) {
        uint4 val = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c == q)
            val = make_uint4(words[4 * (q4 + c)], words[4 * (q4 + c) + 1], words[4 * (q4 + c) + 2],
                             words[4 * (q4 + c) + 3]);
        if (q4 + q < IT / 4) __builtin_nontemporal_store((v4u){val.x, val.y, val.z, val.w}, reinterpret_cast<v4u*>(dst) + q4 + q);
      }
    } else if (q == 0) {
#pragma unroll
      for (int it = 0; it < IT; ++it)
        if (tok0 + it < n_end) dst[it] = words[it];
    }
  } else {
    // V word (group, channel) holds tokens 32*group .. +31; token t at bit
    // 8(t%4) + t/4.  A group is RPG = 32/IT consecutive runs (rows of one
    // wave); this thread's tokens t = IT*sub + it, sub = pair % RPG, sit in
    // byte it%4 at bit (IT/4)*sub + it/4.  Build a compressed IT-bit image
    // per channel (bit (IT/4)*(it%4) + it/4), two channels per register.
    constexpr int RPG = 32 / IT, QB = IT / 4;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int pos = QB * (it & 3) + (it >> 2);
      const uint32_t msk = 0x00010001u << pos;
      acc[0] |= (hsub2u(t0, v[it].x) >> (15 - pos)) & msk;
      acc[1] |= (hsub2u(t1, v[it].y) >> (15 - pos)) & msk;
      acc[2] |= (hsub2u(t2, v[it].z) >> (15 - pos)) & msk;
      acc[3] |= (hsub2u(t3, v[it].w) >> (15 - pos)) & msk;
    }
    const int tokp = base + IT * pair;              // first token of this thread's run
    int nvalid = n_end - tokp;
    nvalid = nvalid < 0 ? 0 : (nvalid > IT ? IT : nvalid);
    uint32_t vmask = 0;
#pragma unroll
    for (int it = 0; it < IT; ++it)
      if (it < nvalid) vmask |= 1u << (QB * (it & 3) + (it >> 2));
    vmask |= vmask << 16;
    const int sub = pair % RPG;
    uint32_t out[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t c = acc[m] & vmask;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t cc = (c >> (16 * hh)) & 0xFFFFu;
        uint32_t wd = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) wd |= ((cc >> (QB * bb)) & ((1u << QB) - 1)) << (8 * bb);
        wd <<= QB * sub;
        wd |= (uint32_t)__shfl_xor((int)wd, 16);    // the other runs of the group: rows r ^ 1 ...
        if (RPG == 4) wd |= (uint32_t)__shfl_xor((int)wd, 32);   // ... and r ^ 2, r ^ 3
        out[2 * m + hh] = wd;
      }
    }
    const int group = (base >> 5) + pair / RPG;
    const int R = (n_codes + 31) >> 5;
    const int R_end = (n_end + 31) >> 5;
    // every run of the group holds the combined words: runs 0 and 1 store
    // the two halves, one instruction covers the group's 512-byte row
    if (sub < 2 && group < R_end && group < R) {
      uint32_t* dst = cu + (size_t)group * 128 + 8 * k + 4 * sub;
      __builtin_nontemporal_store(sub == 0 ? (v4u){out[0], out[1], out[2], out[3]} : (v4u){out[4], out[5], out[6], out[7]},
                                  reinterpret_cast<v4u*>(dst));
    }
  }
}

}  // namespace cqt
