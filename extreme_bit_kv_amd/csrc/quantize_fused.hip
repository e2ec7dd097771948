// Fused single-read 1-bit quantization of a float16 K or V cache.
//
// QbitAI article on CalibQuant, "Method" part 1: per channel, the range over
// the n tokens of one head fixes the uniform quantizer; with b = 1 a value
// becomes 1 exactly when it lies above the midpoint of its channel's range
// (round-half-to-even sends the midpoint itself to 0).
//
// The input is read from HBM once.  A persistent grid walks (unit, chunk)
// items, a unit being one (batch, head) and a chunk 512
// tokens (128 KB).  A workgroup keeps its chunk in registers, reduces the
// chunk's per-channel min/max, meets the other chunks of the unit at a
// rendezvous in the workspace, and then decides the codes from the registers:
// for float16 x,  x > (mn+mx)/2  <=>  x > t  with t the largest float16 not
// above the exact midpoint, so the code is the sign bit of the packed
// float16 difference t - x (exact: a non-zero difference of two float16
// values never rounds to zero, and t is never -0).
//
// Items are dealt so that all chunks of a unit run in the same round on
// distinct workgroups (the grid is a multiple of the chunk count), and the
// grid is never larger than the number of workgroups the device holds at
// once, so on a device not filled by other work every wait ends.  The waits
// are also bounded: past the bound the workgroup records a time-out in the
// workspace status word and goes on.  (A cooperative launch would guarantee
// co-residency formally, but on this runtime it costs about 20 us of
// serialization around the kernel, some 8% of a long-context launch.)
//
// Rendezvous: every chunk publishes, per channel, one 32-bit word holding the
// float16 bit patterns of its min and max; chunk 0 of the unit (the leader)
// gathers the words of all chunks and publishes the unit's word per channel,
// which the other chunks poll.  The launch starts by resetting every such
// word to 0xFFFFFFFF, a value no range word can take (it would be a NaN min),
// so a word is its own ready flag: no cross-word ordering, fence or flag is
// involved.  Words are written and read with agent-scope atomic accesses,
// coherent across the chip without cache maintenance.
//
// Register tile (8 waves, 16 rows per thread): thread (wave w, lane l) with
// r = l/16 and k = l%16 holds channels 8k..8k+7 of tokens
// base + 16(4w + r) + it, it < 16, as 16 uint4; each load instruction of a
// wave reads four whole 256-byte rows.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kWaves = 8;              // waves per workgroup
constexpr int kRows = 16;              // consecutive tokens per thread
constexpr int kChunk = 4 * kWaves * kRows;   // tokens per item (512)
constexpr long kSpinLimit = 4000000;   // bounded wait (a few seconds); normal waits are microseconds

constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr int kGather = 4;             // chunk words a gathering thread loads at once

struct Ws {
  int* status;       // [0] time-out flag
  uint32_t* slot;    // [units][S][128]: chunk range words (min16 | max16 << 16)
  uint32_t* fin;     // [units][128]: unit range words
};

__host__ __device__ inline size_t ws_bytes(int units, int S) {
  return 256 + (size_t)units * S * 128 * 4 + (size_t)units * 128 * 4;
}

__host__ __device__ inline Ws carve(void* base, int units, int S) {
  char* p = (char*)base;
  Ws w;
  w.status = (int*)p;
  w.slot = (uint32_t*)(p + 256);
  w.fin = w.slot + (size_t)units * S * 128;
  return w;
}

__global__ void qf_init(Ws w, long words) {       // slot and fin are contiguous
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < words) w.slot[i] = kEmpty;
  if (i == 0) w.status[0] = 0;
}

__device__ __forceinline__ void st_word(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_word(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Largest float16 t with t <= v (v exact in float64), never -0.
__device__ unsigned short rd_half(double v) {
  unsigned short h = __half_as_ushort(__float2half_rn((float)v));
  auto val = [](unsigned short b) { return (double)__half2float(__ushort_as_half(b)); };
  auto pred = [](unsigned short b) -> unsigned short {
    if (b == 0x0000 || b == 0x8000) return 0x8001;      // below zero: -smallest subnormal
    return (b & 0x8000) ? (unsigned short)(b + 1) : (unsigned short)(b - 1);
  };
  auto succ = [](unsigned short b) -> unsigned short {
    if (b == 0x8000 || b == 0x0000) return 0x0001;
    return (b & 0x8000) ? (unsigned short)(b - 1) : (unsigned short)(b + 1);
  };
  for (int i = 0; i < 3 && val(h) > v; ++i) h = pred(h);
  for (int i = 0; i < 3 && val(succ(h)) <= v; ++i) h = succ(h);
  if (h == 0x8000) h = 0x0000;
  return h;
}

struct Smem {
  uint32_t red_min[kWaves][16][4], red_max[kWaves][16][4];
  float part_lo[kWaves * 64 / 128][128], part_hi[kWaves * 64 / 128][128];   // leader's gather
  uint32_t thr[64];                                   // per channel pair: float16 thresholds
};

// Register tile of one item: channels 8k..8k+7 of tokens base + 16 pair + it
// (rows past n repeat the last row).
__device__ __forceinline__ void load_chunk(uint4 (&v)[kRows], const __half* __restrict__ x, int n, long item,
                                           int S, int pair, int k) {
  const int u = (int)(item / S), s = (int)(item % S);
  const __half* xu = x + (size_t)u * n * 128;
  const int base = s * kChunk;
#pragma unroll
  for (int it = 0; it < kRows; ++it) {
    const int tok = min(base + kRows * pair + it, n - 1);
    v[it] = *reinterpret_cast<const uint4*>(xu + (size_t)tok * 128 + 8 * k);
  }
}

// One item: range of the chunk in `v`, the unit's rendezvous, codes and
// stores.
template <int LAYOUT>
__device__ __forceinline__ void qf_item(const uint4 (&v)[kRows], long item, int n, int S,
                                        uint32_t* __restrict__ codes, float* __restrict__ scale,
                                        float* __restrict__ minv, const Ws& w, Smem& sm) {
  constexpr int IT = kRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 4, k = lane & 15;
  const int pair = 4 * wave + r;                      // IT-token run owned by this (wave, row)
  const int u = (int)(item / S), s = (int)(item % S);
  const int base = s * kChunk;
    // ---- chunk min/max per channel ------------------------------------------
    uint32_t mn[4], mx[4];
    mn[0] = mx[0] = v[0].x; mn[1] = mx[1] = v[0].y; mn[2] = mx[2] = v[0].z; mn[3] = mx[3] = v[0].w;
#pragma unroll
    for (int it = 1; it < IT; ++it) {
      mn[0] = hmin2u(mn[0], v[it].x); mx[0] = hmax2u(mx[0], v[it].x);
      mn[1] = hmin2u(mn[1], v[it].y); mx[1] = hmax2u(mx[1], v[it].y);
      mn[2] = hmin2u(mn[2], v[it].z); mx[2] = hmax2u(mx[2], v[it].z);
      mn[3] = hmin2u(mn[3], v[it].w); mx[3] = hmax2u(mx[3], v[it].w);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      mn[m] = hmin2u(mn[m], (uint32_t)__shfl_xor((int)mn[m], 16));
      mx[m] = hmax2u(mx[m], (uint32_t)__shfl_xor((int)mx[m], 16));
      mn[m] = hmin2u(mn[m], (uint32_t)__shfl_xor((int)mn[m], 32));
      mx[m] = hmax2u(mx[m], (uint32_t)__shfl_xor((int)mx[m], 32));
    }
    if (r == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) { sm.red_min[wave][k][m] = mn[m]; sm.red_max[wave][k][m] = mx[m]; }
    }
    __syncthreads();
    // ---- publish this chunk's range, then obtain the unit's ------------------
    const bool leader = s == 0;
    if (tid < 128) {
      // thread tid: channel tid = 8 kk + 2 m + hi
      const int kk = tid >> 3, m = (tid & 7) >> 1, hi = tid & 1;
      float lo_v = INFINITY, hi_v = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        uint32_t a = sm.red_min[ww][kk][m], b = sm.red_max[ww][kk][m];
        lo_v = fminf(lo_v, hi ? hi_f(a) : lo_f(a));
        hi_v = fmaxf(hi_v, hi ? hi_f(b) : lo_f(b));
      }
      const uint32_t word = (uint32_t)__half_as_ushort(__float2half_rn(lo_v)) |
                            ((uint32_t)__half_as_ushort(__float2half_rn(hi_v)) << 16);
      st_word(w.slot + ((size_t)u * S + s) * 128 + tid, word);
    }
    uint32_t uw = 0;
    if (leader) {
      // every thread gathers: channel tid % 128 over its quarter's chunks,
      // kGather words per poll, so the whole gather costs one round trip
      constexpr int Q = kWaves * 64 / 128;
      const int c = tid & 127, q0 = tid >> 7;
      float lo_v = INFINITY, hi_v = -INFINITY;
      const uint32_t* src = w.slot + (size_t)u * S * 128 + c;
      for (int c0 = q0 * kGather; c0 < S; c0 += Q * kGather) {
        uint32_t wd[kGather];
        long spins = 0;
        for (;;) {
          bool ready = true;
#pragma unroll
          for (int q = 0; q < kGather; ++q) {
            wd[q] = c0 + q < S ? ld_word(src + (size_t)(c0 + q) * 128) : 0u;
            ready &= wd[q] != kEmpty;
          }
          if (ready) break;
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            atomicExch(w.status, 1);
            break;
          }
        }
#pragma unroll
        for (int q = 0; q < kGather; ++q) {
          if (c0 + q < S) {
            lo_v = fminf(lo_v, lo_f(wd[q]));
            hi_v = fmaxf(hi_v, hi_f(wd[q]));
          }
        }
      }
      sm.part_lo[q0][c] = lo_v;
      sm.part_hi[q0][c] = hi_v;
      __syncthreads();
      if (tid < 128) {
#pragma unroll
        for (int q = 1; q < Q; ++q) {
          lo_v = fminf(lo_v, sm.part_lo[q][tid]);
          hi_v = fmaxf(hi_v, sm.part_hi[q][tid]);
        }
        uw = (uint32_t)__half_as_ushort(__float2half_rn(lo_v)) |
             ((uint32_t)__half_as_ushort(__float2half_rn(hi_v)) << 16);
        st_word(w.fin + (size_t)u * 128 + tid, uw);
      }
    } else if (tid < 128) {
      long spins = 0;
      while ((uw = ld_word(w.fin + (size_t)u * 128 + tid)) == kEmpty) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          atomicExch(w.status, 1);
          break;
        }
      }
    }
    if (tid < 128) {
      const float lo_v = lo_f(uw), hi_v = hi_f(uw);
      unsigned short t = rd_half(0.5 * ((double)lo_v + (double)hi_v));
      reinterpret_cast<unsigned short*>(sm.thr)[tid] = t;
      if (leader) {
        scale[(size_t)u * 128 + tid] = (float)((double)hi_v - (double)lo_v);
        minv[(size_t)u * 128 + tid] = lo_v;
      }
    }
    __syncthreads();
    const uint32_t t0 = sm.thr[4 * k + 0], t1 = sm.thr[4 * k + 1], t2 = sm.thr[4 * k + 2], t3 = sm.thr[4 * k + 3];

    // ---- codes: sign bits of t - x ------------------------------------------
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
      {
        const int g = k >> 2, q = k & 3;
        const int tok0 = base + IT * pair;
        uint32_t* dst = codes + ((size_t)u * 4 + g) * n + tok0;
        if (tok0 + IT <= n && (n & 3) == 0) {
#pragma unroll
          for (int q4 = 0; q4 < IT / 4; q4 += 4) {
            uint4 val = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (c == q)
                val = make_uint4(words[4 * (q4 + c)], words[4 * (q4 + c) + 1], words[4 * (q4 + c) + 2],
                                 words[4 * (q4 + c) + 3]);
            if (q4 + q < IT / 4) reinterpret_cast<uint4*>(dst)[q4 + q] = val;
          }
        } else if (q == 0) {
#pragma unroll
          for (int it = 0; it < IT; ++it)
            if (tok0 + it < n) dst[it] = words[it];
        }
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
      int nvalid = n - tokp;
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
      const int R = (n + 31) >> 5;
      // every run of the group holds the combined words: runs 0 and 1 store
      // the two halves, one instruction covers the group's 512-byte row
      if (sub < 2 && group < R) {
        uint32_t* dst = codes + ((size_t)u * R + group) * 128 + 8 * k + 4 * sub;
        *reinterpret_cast<uint4*>(dst) = sub == 0 ? make_uint4(out[0], out[1], out[2], out[3])
                                                  : make_uint4(out[4], out[5], out[6], out[7]);
      }
    }
    // No barrier here: the next item writes red_* before, and thr / part_*
    // only after, a barrier that every thread reaches after its last read of
    // them in this item, so the LDS reuse is already ordered; the code stores
    // drain while the next tile loads.
}

template <int LAYOUT>
__global__ void __launch_bounds__(kWaves * 64) qf_b1(const __half* __restrict__ x, int n, int units, int S,
                                                     uint32_t* __restrict__ codes, float* __restrict__ scale,
                                                     float* __restrict__ minv, Ws w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pair = 4 * wave + (lane >> 4), k = lane & 15;
  __shared__ Smem sm;
  const long items = (long)units * S;
  uint4 v[kRows];
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    load_chunk(v, x, n, item, S, pair, k);
    qf_item<LAYOUT>(v, item, n, S, codes, scale, minv, w, sm);
  }
}

// Co-resident workgroups of `fn` on the current device (cached per device and layout).
long capacity_of(const void* fn, int layout) {
  static long cache[64][2];
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev][layout] > 0) return cache[dev][layout];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWaves * 64, 0) != hipSuccess) return 0;
  cache[dev][layout] = (long)cus * per_cu;
  return cache[dev][layout];
}

}  // namespace

namespace cqi {

size_t quant_fused_ws(int B, int H, int n, int d) { return ws_bytes(B * H, (n + kChunk - 1) / kChunk); }

// All chunks of a unit must be resident together, so a unit may have at most
// as many chunks as the device holds workgroups of the kernel at once.
bool quant_fused_supported(const QuantArgs& a) {
  if (!(a.dtype == CQ_F16 && a.bits == 1 && a.d == 128 && a.n >= 1 && a.n <= (1 << 20) &&
        (long)a.B * a.H >= 1))
    return false;
  const void* fn = a.layout == CQ_LAYOUT_K ? (const void*)qf_b1<CQ_LAYOUT_K> : (const void*)qf_b1<CQ_LAYOUT_V>;
  return capacity_of(fn, a.layout == CQ_LAYOUT_K ? 0 : 1) >= (a.n + kChunk - 1) / kChunk;
}

hipError_t quant_fused(const QuantArgs& a) {
  const int units = a.B * a.H;
  const int S = (a.n + kChunk - 1) / kChunk;
  Ws w = carve(a.ws, units, S);
  const void* fn = a.layout == CQ_LAYOUT_K ? (const void*)qf_b1<CQ_LAYOUT_K> : (const void*)qf_b1<CQ_LAYOUT_V>;
  const long capacity = capacity_of(fn, a.layout == CQ_LAYOUT_K ? 0 : 1);
  if (capacity < S) return hipErrorInvalidConfiguration;
  long grid = (capacity / S) * S;
  const long items = (long)units * S;
  if (grid > items) grid = items;
  const long words = (long)units * (S + 1) * 128;
  CQ_LAUNCH(qf_init, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, a.stream, w, words);
  const __half* x = (const __half*)a.x;
  int n = a.n, Sv = S, un = units;
  void* args[] = {(void*)&x, (void*)&n, (void*)&un, (void*)&Sv, (void*)&a.codes, (void*)&a.scale,
                  (void*)&a.minv, (void*)&w};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kWaves * 64), args, 0, a.stream);
}

}  // namespace cqi
