// Fused single-read 1-bit quantization of a float16 K or V cache.
//
// QbitAI article on CalibQuant, "Method" part 1: per channel, the range over
// the n tokens of one head fixes the uniform quantizer; with b = 1 a value
// becomes 1 exactly when it lies above the midpoint of its channel's range
// (round-half-to-even sends the midpoint itself to 0).
//
// The input is read from HBM once.  A persistent, cooperatively launched grid
// walks (unit, chunk) items, a unit being one (batch, head) and a chunk 256
// tokens.  Each workgroup keeps its 64 KB chunk in registers, reduces the
// chunk's per-channel min/max, merges it into the unit's min/max with device
// atomics, and waits at a per-unit arrival counter until every chunk of the
// unit has contributed.  The codes are then decided from the registers:
// for float16 x,  x > (mn+mx)/2  <=>  x > t  with t the largest float16 not
// above the exact midpoint, so the code is the sign bit of the packed
// float16 difference t - x (exact: a non-zero difference of two float16
// values never rounds to zero, and t is never -0).
//
// Items are dealt so that all chunks of a unit run in the same round on
// distinct, co-resident workgroups (the grid is a multiple of the chunk
// count), so every wait ends.  The wait is also bounded: past the bound the
// workgroup records a time-out in the workspace status word and goes on.
//
// Register tile: thread (wave w, lane l) with r = l/16 and k = l%16 holds
// channels 8k..8k+7 of tokens  base + 16*(4w + r) + it,  it = 0..15, as
// 16 uint4.  Each load instruction of a wave reads four whole 256-byte rows.
#include "cq_device.h"
#include "cq_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;            // tokens per item
constexpr int kIt = 16;                // tokens per thread
constexpr long kSpinLimit = 4000000;   // bounded wait (a few seconds); normal waits are microseconds

struct Ws {
  int* status;      // [0] time-out flag
  float* slot;      // [units][S][256]: each chunk's channel minima (0..127) and maxima (128..255)
  float* fin;       // [units][256]: the unit's channel minima and maxima
  int* flag;        // [units][S]: chunk s has published its slot
  int* fflag;       // [units]: the unit's range is published
};

__host__ __device__ inline size_t ws_bytes(int units, int S) {
  return 256 + (size_t)units * S * 256 * 4 + (size_t)units * 256 * 4 + (size_t)units * S * 4 +
         (size_t)units * 4;
}

__host__ __device__ inline Ws carve(void* base, int units, int S) {
  char* p = (char*)base;
  Ws w;
  w.status = (int*)p;
  w.slot = (float*)(p + 256);
  w.fin = w.slot + (size_t)units * S * 256;
  w.flag = (int*)(w.fin + (size_t)units * 256);
  w.fflag = w.flag + (size_t)units * S;
  return w;
}

__global__ void qf_init(Ws w, int units, int S) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long)units * S) w.flag[i] = 0;
  if (i < units) w.fflag[i] = 0;
  if (i == 0) w.status[0] = 0;
}

// Cross-workgroup exchange.  Every word that one workgroup hands to another
// (chunk ranges, the unit's range, flags) is written and read with
// agent-scope atomic accesses, which are coherent across the chip without
// cache maintenance.  Order comes from waiting for the stores to be
// acknowledged (s_waitcnt vmcnt(0)) before the flag is raised, and from the
// reader issuing its data loads only after it has seen the flag.  No
// L2 write-back / invalidate fence is needed, because no plain (cacheable)
// access takes part in the exchange.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void raise_flag(int* p) {
  __hip_atomic_store(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until *p == 1 (relaxed coherent polls).
__device__ __forceinline__ void wait_flag(int* p, int* status) {
  long spins = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      atomicExch(status, 1);
      break;
    }
  }
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

template <int LAYOUT>
__global__ void __launch_bounds__(kThreads) qf_b1(const __half* __restrict__ x, int n, int units, int S,
                                                  uint32_t* __restrict__ codes, float* __restrict__ scale,
                                                  float* __restrict__ minv, Ws w) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 4, k = lane & 15;
  const int pair = 4 * wave + r;                      // 16-token run owned by this (wave, row)
  __shared__ uint32_t red_min[4][16][4], red_max[4][16][4];
  __shared__ uint32_t thr[64];                        // per channel pair: float16 thresholds
  const long items = (long)units * S;

  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = (int)(item / S), s = (int)(item % S);
    const int base = s * kChunk;
    const __half* xu = x + (size_t)u * n * 128;

    // ---- load the chunk (rows past n repeat the last row) ------------------
    uint4 v[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      int tok = min(base + 16 * pair + it, n - 1);
      v[it] = *reinterpret_cast<const uint4*>(xu + (size_t)tok * 128 + 8 * k);
    }
    // ---- chunk min/max per channel ------------------------------------------
    uint32_t mn[4], mx[4];
    mn[0] = mx[0] = v[0].x; mn[1] = mx[1] = v[0].y; mn[2] = mx[2] = v[0].z; mn[3] = mx[3] = v[0].w;
#pragma unroll
    for (int it = 1; it < kIt; ++it) {
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
      for (int m = 0; m < 4; ++m) { red_min[wave][k][m] = mn[m]; red_max[wave][k][m] = mx[m]; }
    }
    __syncthreads();
    // ---- publish this chunk's range, then obtain the unit's ------------------
    float* my = w.slot + ((size_t)u * S + s) * 256;
    if (tid < 128) {
      const int kk = tid >> 3, m = (tid & 7) >> 1, hi = tid & 1;
      float lo_v = INFINITY, hi_v = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        uint32_t a = red_min[ww][kk][m], b = red_max[ww][kk][m];
        lo_v = fminf(lo_v, hi ? hi_f(a) : lo_f(a));
        hi_v = fmaxf(hi_v, hi ? hi_f(b) : lo_f(b));
      }
      st_coh(my + tid, lo_v);
      st_coh(my + 128 + tid, hi_v);
      stores_done();                           // acknowledged before the barrier
    }
    __syncthreads();
    if (tid == 0) raise_flag(w.flag + (size_t)u * S + s);
    if (s == 0) {
      // chunk 0 of the unit gathers every chunk's range (one flag per chunk: no
      // address is contended) and publishes the unit's range under fflag
      if (tid < 64) {
        long spins = 0;
        for (;;) {
          int ok = 1;
          for (int c = tid; c < S; c += 64)
            ok &= __hip_atomic_load(w.flag + (size_t)u * S + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
          if (__all(ok)) break;
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            if (tid == 0) atomicExch(w.status, 1);
            break;
          }
        }
      }
      __syncthreads();
      {
        const float* src = w.slot + (size_t)u * S * 256 + tid;
        float acc = ld_coh(src);
        for (int c = 1; c < S; ++c) {
          float vv = ld_coh(src + (size_t)c * 256);
          acc = tid < 128 ? fminf(acc, vv) : fmaxf(acc, vv);
        }
        st_coh(w.fin + (size_t)u * 256 + tid, acc);
        stores_done();
      }
      __syncthreads();
      if (tid == 0) raise_flag(w.fflag + u);
    } else if (tid == 0) {
      wait_flag(w.fflag + u, w.status);
    }
    __syncthreads();
    if (tid < 128) {
      const float lo_v = ld_coh(w.fin + (size_t)u * 256 + tid);
      const float hi_v = ld_coh(w.fin + (size_t)u * 256 + 128 + tid);
      unsigned short t = rd_half(0.5 * ((double)lo_v + (double)hi_v));
      reinterpret_cast<unsigned short*>(thr)[tid] = t;
      if (s == 0) {
        scale[(size_t)u * 128 + tid] = (float)((double)hi_v - (double)lo_v);
        minv[(size_t)u * 128 + tid] = lo_v;
      }
    }
    __syncthreads();
    const uint32_t t0 = thr[4 * k + 0], t1 = thr[4 * k + 1], t2 = thr[4 * k + 2], t3 = thr[4 * k + 3];

    // ---- codes: sign bits of t - x ------------------------------------------
    if (LAYOUT == CQ_LAYOUT_K) {
      // token word w holds channels 32w..32w+31; channel j at bit 8(j%4) + (j%32)/4.
      // This thread's channels 8k+e land at 8(e%4) + 2(k%4) + e/4.
      const int sh = 2 * (k & 3);
      uint32_t words[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
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
      if ((k & 3) == 0) {
        const int g = k >> 2;
        const int tok0 = base + 16 * pair;
        uint32_t* dst = codes + ((size_t)u * 4 + g) * n + tok0;
        if (tok0 + kIt <= n && (n & 3) == 0) {
#pragma unroll
          for (int q4 = 0; q4 < kIt / 4; ++q4)
            reinterpret_cast<uint4*>(dst)[q4] =
                make_uint4(words[4 * q4], words[4 * q4 + 1], words[4 * q4 + 2], words[4 * q4 + 3]);
        } else {
#pragma unroll
          for (int it = 0; it < kIt; ++it)
            if (tok0 + it < n) dst[it] = words[it];
        }
      }
    } else {
      // V word (group, channel) holds tokens 32*group .. +31; token t at bit 8(t%4) + t/4.
      // This thread's tokens are t = 16*half + it of group pair/2, half = pair%2:
      // byte it%4, bit it/4 + 4*half.  Build a compressed 16-bit image per channel
      // (bit 4*(it%4) + it/4), two channels per register.
      uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int pos = 4 * (it & 3) + (it >> 2);
        const uint32_t msk = 0x00010001u << pos;
        acc[0] |= (hsub2u(t0, v[it].x) >> (15 - pos)) & msk;
        acc[1] |= (hsub2u(t1, v[it].y) >> (15 - pos)) & msk;
        acc[2] |= (hsub2u(t2, v[it].z) >> (15 - pos)) & msk;
        acc[3] |= (hsub2u(t3, v[it].w) >> (15 - pos)) & msk;
      }
      const int tokp = base + 16 * pair;              // first token of this thread's run
      int nvalid = n - tokp;
      nvalid = nvalid < 0 ? 0 : (nvalid > kIt ? kIt : nvalid);
      uint32_t vmask = 0;
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        if (it < nvalid) vmask |= 1u << (4 * (it & 3) + (it >> 2));
      vmask |= vmask << 16;
      const int half = pair & 1;
      uint32_t out[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t c = acc[m] & vmask;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t cc = (c >> (16 * hh)) & 0xFFFFu;
          uint32_t wd = (cc & 0xFu) | ((cc & 0xF0u) << 4) | ((cc & 0xF00u) << 8) | ((cc & 0xF000u) << 12);
          wd <<= 4 * half;
          wd |= (uint32_t)__shfl_xor((int)wd, 16);    // partner row holds the other half
          out[2 * m + hh] = wd;
        }
      }
      const int group = (base >> 5) + (pair >> 1);
      const int R = (n + 31) >> 5;
      if (half == 0 && group < R) {
        uint32_t* dst = codes + ((size_t)u * R + group) * 128 + 8 * k;
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(out[0], out[1], out[2], out[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(out[4], out[5], out[6], out[7]);
      }
    }
    __syncthreads();       // LDS tiles are reused by the next item
  }
}

struct Launch {
  int grid;
  int S;
};

// Co-resident workgroups of `fn` on the current device (cached per device and layout).
long capacity_of(const void* fn, int layout) {
  static long cache[64][2];
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev][layout] > 0) return cache[dev][layout];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) return 0;
  cache[dev][layout] = (long)cus * per_cu;
  return cache[dev][layout];
}

bool plan(const cqi::QuantArgs& a, Launch& L, const void* fn) {
  const int units = a.B * a.H;
  L.S = (a.n + kChunk - 1) / kChunk;
  const long capacity = capacity_of(fn, a.layout);
  if (capacity < L.S) return false;
  long grid = (capacity / L.S) * L.S;
  const long items = (long)units * L.S;
  if (grid > items) grid = items;
  L.grid = (int)grid;
  return true;
}

}  // namespace

namespace cqi {

size_t quant_fused_ws(int B, int H, int n, int d) { return ws_bytes(B * H, (n + kChunk - 1) / kChunk); }

bool quant_fused_supported(const QuantArgs& a) {
  return a.dtype == CQ_F16 && a.bits == 1 && a.d == 128 && a.n >= 1 && a.n <= (1 << 20) &&
         (long)a.B * a.H >= 1;
}

hipError_t quant_fused(const QuantArgs& a) {
  const int units = a.B * a.H;
  Ws w = carve(a.ws, units, (a.n + kChunk - 1) / kChunk);
  const void* fn = a.layout == CQ_LAYOUT_K ? (const void*)qf_b1<CQ_LAYOUT_K> : (const void*)qf_b1<CQ_LAYOUT_V>;
  Launch L;
  if (!plan(a, L, fn)) return hipErrorInvalidConfiguration;
  const long init_n = (long)units * L.S;
  CQ_LAUNCH(qf_init, dim3((unsigned)((init_n + 255) / 256)), dim3(256), 0, a.stream, w, units, L.S);
  const __half* x = (const __half*)a.x;
  int n = a.n, S = L.S;
  void* args[] = {(void*)&x, (void*)&n, (void*)&units, (void*)&S, (void*)&a.codes, (void*)&a.scale,
                  (void*)&a.minv, (void*)&w};
  return hipLaunchCooperativeKernel(fn, dim3(L.grid), dim3(kThreads), args, 0, a.stream);
}

}  // namespace cqi
