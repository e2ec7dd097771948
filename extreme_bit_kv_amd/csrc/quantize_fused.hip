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
#include "cq_tile1.h"

namespace {

using namespace cqt;
constexpr int kChunk = kTile;          // tokens per item (512)
constexpr long kSpinLimit = 4000000;   // default bounded wait (a few seconds); normal waits are microseconds

constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr int kGather = 4;             // chunk words a gathering thread loads at once

struct Ws {
  int* status;       // [0] time-out flag of this call, [1] of any call since the caller zeroed it
  long spin_limit;   // unsuccessful polls before a workgroup gives up
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
  w.spin_limit = kSpinLimit;
  w.slot = (uint32_t*)(p + 256);
  w.fin = w.slot + (size_t)units * S * 128;
  return w;
}

// slot and fin are contiguous, 16-byte aligned, a multiple of 128 words.
// The status word is cleared unless this launch is the second tensor of a
// pair quantized one after the other (the first one's time-out must stay).
__global__ void qf_init(Ws w, long quads, int reset_status) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < quads) reinterpret_cast<uint4*>(w.slot)[i] = make_uint4(kEmpty, kEmpty, kEmpty, kEmpty);
  if (i == 0 && reset_status) w.status[0] = 0;
}

__device__ __forceinline__ void st_word(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_word(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Smem {
  uint32_t red_min[kWaves][16][4], red_max[kWaves][16][4];
  float part_lo[kWaves * 64 / 128][128], part_hi[kWaves * 64 / 128][128];   // leader's gather
  uint32_t thr[64];                                   // per channel pair: float16 thresholds
};

// Register tile of one item: channels 8k..8k+7 of tokens base + 16 pair + it
// (rows past n repeat the last row).  The input is read once, so the loads
// are non-temporal, which shortens each workgroup's load phase (a round's
// time is a chain of latencies: load, rendezvous, codes).
__device__ __forceinline__ void load_chunk(uint4 (&v)[kRows], const __half* __restrict__ x, int n, long item,
                                           int S, int pair, int k) {
  const int u = (int)(item / S), s = (int)(item % S);
  const __half* xu = x + (size_t)u * n * 128;
  const int base = s * kChunk;
#pragma unroll
  for (int it = 0; it < kRows; ++it) {
    const int tok = min(base + kRows * pair + it, n - 1);
    v[it] = cqd::ld_nt(xu + (size_t)tok * 128 + 8 * k);
  }
}

// One item: range of the chunk in `v`, the unit's rendezvous, codes and
// stores.
constexpr int kPfRows = kRows / 2;    // rows of the next item requested into LDS during a rendezvous
typedef uint4 PfBuf[kPfRows][kWaves][64];

template <int LAYOUT>
__device__ __forceinline__ void qf_item(const uint4 (&v)[kRows], long item, int n, int S,
                                        uint32_t* __restrict__ codes, float* __restrict__ scale,
                                        float* __restrict__ minv, const Ws& w, Smem& sm,
                                        const __half* nx = nullptr, int nbase = 0, PfBuf* pf = nullptr) {
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
    if (pf != nullptr && nx != nullptr && !leader) {
      // the first rows of this thread's part of the next item go straight to
      // LDS while the rendezvous waits (each wave its own slots; the barrier
      // before the thresholds are read waits for them)
#pragma unroll
      for (int it = 0; it < kPfRows; ++it) {
        const int tok = min(nbase + kRows * pair + it, n - 1);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(nx + (size_t)tok * 128 + 8 * k),
                                         &(*pf)[it][wave][0], 16, 0, 0);
      }
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
          if (++spins > w.spin_limit) {
            atomicExch(w.status, 1);
            atomicExch(w.status + 1, 1);
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
        if (++spins > w.spin_limit) {
          atomicExch(w.status, 1);
          atomicExch(w.status + 1, 1);
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
    store_tile_codes<LAYOUT>(v, t0, t1, t2, t3,
                             codes + (size_t)u * (LAYOUT == CQ_LAYOUT_K ? 4 * (size_t)n : 128 * (size_t)((n + 31) >> 5)),
                             base, n, n, pair, k);
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

// K and V of one layer in one launch: the items of K (each (unit, chunk))
// come first, then those of V, each tensor with rendezvous words of its own.
// The boundary between them is a multiple of the chunk count, so all chunks
// of a unit still run in the same round.  One launch saves the second word
// reset, launch gap and first and last round of two separate calls.
// A workgroup that is not its unit's leader requests the first half of its
// next item straight into LDS as soon as it has published its chunk range:
// the rendezvous wait covers those loads, and the next item streams only the
// other half.  The leader does not: its gather is on every chunk's critical
// path, and a poll returns only after the loads issued before it.
__global__ void __launch_bounds__(kWaves * 64) qf_b1_pair(const __half* __restrict__ xk, const __half* __restrict__ xv,
                                                          int n, int units, int S, uint32_t* __restrict__ kcodes,
                                                          float* __restrict__ kscale, float* __restrict__ kminv,
                                                          uint32_t* __restrict__ vcodes, float* __restrict__ vscale,
                                                          float* __restrict__ vminv, Ws wk, Ws wv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pair = 4 * wave + (lane >> 4), k = lane & 15;
  __shared__ Smem sm;
  __shared__ __align__(16) PfBuf pf;
  const long per = (long)units * S, total = 2 * per;
  uint4 v[kRows];
  bool have = false;
  auto next_src = [&](long nitem, int& nbase) -> const __half* {
    if (nitem >= total) return nullptr;
    const long nl = nitem < per ? nitem : nitem - per;
    nbase = (int)(nl % S) * kChunk;
    return (nitem < per ? xk : xv) + (size_t)(nl / S) * n * 128;
  };
  auto fetch = [&](const __half* x, long li) {
    if (!have) {
      load_chunk(v, x, n, li, S, pair, k);
      return;
    }
    const int base = (int)(li % S) * kChunk;
    const __half* xu = x + (size_t)(li / S) * n * 128;
#pragma unroll
    for (int it = 0; it < kPfRows; ++it) v[it] = pf[it][wave][lane];
#pragma unroll
    for (int it = kPfRows; it < kRows; ++it)
      v[it] = cqd::ld_nt(xu + (size_t)min(base + kRows * pair + it, n - 1) * 128 + 8 * k);
  };
  long item = blockIdx.x;
  for (; item < per; item += gridDim.x) {
    fetch(xk, item);
    int nbase = 0;
    const __half* nx = next_src(item + gridDim.x, nbase);
    qf_item<CQ_LAYOUT_K>(v, item, n, S, kcodes, kscale, kminv, wk, sm, nx, nbase, &pf);
    have = nx != nullptr && item % S != 0;
  }
  for (; item < total; item += gridDim.x) {
    fetch(xv, item - per);
    int nbase = 0;
    const __half* nx = next_src(item + gridDim.x, nbase);
    qf_item<CQ_LAYOUT_V>(v, item - per, n, S, vcodes, vscale, vminv, wv, sm, nx, nbase, &pf);
    have = nx != nullptr && (item - per) % S != 0;
  }
}

// Co-resident workgroups of `fn` on the current device (cached per device and layout).
long capacity_of(const void* fn, int layout) {
  static long cache[64][3];
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

// K and V together: the two tensors' words follow each other in the workspace
// (one status word), reset by one launch.
size_t quant_fused_pair_ws(int B, int H, int n, int d) {
  const int S = (n + kChunk - 1) / kChunk;
  return ws_bytes(B * H, S) + (ws_bytes(B * H, S) - 256);
}

bool quant_fused_pair_supported(const QuantArgs& a) {
  if (!(a.dtype == CQ_F16 && a.bits == 1 && a.d == 128 && a.n >= 1 && a.n <= (1 << 20) && (long)a.B * a.H >= 1))
    return false;
  return capacity_of((const void*)qf_b1_pair, 2) >= (a.n + kChunk - 1) / kChunk;
}

hipError_t quant_fused_pair(const QuantArgs& k, const QuantArgs& v) {
  const int units = k.B * k.H;
  const int S = (k.n + kChunk - 1) / kChunk;
  Ws wk = carve(k.ws, units, S);
  wk.spin_limit = k.spin_limit > 0 ? k.spin_limit : kSpinLimit;
  Ws wv;
  wv.status = wk.status;
  wv.spin_limit = wk.spin_limit;
  wv.slot = wk.fin + (size_t)units * 128;
  wv.fin = wv.slot + (size_t)units * S * 128;
  const void* fn = (const void*)qf_b1_pair;
  const long capacity = capacity_of(fn, 2);
  if (capacity < S) return hipErrorInvalidConfiguration;
  long grid = (capacity / S) * S;
  const long items = 2L * units * S;
  if (grid > items) grid = items;
  const long quads = 2L * units * (S + 1) * 128 / 4;     // both tensors' words
  CQ_LAUNCH(qf_init, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, k.stream, wk, quads, 1);
  const __half* xk = (const __half*)k.x;
  const __half* xv = (const __half*)v.x;
  int n = k.n, Sv = S, un = units;
  void* args[] = {(void*)&xk, (void*)&xv, (void*)&n, (void*)&un, (void*)&Sv, (void*)&k.codes, (void*)&k.scale,
                  (void*)&k.minv, (void*)&v.codes, (void*)&v.scale, (void*)&v.minv, (void*)&wk, (void*)&wv};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kWaves * 64), args, 0, k.stream);
}

hipError_t quant_fused(const QuantArgs& a) {
  const int units = a.B * a.H;
  const int S = (a.n + kChunk - 1) / kChunk;
  Ws w = carve(a.ws, units, S);
  w.spin_limit = a.spin_limit > 0 ? a.spin_limit : kSpinLimit;
  const void* fn = a.layout == CQ_LAYOUT_K ? (const void*)qf_b1<CQ_LAYOUT_K> : (const void*)qf_b1<CQ_LAYOUT_V>;
  const long capacity = capacity_of(fn, a.layout == CQ_LAYOUT_K ? 0 : 1);
  if (capacity < S) return hipErrorInvalidConfiguration;
  long grid = (capacity / S) * S;
  const long items = (long)units * S;
  if (grid > items) grid = items;
  const long quads = (long)units * (S + 1) * 128 / 4;
  CQ_LAUNCH(qf_init, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, a.stream, w, quads, a.reset_status);
  const __half* x = (const __half*)a.x;
  int n = a.n, Sv = S, un = units;
  void* args[] = {(void*)&x, (void*)&n, (void*)&un, (void*)&Sv, (void*)&a.codes, (void*)&a.scale,
                  (void*)&a.minv, (void*)&w};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kWaves * 64), args, 0, a.stream);
}

}  // namespace cqi
