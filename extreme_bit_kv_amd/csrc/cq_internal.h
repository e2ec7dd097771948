// Internal launch interface between the C-ABI layer (cq_api.cpp) and the
// kernel translation units.  Host-side only; no HIP kernel code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/cq.h"

namespace cqi {

constexpr int kHeadDim = 128;    // head dimension implemented by the kernels

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch and return the launch status from the enclosing function on failure.
#define CQ_LAUNCH(...)                                 \
  do {                                                 \
    hipLaunchKernelGGL(__VA_ARGS__);                   \
    hipError_t cq_launch_err_ = hipGetLastError();     \
    if (cq_launch_err_ != hipSuccess) return cq_launch_err_; \
  } while (0)

// ---- quantization -------------------------------------------------------
struct QuantArgs {
  const void* x;
  int dtype;            // cq_dtype
  int B, H, n, d, bits, layout;
  uint32_t* codes;
  float* scale;
  float* minv;
  void* ws;             // first kWsHeader bytes: the status word, then the path's own data
  hipStream_t stream;
  long spin_limit = 0;  // fused path: unsuccessful polls before giving up; 0 = default
  int reset_status = 1; // 0: keep the status word (the second tensor of a pair)
};
constexpr size_t kWsHeader = 256;   // quantization workspace header (status word at offset 0)
size_t quant_generic_ws(int B, int H, int n, int d);
hipError_t quant_generic(const QuantArgs& a);

size_t quant_fused_ws(int B, int H, int n, int d);
bool quant_fused_supported(const QuantArgs& a);
hipError_t quant_fused(const QuantArgs& a);
// K (CQ_LAYOUT_K) and V (CQ_LAYOUT_V) of one layer in one launch; k.ws holds both tensors' words
size_t quant_fused_pair_ws(int B, int H, int n, int d);
bool quant_fused_pair_supported(const QuantArgs& a);
hipError_t quant_fused_pair(const QuantArgs& k, const QuantArgs& v);

// ---- chunked prefill: range update and row quantization ----------------
struct RowsArgs {
  const void* x;        // [B][H][x_rows][d]
  int dtype;            // cq_dtype
  int B, H;
  long x_rows;
  int t0, m, d;         // rows [t0, t0 + m) of every (b, h)
  hipStream_t stream;
};
hipError_t range_update(const RowsArgs& a, float* mn, float* mx, int reset, uint32_t* grew);
hipError_t quant_rows(const RowsArgs& a, int bits, int layout, const float* mn, const float* mx,
                      const uint32_t* unit_mask, int n_codes, uint32_t* codes, float* scale, float* minv);
hipError_t quant_rows_generic(const RowsArgs& a, int bits, int layout, const float* mn, const float* mx,
                              const uint32_t* unit_mask, int n_codes, uint32_t* codes, float* scale, float* minv);

// ---- decode -------------------------------------------------------------
struct DecodeArgs {
  const void* q;
  int q_dtype;
  const uint32_t* k_codes;
  const float* k_scale;
  const float* k_min;
  const uint32_t* v_codes;
  const float* v_scale;
  const float* v_min;
  const void* k_tail;
  const void* v_tail;
  int tail_dtype;
  int B, Hq, Hkv, n, T, d, bits;
  int nc;               // token capacity of the code buffers (>= n; their layout is that of nc tokens)
  float sm_scale;
  int calib_on;
  float a_lo, c_lo, a_hi, c_hi;
  void* out;
  int out_dtype;
  void* ws;
  int splits;           // generic path: 0 = automatic
  hipStream_t stream;
};
int decode_generic_splits(int n, int units, int requested);
size_t decode_generic_ws(int B, int Hq, int Hkv, int n, int T, int d, int splits);
hipError_t decode_generic(const DecodeArgs& a);

// b = 1, keys read once with the visual scores kept in registers (one 8-wave
// workgroup per CU walking its units, the value pass of one unit beside the key
// pass of the next)
bool decode_pipe_supported(const DecodeArgs& a);
hipError_t decode_pipe(const DecodeArgs& a);

// Per-device fixed scratch of the entry points that allocate nothing: its
// device address on the current device (resolved once per device).
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t scratch_address(void** out);

// b = 1, every code tile of a unit in flight at once (n <= 8192, T <= 256;
// one 8-wave workgroup per unit, at most one unit per CU)
bool decode_wide_supported(const DecodeArgs& a);
bool decode_wide_preferred(const DecodeArgs& a);   // the automatic choice
hipError_t decode_wide(const DecodeArgs& a);

// b = 1, visual scores kept in LDS (one 16-wave workgroup per CU walking its units)
bool decode_lds_supported(const DecodeArgs& a);
bool decode_lds_preferred(const DecodeArgs& a);   // the automatic choice
hipError_t decode_lds(const DecodeArgs& a);

size_t decode_fast_ws(int B, int Hq, int Hkv, int n, int T, int d);
bool decode_fast_supported(const DecodeArgs& a);
hipError_t decode_fast(const DecodeArgs& a);

// b = 1 as two launches over token chunks; `requested` chunks per unit, 0 = automatic
bool decode_split_supported(const DecodeArgs& a);
bool decode_split_preferred(const DecodeArgs& a, bool one_ok);   // the automatic choice
size_t decode_split_ws(int B, int Hkv, int n, int T, int requested);
size_t decode_split_ws_max(int B, int Hkv, int n, int T);
hipError_t decode_split(const DecodeArgs& a, int requested);

// visual scores only (generic kernel), float32 [B][Hq][n]
hipError_t visual_scores(const void* q, int q_dtype, const uint32_t* k_codes, const float* k_scale,
                         const float* k_min, int B, int Hq, int Hkv, int n, int bits, float sm_scale,
                         float* scores, hipStream_t st);

// ---- calibration --------------------------------------------------------
hipError_t calibrate_rows(const float* scores, int R, int n, int enabled, float a_lo, float c_lo,
                          float a_hi, float c_hi, float* out, float* row_minmax, hipStream_t st);

// ---- fp16 baseline ------------------------------------------------------
size_t decode_fp16_ws(int B, int Hq, int Hkv, int N, int d);
hipError_t decode_fp16(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N,
                       int d, float sm_scale, void* out, void* ws, hipStream_t st);
hipError_t scores_fp16(const void* q, const void* k, int B, int Hq, int Hkv, int N, float sm_scale, float* scores,
                       hipStream_t st);

}  // namespace cqi
