// C ABI of libcq: argument validation, path selection, workspace carving and
// launches.  Every entry point validates before enqueuing anything, returns a
// cq_status and never throws.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "../../include/cq.h"
#include "cq_internal.h"

namespace {

bool valid_bits(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }
bool valid_dtype(int32_t t) { return t == CQ_F16 || t == CQ_F32; }
// bulk buffers are read and written with 16-byte vector accesses
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
int opt_path(const cq_opts* o) { return o ? o->path : CQ_PATH_AUTO; }
long opt_polls(const cq_opts* o) { return o ? (long)o->max_polls : 0L; }

thread_local int32_t g_last_hip_error = 0;

cq_status from_hip(hipError_t e) {
  if (e == hipSuccess) return CQ_OK;
  g_last_hip_error = (int32_t)e;
  return CQ_ERR_HIP;
}

// A HIP error left pending by earlier, unrelated calls of the same thread
// (for instance from the framework that owns the tensors) must not be
// reported as a failure of this library's launches.
void clear_stale_hip_error() { (void)hipGetLastError(); }

// Size of a tensor of `count` elements must fit a signed 64-bit byte count
// and every per-(batch, head) index the kernels form in 32 bits.
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
  if (a < 0 || b < 0 || c < 0 || d < 0) return false;
  const int64_t lim = (int64_t)1 << 31;
  if (c * d >= lim) return false;                       // per-unit element count
  return a * b < lim;
}

}  // namespace

extern "C" {

int32_t cq_abi_version(void) { return CQ_ABI_VERSION; }

int32_t cq_last_hip_error(void) { return g_last_hip_error; }

const char* cq_status_str(cq_status s) {
  switch (s) {
    case CQ_OK: return "CQ_OK";
    case CQ_ERR_INVALID_ARG: return "CQ_ERR_INVALID_ARG: invalid argument";
    case CQ_ERR_UNSUPPORTED: return "CQ_ERR_UNSUPPORTED: valid arguments not supported by this build";
    case CQ_ERR_WORKSPACE: return "CQ_ERR_WORKSPACE: workspace missing or too small";
    case CQ_ERR_HIP: return "CQ_ERR_HIP: HIP runtime call failed";
    case CQ_ERR_TIMEOUT: return "CQ_ERR_TIMEOUT: a quantize workgroup gave up waiting; its outputs are invalid";
  }
  return "unknown cq_status";
}

// ---------------------------------------------------------------------------
size_t cq_quantize_kv_workspace(int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits) {
  if (!fits(B, H, n, d) || d <= 0 || !valid_bits(bits)) return 0;
  size_t g = cqi::quant_generic_ws(B, H, n, d);
  size_t f = cqi::quant_fused_ws(B, H, n, d);
  return g > f ? g : f;
}

cq_status cq_quantize_kv(const void* x, cq_dtype x_dtype, int32_t B, int32_t H, int32_t n, int32_t d,
                         int32_t bits, cq_layout layout, uint32_t* codes, float* scale, float* minv,
                         void* workspace, size_t workspace_bytes, const cq_opts* opts, void* stream) {
  if (!fits(B, H, n, d) || d <= 0 || !valid_bits(bits) || !valid_dtype(x_dtype) ||
      (layout != CQ_LAYOUT_K && layout != CQ_LAYOUT_V))
    return CQ_ERR_INVALID_ARG;
  if ((d * bits) % 32 != 0) return CQ_ERR_INVALID_ARG;
  const int path = opt_path(opts);
  if (path < CQ_PATH_AUTO || path > CQ_PATH_FAST_WIDE || opt_polls(opts) < 0) return CQ_ERR_INVALID_ARG;
  const int64_t units = (int64_t)B * H;
  if (units > 0) {
    if (scale == nullptr || minv == nullptr) return CQ_ERR_INVALID_ARG;
    if (n > 0 && (x == nullptr || codes == nullptr)) return CQ_ERR_INVALID_ARG;
    if (!al16(x) || !al16(codes) || !al4(scale) || !al4(minv) || !al16(workspace)) return CQ_ERR_INVALID_ARG;
  }
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  cqi::QuantArgs a{x, x_dtype, B, H, n, d, bits, layout, codes, scale, minv, workspace, (hipStream_t)stream,
                   opt_polls(opts), 1};
  const bool fused_ok = cqi::quant_fused_supported(a);
  if (path >= CQ_PATH_FAST && !fused_ok) return CQ_ERR_UNSUPPORTED;
  const bool use_fused = fused_ok && path != CQ_PATH_GENERIC;
  const size_t need = use_fused ? cqi::quant_fused_ws(B, H, n, d) : cqi::quant_generic_ws(B, H, n, d);
  if (need > 0 && units > 0 && n > 0 && (workspace == nullptr || workspace_bytes < need)) return CQ_ERR_WORKSPACE;
  clear_stale_hip_error();
  return from_hip(use_fused ? cqi::quant_fused(a) : cqi::quant_generic(a));
}

// ---------------------------------------------------------------------------
size_t cq_quantize_kv_pair_workspace(int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits) {
  if (!fits(B, H, n, d) || d <= 0 || !valid_bits(bits)) return 0;
  const size_t one = cq_quantize_kv_workspace(B, H, n, d, bits);
  const size_t pair = cqi::quant_fused_pair_ws(B, H, n, d);
  return one > pair ? one : pair;
}

cq_status cq_quantize_kv_pair(const void* k, const void* v, cq_dtype x_dtype, int32_t B, int32_t H, int32_t n,
                              int32_t d, int32_t bits, uint32_t* k_codes, float* k_scale, float* k_min,
                              uint32_t* v_codes, float* v_scale, float* v_min, void* workspace,
                              size_t workspace_bytes, const cq_opts* opts, void* stream) {
  if (!fits(B, H, n, d) || d <= 0 || !valid_bits(bits) || !valid_dtype(x_dtype)) return CQ_ERR_INVALID_ARG;
  if ((d * bits) % 32 != 0) return CQ_ERR_INVALID_ARG;
  const int path = opt_path(opts);
  if (path < CQ_PATH_AUTO || path > CQ_PATH_FAST_WIDE || opt_polls(opts) < 0) return CQ_ERR_INVALID_ARG;
  const int64_t units = (int64_t)B * H;
  if (units > 0) {
    if (k_scale == nullptr || k_min == nullptr || v_scale == nullptr || v_min == nullptr) return CQ_ERR_INVALID_ARG;
    if (n > 0 && (k == nullptr || v == nullptr || k_codes == nullptr || v_codes == nullptr)) return CQ_ERR_INVALID_ARG;
    if (!al16(k) || !al16(v) || !al16(k_codes) || !al16(v_codes) || !al4(k_scale) || !al4(k_min) ||
        !al4(v_scale) || !al4(v_min) || !al16(workspace))
      return CQ_ERR_INVALID_ARG;
  }
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  cqi::QuantArgs ka{k, x_dtype, B, H, n, d, bits, CQ_LAYOUT_K, k_codes, k_scale, k_min, workspace,
                    (hipStream_t)stream, opt_polls(opts), 1};
  // the V tensor, run after K on the same workspace, keeps K's status word
  cqi::QuantArgs va{v, x_dtype, B, H, n, d, bits, CQ_LAYOUT_V, v_codes, v_scale, v_min, workspace,
                    (hipStream_t)stream, opt_polls(opts), 0};
  const bool pair_ok = cqi::quant_fused_pair_supported(ka) && path != CQ_PATH_GENERIC;
  if (pair_ok) {
    const size_t need = cqi::quant_fused_pair_ws(B, H, n, d);
    if (workspace == nullptr || workspace_bytes < need) return CQ_ERR_WORKSPACE;
    clear_stale_hip_error();
    return from_hip(cqi::quant_fused_pair(ka, va));
  }
  // one tensor after the other, sharing the workspace (stream order keeps them apart)
  const bool fused_ok = cqi::quant_fused_supported(ka) && cqi::quant_fused_supported(va);
  if (path >= CQ_PATH_FAST && !fused_ok) return CQ_ERR_UNSUPPORTED;
  const bool use_fused = fused_ok && path != CQ_PATH_GENERIC;
  const size_t need = use_fused ? cqi::quant_fused_ws(B, H, n, d) : cqi::quant_generic_ws(B, H, n, d);
  if (need > 0 && units > 0 && n > 0 && (workspace == nullptr || workspace_bytes < need)) return CQ_ERR_WORKSPACE;
  clear_stale_hip_error();
  const hipError_t e = use_fused ? cqi::quant_fused(ka) : cqi::quant_generic(ka);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(use_fused ? cqi::quant_fused(va) : cqi::quant_generic(va));
}

cq_status cq_quantize_status(const void* workspace, void* stream) {
  if (workspace == nullptr || !al16(workspace)) return CQ_ERR_INVALID_ARG;
  clear_stale_hip_error();
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return from_hip(e);
  return word == 0 ? CQ_OK : CQ_ERR_TIMEOUT;
}

// ---------------------------------------------------------------------------
cq_status cq_kv_range_update(const void* x, cq_dtype x_dtype, int32_t B, int32_t H, int32_t x_rows, int32_t t0,
                             int32_t m, int32_t d, float* mn, float* mx, int32_t reset, uint32_t* grew,
                             void* stream) {
  if (!fits(B, H, x_rows, d) || d <= 0 || !valid_dtype(x_dtype) || t0 < 0 || m < 0 ||
      (int64_t)t0 + m > x_rows || (reset != 0 && reset != 1))
    return CQ_ERR_INVALID_ARG;
  if (reset && m == 0) return CQ_ERR_INVALID_ARG;                 // a range needs a row
  const int64_t units = (int64_t)B * H;
  if (units > 0) {
    if (mn == nullptr || mx == nullptr || (m > 0 && x == nullptr)) return CQ_ERR_INVALID_ARG;
    if (!al16(x) || !al4(mn) || !al4(mx) || !al4(grew)) return CQ_ERR_INVALID_ARG;
  }
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  cqi::RowsArgs a{x, x_dtype, B, H, (long)x_rows, t0, m, d, (hipStream_t)stream};
  clear_stale_hip_error();
  return from_hip(cqi::range_update(a, mn, mx, reset, grew));
}

cq_status cq_quantize_kv_rows(const void* x, cq_dtype x_dtype, int32_t B, int32_t H, int32_t x_rows, int32_t t0,
                              int32_t m, int32_t d, int32_t bits, cq_layout layout, const float* mn, const float* mx,
                              const uint32_t* unit_mask, int32_t n, uint32_t* codes, float* scale, float* minv,
                              void* stream) {
  if (!fits(B, H, x_rows, d) || !fits(B, H, n, d) || d <= 0 || !valid_bits(bits) || !valid_dtype(x_dtype) ||
      (layout != CQ_LAYOUT_K && layout != CQ_LAYOUT_V))
    return CQ_ERR_INVALID_ARG;
  if ((d * bits) % 32 != 0 || t0 < 0 || m < 0 || (int64_t)t0 + m > n || (int64_t)t0 + m > x_rows)
    return CQ_ERR_INVALID_ARG;
  if (t0 % 32 != 0 || (m % 32 != 0 && t0 + m != n)) return CQ_ERR_INVALID_ARG;   // whole V words per call
  const int64_t units = (int64_t)B * H;
  if (units > 0 && m > 0) {
    if (x == nullptr || codes == nullptr || mn == nullptr || mx == nullptr || scale == nullptr || minv == nullptr)
      return CQ_ERR_INVALID_ARG;
    if (!al16(x) || !al16(codes) || !al4(mn) || !al4(mx) || !al4(unit_mask) || !al4(scale) || !al4(minv))
      return CQ_ERR_INVALID_ARG;
  }
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  cqi::RowsArgs a{x, x_dtype, B, H, (long)x_rows, t0, m, d, (hipStream_t)stream};
  clear_stale_hip_error();
  return from_hip(cqi::quant_rows(a, bits, layout, mn, mx, unit_mask, n, codes, scale, minv));
}

// ---------------------------------------------------------------------------
size_t cq_decode_attn_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t T, int32_t d,
                                int32_t bits) {
  if (!fits(B, Hq, n, d) || !fits(B, Hkv, T, d) || Hkv <= 0 || Hq % Hkv != 0 || !valid_bits(bits)) return 0;
  // enough for any split count a caller may request (the path clamps it)
  int S = cqi::decode_generic_splits(n, B * Hkv, 1 << 30);
  size_t g = cqi::decode_generic_ws(B, Hq, Hkv, n, T, d, S);
  size_t f = cqi::decode_fast_ws(B, Hq, Hkv, n, T, d);
  size_t c = bits == 1 ? cqi::decode_split_ws_max(B, Hkv, n, T) : 0;   // any chunk count
  size_t m = g > f ? g : f;
  return m > c ? m : c;
}

static_assert(CQ_NOALLOC_SCRATCH_BYTES == cqi::kScratchBytes, "scratch size of the header and the library");

namespace {

// cq_decode_attn and cq_decode_attn_noalloc; with `fixed_scratch` the
// workspace is the device's fixed scratch array (the caller's pointer is NULL).
cq_status decode_entry(const void* q, cq_dtype q_dtype, const uint32_t* k_codes, const float* k_scale,
                       const float* k_min, const uint32_t* v_codes, const float* v_scale, const float* v_min,
                       const void* k_tail, const void* v_tail, cq_dtype tail_dtype, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t n, int32_t T, int32_t d, int32_t bits, float sm_scale,
                       const cq_calib* calib, void* out, cq_dtype out_dtype, void* workspace,
                       size_t workspace_bytes, bool fixed_scratch, const cq_opts* opts, void* stream) {
  if (!fits(B, Hq, n, d) || !fits(B, Hkv, T, d) || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || d <= 0 ||
      !valid_bits(bits) || !valid_dtype(q_dtype) || !valid_dtype(out_dtype) || !valid_dtype(tail_dtype))
    return CQ_ERR_INVALID_ARG;
  if ((d * bits) % 32 != 0 || n + (int64_t)T < 1) return CQ_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return CQ_ERR_INVALID_ARG;
  const int path = opt_path(opts);
  if (path < CQ_PATH_AUTO || path > CQ_PATH_FAST_WIDE || (opts && opts->splits < 0)) return CQ_ERR_INVALID_ARG;
  // token capacity of the code buffers: the first n of n_cap tokens are attended over
  const int32_t n_cap = opts && opts->n_cap != 0 ? opts->n_cap : n;
  if (n_cap < n || !fits(B, Hkv, n_cap, d) || (n_cap != n && n_cap % 32 != 0)) return CQ_ERR_INVALID_ARG;
  if (B > 0) {
    if (q == nullptr || out == nullptr) return CQ_ERR_INVALID_ARG;
    if (n > 0 && (k_codes == nullptr || k_scale == nullptr || k_min == nullptr || v_codes == nullptr ||
                  v_scale == nullptr || v_min == nullptr))
      return CQ_ERR_INVALID_ARG;
    if (T > 0 && (k_tail == nullptr || v_tail == nullptr)) return CQ_ERR_INVALID_ARG;
    if (!al16(k_codes) || !al16(v_codes) || !al16(k_tail) || !al16(v_tail) || !al16(workspace) ||
        !al4(k_scale) || !al4(k_min) || !al4(v_scale) || !al4(v_min) || !al4(q) || !al4(out))
      return CQ_ERR_INVALID_ARG;
  }
  if (T == 0 && (k_tail != nullptr || v_tail != nullptr)) return CQ_ERR_INVALID_ARG;
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  if (Hq / Hkv > 8) return CQ_ERR_UNSUPPORTED;
  cqi::DecodeArgs a{};
  a.q = q; a.q_dtype = q_dtype;
  a.k_codes = k_codes; a.k_scale = k_scale; a.k_min = k_min;
  a.v_codes = v_codes; a.v_scale = v_scale; a.v_min = v_min;
  a.k_tail = k_tail; a.v_tail = v_tail; a.tail_dtype = tail_dtype;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.n = n; a.T = T; a.d = d; a.bits = bits; a.nc = n_cap;
  a.sm_scale = sm_scale;
  a.calib_on = (calib != nullptr && calib->enabled) ? 1 : 0;
  if (a.calib_on) { a.a_lo = calib->a_lo; a.c_lo = calib->c_lo; a.a_hi = calib->a_hi; a.c_hi = calib->c_hi; }
  a.out = out; a.out_dtype = out_dtype;
  a.ws = workspace;
  a.splits = opts ? opts->splits : 0;
  a.stream = (hipStream_t)stream;
  const bool one_ok = cqi::decode_fast_supported(a);
  const bool split_ok = cqi::decode_split_supported(a);
  const bool pipe_ok = cqi::decode_pipe_supported(a);
  enum { kGeneric, kOne, kSplit, kLds, kPipe, kWide } use = kGeneric;
  if (path == CQ_PATH_FAST_WIDE) {
    if (!cqi::decode_wide_supported(a)) return CQ_ERR_UNSUPPORTED;
    use = kWide;
  } else if (path == CQ_PATH_FAST_LDS) {
    if (!cqi::decode_lds_supported(a)) return CQ_ERR_UNSUPPORTED;
    use = kLds;
  } else if (path == CQ_PATH_FAST_PIPE) {
    if (!pipe_ok) return CQ_ERR_UNSUPPORTED;
    use = kPipe;
  } else if (path == CQ_PATH_FAST_ONE) {
    if (!one_ok) return CQ_ERR_UNSUPPORTED;
    use = kOne;
  } else if (path == CQ_PATH_FAST_SPLIT) {
    if (!split_ok) return CQ_ERR_UNSUPPORTED;
    use = kSplit;
  } else if (path == CQ_PATH_FAST || (path == CQ_PATH_AUTO && !(opts && opts->splits > 0))) {
    if (cqi::decode_wide_preferred(a)) use = kWide;
    else if (cqi::decode_lds_preferred(a)) use = kLds;
    else if (cqi::decode_split_preferred(a, one_ok)) use = kSplit;
    else if (one_ok) use = kOne;
    else if (path == CQ_PATH_FAST) return CQ_ERR_UNSUPPORTED;
  }
  const int req = use == kSplit && path == CQ_PATH_FAST_SPLIT ? a.splits : 0;
  size_t need;
  if (use == kPipe || use == kWide) need = 0;
  else if (use == kOne || use == kLds) need = cqi::decode_fast_ws(B, Hq, Hkv, n, T, d);
  else if (use == kSplit) need = cqi::decode_split_ws(B, Hkv, n, T, req);
  else need = cqi::decode_generic_ws(B, Hq, Hkv, n, T, d, cqi::decode_generic_splits(n, B * Hkv, a.splits));
  if (fixed_scratch) {
    if (need > cqi::kScratchBytes) return CQ_ERR_WORKSPACE;
    if (B > 0) {
      clear_stale_hip_error();
      void* ptr = nullptr;
      const hipError_t e = cqi::scratch_address(&ptr);
      if (e != hipSuccess) return from_hip(e);
      a.ws = ptr;
    }
  } else if (B > 0 && need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return CQ_ERR_WORKSPACE;
  }
  clear_stale_hip_error();
  if (use == kPipe) return from_hip(cqi::decode_pipe(a));
  if (use == kWide) return from_hip(cqi::decode_wide(a));
  if (use == kLds) return from_hip(cqi::decode_lds(a));
  if (use == kOne) return from_hip(cqi::decode_fast(a));
  if (use == kSplit) return from_hip(cqi::decode_split(a, req));
  return from_hip(cqi::decode_generic(a));
}

}  // namespace

cq_status cq_decode_attn(const void* q, cq_dtype q_dtype, const uint32_t* k_codes, const float* k_scale,
                         const float* k_min, const uint32_t* v_codes, const float* v_scale, const float* v_min,
                         const void* k_tail, const void* v_tail, cq_dtype tail_dtype, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t n, int32_t T, int32_t d, int32_t bits, float sm_scale,
                         const cq_calib* calib, void* out, cq_dtype out_dtype, void* workspace,
                         size_t workspace_bytes, const cq_opts* opts, void* stream) {
  return decode_entry(q, q_dtype, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail, v_tail, tail_dtype, B,
                      Hq, Hkv, n, T, d, bits, sm_scale, calib, out, out_dtype, workspace, workspace_bytes, false,
                      opts, stream);
}

cq_status cq_decode_attn_noalloc(const void* q, cq_dtype q_dtype, const uint32_t* k_codes, const float* k_scale,
                                 const float* k_min, const uint32_t* v_codes, const float* v_scale,
                                 const float* v_min, const void* k_tail, const void* v_tail, cq_dtype tail_dtype,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t T, int32_t d, int32_t bits,
                                 float sm_scale, const cq_calib* calib, void* out, cq_dtype out_dtype,
                                 const cq_opts* opts, void* stream) {
  return decode_entry(q, q_dtype, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail, v_tail, tail_dtype, B,
                      Hq, Hkv, n, T, d, bits, sm_scale, calib, out, out_dtype, nullptr, 0, true, opts, stream);
}

// ---------------------------------------------------------------------------
cq_status cq_visual_scores(const void* q, cq_dtype q_dtype, const uint32_t* k_codes, const float* k_scale,
                           const float* k_min, int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t d,
                           int32_t bits, float sm_scale, float* scores, void* stream) {
  if (!fits(B, Hq, n, d) || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || d <= 0 || n < 1 || !valid_bits(bits) ||
      !valid_dtype(q_dtype) || (d * bits) % 32 != 0 || !(sm_scale == sm_scale))
    return CQ_ERR_INVALID_ARG;
  if (B > 0 && (q == nullptr || k_codes == nullptr || k_scale == nullptr || k_min == nullptr || scores == nullptr))
    return CQ_ERR_INVALID_ARG;
  if (B > 0 && (!al16(k_codes) || !al4(q) || !al4(k_scale) || !al4(k_min) || !al4(scores)))
    return CQ_ERR_INVALID_ARG;
  if (d != cqi::kHeadDim || Hq / Hkv > 8) return CQ_ERR_UNSUPPORTED;
  clear_stale_hip_error();
  return from_hip(cqi::visual_scores(q, q_dtype, k_codes, k_scale, k_min, B, Hq, Hkv, n, bits, sm_scale, scores,
                                     (hipStream_t)stream));
}

cq_status cq_scores_fp16(const void* q, const void* k, int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                         float sm_scale, float* scores, void* stream) {
  if (!fits(B, Hkv, N, d) || !fits(B, Hq, N, 1) || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || N < 1 || d <= 0 ||
      !(sm_scale == sm_scale))
    return CQ_ERR_INVALID_ARG;
  if (B > 0 && (q == nullptr || k == nullptr || scores == nullptr)) return CQ_ERR_INVALID_ARG;
  if (B > 0 && (!al16(k) || !al4(q) || !al4(scores))) return CQ_ERR_INVALID_ARG;
  if (d != cqi::kHeadDim || Hq / Hkv > 8) return CQ_ERR_UNSUPPORTED;
  clear_stale_hip_error();
  return from_hip(cqi::scores_fp16(q, k, B, Hq, Hkv, N, sm_scale, scores, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
cq_status cq_calibrate(const float* scores, int32_t R, int32_t n, const cq_calib* calib, float* out,
                       float* row_minmax, void* stream) {
  if (R < 0 || n < 1 || (int64_t)R * n >= ((int64_t)1 << 40) || calib == nullptr) return CQ_ERR_INVALID_ARG;
  if (R > 0 && (scores == nullptr || out == nullptr)) return CQ_ERR_INVALID_ARG;
  clear_stale_hip_error();
  return from_hip(cqi::calibrate_rows(scores, R, n, calib->enabled, calib->a_lo, calib->c_lo, calib->a_hi,
                                      calib->c_hi, out, row_minmax, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
size_t cq_decode_attn_fp16_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d) {
  if (!fits(B, Hkv, N, d) || Hkv <= 0 || Hq % Hkv != 0 || N < 1) return 0;
  return cqi::decode_fp16_ws(B, Hq, Hkv, N, d);
}

cq_status cq_decode_attn_fp16(const void* q, const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t N, int32_t d, float sm_scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!fits(B, Hkv, N, d) || !fits(B, Hq, 1, d) || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || N < 1 || d <= 0)
    return CQ_ERR_INVALID_ARG;
  if (B > 0 && (q == nullptr || k == nullptr || v == nullptr || out == nullptr)) return CQ_ERR_INVALID_ARG;
  if (B > 0 && (!al16(k) || !al16(v) || !al16(workspace) || !al4(q) || !al4(out))) return CQ_ERR_INVALID_ARG;
  if (d != cqi::kHeadDim) return CQ_ERR_UNSUPPORTED;
  if (Hq / Hkv > 8) return CQ_ERR_UNSUPPORTED;
  const size_t need = cqi::decode_fp16_ws(B, Hq, Hkv, N, d);
  if (B > 0 && (workspace == nullptr || workspace_bytes < need)) return CQ_ERR_WORKSPACE;
  clear_stale_hip_error();
  return from_hip(cqi::decode_fp16(q, k, v, B, Hq, Hkv, N, d, sm_scale, out, workspace, (hipStream_t)stream));
}

}  // extern "C"
