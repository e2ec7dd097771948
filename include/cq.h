/*
 * cq.h — C ABI of libcq, a gfx950 (MI355X) implementation of the CalibQuant
 * visual-KV decode path: channel-wise b-bit quantization of the visual KV
 * cache, decode attention that reads only the packed integer codes with the
 * per-channel scale and minimum folded into the query and the output
 * ("post-scaling"), and the calibration map g on the pre-softmax scores.
 *
 * Sources (cited by page title and section):
 *   [ART] QbitAI article on CalibQuant, "在 InternVL-2.5 上达成 10 倍吞吐量提升",
 *         section "Method": part 1 channel-wise KV-cache quantization,
 *         part 2 post-scaling KV-cache management, part 3 post-quantization
 *         calibration.
 *   [ABS] "CalibQuant: 1-Bit KV Cache Quantization for Multimodal LLMs",
 *         abstract (papers.pytorch.kr): plug-and-play, visual-cache
 *         quantization, 1-bit, Triton runtime.
 *
 * Conventions for every entry point:
 *   - Pointers named as device buffers are device pointers (hipMalloc'd or
 *     torch CUDA tensors), caller-allocated and caller-owned; all tensors are
 *     contiguous, row-major, in the shapes given.  `calib` and `opts` are host
 *     pointers.  The library never allocates or frees device memory and keeps
 *     no state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are visible after the stream
 *     is synchronized.  Calls that share a workspace must not overlap.
 *   - Arguments are validated before anything is enqueued.  On a non-CQ_OK
 *     status nothing has been enqueued and no output byte has been written.
 *     CQ_ERR_HIP means a HIP launch call failed (work enqueued before the
 *     failing launch may still run).  Faults inside kernels surface at the
 *     caller's next synchronization, as for any HIP kernel.
 *   - Alignment: bulk device buffers (x, code words, tails, the fp16
 *     baseline's k and v, workspaces) must be 16-byte aligned, every other
 *     device pointer 4-byte aligned (torch allocations are 256-byte
 *     aligned); CQ_ERR_INVALID_ARG otherwise.
 *   - No C++ exception crosses the ABI.
 *
 * Packed code format (this library's storage format; the pages only say that
 * the cache keeps b-bit integer codes plus a per-channel scale and bias):
 *   b in {1,2,4,8}; L = 2^b - 1; E = 32/b codes per 32-bit word.  Element e
 *   (0 <= e < E) of a word occupies bits [off(e), off(e)+b) with
 *        off(e) = 8*(e mod 4) + b*floor(e/4),
 *   so (word >> (b*s)) & (L*0x01010101) yields elements 4s..4s+3 in bytes 0..3.
 *   CQ_LAYOUT_K  codes[B][H][W][n], W = d*b/32: word (b,h,w,i) holds channels
 *                w*E .. w*E+E-1 of token i.
 *   CQ_LAYOUT_V  codes[B][H][R][d], R = ceil(n/E): word (b,h,r,j) holds tokens
 *                r*E .. r*E+E-1 of channel j; bits of tokens >= n are 0.
 *   K is contracted over channels and V over tokens, so each layout keeps the
 *   contraction index inside a word.
 */
#ifndef CQ_H
#define CQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CQ_ABI_VERSION 3

typedef enum {
  CQ_OK = 0,
  CQ_ERR_INVALID_ARG = 1,   /* NULL pointer, negative or inconsistent size, bad enum */
  CQ_ERR_UNSUPPORTED = 2,   /* valid arguments this build does not implement (e.g. d != 128) */
  CQ_ERR_WORKSPACE = 3,     /* workspace pointer NULL or smaller than the query returned */
  CQ_ERR_HIP = 4,           /* a HIP runtime call failed */
  CQ_ERR_TIMEOUT = 5        /* cq_quantize_status: a workgroup of the last quantize call on the
                               workspace gave up waiting; that call's outputs are invalid */
} cq_status;

typedef enum { CQ_F16 = 0, CQ_F32 = 1 } cq_dtype;

typedef enum { CQ_LAYOUT_K = 0, CQ_LAYOUT_V = 1 } cq_layout;

/* Calibration map g ([ART] Method part 3).  For each query head the visual
 * pre-softmax scores s_i (already multiplied by sm_scale) span [m, M]; g is
 * the affine map sending [m, M] onto [t_lo, t_hi] with
 *     t_lo = a_lo*m + c_lo,   t_hi = a_hi*M + c_hi,
 * i.e. g(s) = t_lo + (s - m)*(t_hi - t_lo)/(M - m), and g(s) = t_lo if M == m.
 * The pages lost g's formula and parameters; this endpoint form covers both a
 * relative target (a = tau, c = 0) and a fixed one (a = 0).  Text-tail scores
 * are not calibrated.  enabled == 0 means g is the identity. */
typedef struct {
  int32_t enabled;
  float a_lo, c_lo;
  float a_hi, c_hi;
} cq_calib;

/* Execution path selection, for tests and tuning (NULL opts = automatic).
 * CQ_PATH_FAST picks one of the matrix-core decode schedules itself: at b = 1,
 * when every (batch, kv head) unit gets a CU of its own and at least half the
 * CUs stay free (at most 128 units on a 256-CU MI355X), the all-in-flight one
 * if it takes the shape, else the LDS-score one; otherwise the split one
 * below 64 units, else the one-launch one.  The FAST_ values force one (decode only; for quantization
 * they mean CQ_PATH_FAST):
 *   CQ_PATH_FAST_ONE    one launch, one workgroup per (batch, kv head); it
 *                       keeps the scores of a unit's first key tiles in LDS
 *                       for the value pass and reads the other key tiles
 *                       again (at b > 1 those of the first 6912 tokens when
 *                       there is at most one unit per CU or n >= 4096, 6144
 *                       at b = 2, one workgroup per CU; fewer otherwise, two
 *                       per CU); the results do not depend on which;
 *   CQ_PATH_FAST_SPLIT  b = 1 only: a key-pass launch and a value-pass launch,
 *                       each over token chunks of every (batch, kv head);
 *   CQ_PATH_FAST_LDS    b = 1 only, G * ceil(n/128) <= 256 (n <= 8192 at
 *                       G = 4): one launch, one workgroup per CU walking its
 *                       (batch, kv head) units, the visual scores kept in LDS
 *                       between the key and the value pass (the keys are
 *                       read once); results equal CQ_PATH_FAST_ONE's bit for
 *                       bit.
 *   CQ_PATH_FAST_PIPE   b = 1 only, G in {1, 2, 4}, 32 <= n <= 8192, n a
 *                       multiple of 32, T <= 128: one launch of one 8-wave
 *                       workgroup per CU walking its units, the value pass of
 *                       one unit run beside the key pass of the next; the
 *                       keys are read once and the scores stay on chip.  Its
 *                       key products give CQ_PATH_FAST_ONE's scores; its sums
 *                       and tail are formed in another order, so its results
 *                       match CQ_PATH_FAST_ONE's to the 2e-3 tolerance, not
 *                       bit for bit.  Needs no workspace.
 *   CQ_PATH_FAST_WIDE   b = 1 only, G in {1, 2, 4}, n <= 4096 a multiple of
 *                       32, T <= 256: one launch, one workgroup per (batch,
 *                       kv head) that requests all of its code tiles at once
 *                       and keeps the scores in registers (the keys are read
 *                       once); meant for at most one unit per CU.  Results
 *                       equal CQ_PATH_FAST_ONE's bit for bit.  Needs no
 *                       workspace.
 * At b = 1 the one-launch, LDS-score and pipelined paths take the query as
 * four balanced base-31 digits (about 20 bits); the split path and b > 1 as a
 * 22-bit fixed-point integer. */
typedef enum {
  CQ_PATH_AUTO = 0, CQ_PATH_GENERIC = 1, CQ_PATH_FAST = 2, CQ_PATH_FAST_ONE = 3, CQ_PATH_FAST_SPLIT = 4,
  CQ_PATH_FAST_LDS = 5, CQ_PATH_FAST_PIPE = 6, CQ_PATH_FAST_WIDE = 7
} cq_path;
typedef struct {
  int32_t path;     /* cq_path; a FAST path on an unsupported shape -> CQ_ERR_UNSUPPORTED */
  int32_t splits;   /* generic decode: token splits per (batch, kv head); 0 = automatic;
                       clamped to [1, min(64, ceil(n/32))].  Under CQ_PATH_AUTO a
                       value > 0 selects the generic decode.  CQ_PATH_FAST_SPLIT:
                       chunks per (batch, kv head), 0 = automatic, rounded so that
                       a chunk is 4, 8, 16 or 32 tiles of 128 tokens. */
  int32_t max_polls; /* quantization: unsuccessful polls of a rendezvous word after
                       which a workgroup of the fused path gives up (and the call's
                       status word reads 1); 0 = the default bound of a few seconds,
                       negative -> CQ_ERR_INVALID_ARG.  A small value forces the
                       time-out path from the host (tests). */
  int32_t n_cap;    /* decode: the token capacity the visual code buffers are
                       laid out for (0 = n).  With n_cap > n the K and V words
                       are those of cq_quantize_kv / cq_quantize_kv_rows for
                       n_cap tokens ([B][Hkv][d*bits/32][n_cap] and
                       [B][Hkv][ceil(n_cap*bits/32)][d]) of which the first n
                       are attended over, so a cache that grows frame by frame
                       is decoded in place between appends.  Requires
                       n <= n_cap and n_cap % 32 == 0 when n_cap != n, else
                       CQ_ERR_INVALID_ARG; ignored by quantization. */
} cq_opts;

/* ABI version of the loaded library (CQ_ABI_VERSION).  Version 2 added
 * cq_opts.max_polls, CQ_ERR_TIMEOUT and cq_quantize_status; version 3
 * cq_opts.n_cap. */
int32_t cq_abi_version(void);

/* hipError_t of the most recent CQ_ERR_HIP returned on the calling thread
 * (0 if none).  A HIP error left pending by earlier calls of other code on the
 * thread is cleared, not reported, when an entry point starts its launches. */
int32_t cq_last_hip_error(void);

/* Human-readable name of a status code; never NULL. */
const char* cq_status_str(cq_status s);

/* ------------------------------------------------------------------------
 * cq_quantize_kv — channel-wise b-bit quantization and bit-packing of one
 * K or V cache tensor ([ART] Method part 1: uniform integer quantization with
 * the range refined per channel over the n tokens of one head; the same is
 * applied to V).
 *
 *   x         device, [B][H][n][d] of x_dtype (CQ_F16 or CQ_F32), finite values
 *   bits      1, 2, 4 or 8
 *   layout    CQ_LAYOUT_K or CQ_LAYOUT_V (see the packed format above)
 *   codes     device, uint32 words in `layout` for every (b, h)
 *   scale     device, float32 [B][H][d]: (max - min)/L, correctly rounded
 *   minv      device, float32 [B][H][d]: per-channel minimum (exact)
 *   workspace device, >= cq_quantize_kv_workspace(...) bytes (may be NULL
 *             when that is 0).  Its first 256 bytes are a header on every
 *             path; the first int32 is a status word that the call sets to 0
 *             and that a workgroup of the fused path sets to 1 if it gave up
 *             waiting for the other chunks of its (batch, head) (the outputs
 *             are then invalid).  cq_quantize_status reads it.  The second
 *             int32 is set to 1 by every call that timed out and is never
 *             cleared by the library: a caller that zeroes it once can check
 *             a whole run of calls at its end.  The fused
 *             path launches no more workgroups than the device holds at once;
 *             a time-out needs other work to keep part of the device busy
 *             for seconds (or a small opts->max_polls).  CQ_PATH_GENERIC has
 *             no such wait.
 *   The fused path takes fp16 input at b = 1 when every 512-token chunk of a
 *   (b, h) fits on the device at once (n <= 512 x the co-resident workgroups,
 *   262144 tokens on a 256-CU MI355X); otherwise CQ_PATH_AUTO uses the
 *   generic kernels and CQ_PATH_FAST returns CQ_ERR_UNSUPPORTED.
 *
 * For each (b, h, channel j) with mn = min_i x, mx = max_i x over the n tokens:
 *   code(i, j) = round-half-to-even((x_ij - mn)*L/(mx - mn)), decided exactly;
 *   code = 0 for every token of a channel with mx == mn (scale is then 0).
 * n == 0 writes scale = minv = 0 and no code word.  Requires d*b % 32 == 0.
 * ------------------------------------------------------------------------ */
size_t cq_quantize_kv_workspace(int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits);

cq_status cq_quantize_kv(const void* x, cq_dtype x_dtype,
                         int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits,
                         cq_layout layout,
                         uint32_t* codes, float* scale, float* minv,
                         void* workspace, size_t workspace_bytes,
                         const cq_opts* opts, void* stream);

/* ------------------------------------------------------------------------
 * cq_quantize_kv_pair — one layer's visual K and V in one call: the same
 * outputs as cq_quantize_kv(k, .., CQ_LAYOUT_K, k_codes, k_scale, k_min) and
 * cq_quantize_kv(v, .., CQ_LAYOUT_V, v_codes, v_scale, v_min), bit for bit
 * ([ART] Method part 1 applied to K and to V alike).
 *
 *   k, v      device, [B][H][n][d] of x_dtype each
 *   k_*, v_*  as the outputs of cq_quantize_kv for CQ_LAYOUT_K / CQ_LAYOUT_V
 *   workspace device, >= cq_quantize_kv_pair_workspace(...) bytes; its first
 *             int32 is the status word of cq_quantize_kv
 *   opts      NULL / CQ_PATH_AUTO: at b = 1 with float16 input the fused
 *             kernel takes the chunks of both tensors in one launch (one
 *             word reset, one launch); other shapes run the two tensors one
 *             after the other.  CQ_PATH_GENERIC and CQ_PATH_FAST as for
 *             cq_quantize_kv.
 * Errors and limits as for cq_quantize_kv.
 * ------------------------------------------------------------------------ */
size_t cq_quantize_kv_pair_workspace(int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits);

/* ------------------------------------------------------------------------
 * cq_quantize_status — whether the last cq_quantize_kv / cq_quantize_kv_pair
 * call on `workspace` completed every wait of its fused kernel ([ART] Method
 * part 1 takes each channel's range over all n tokens of a head, so the
 * chunks of one head meet before any code is decided).
 *
 *   workspace  device, the workspace that call used (>= 4 bytes, 16-byte
 *              aligned)
 *   stream     the stream that call was enqueued on; it is synchronized
 *              (the status word is read after all earlier work on it)
 * Returns CQ_OK when no workgroup gave up, CQ_ERR_TIMEOUT when one did (the
 * call's codes, scales and minima are then invalid), CQ_ERR_INVALID_ARG for
 * a NULL or misaligned workspace, CQ_ERR_HIP if the copy or the
 * synchronization failed.  Enqueues a 4-byte device-to-host copy; allocates
 * nothing.
 * ------------------------------------------------------------------------ */
cq_status cq_quantize_status(const void* workspace, void* stream);

cq_status cq_quantize_kv_pair(const void* k, const void* v, cq_dtype x_dtype,
                              int32_t B, int32_t H, int32_t n, int32_t d, int32_t bits,
                              uint32_t* k_codes, float* k_scale, float* k_min,
                              uint32_t* v_codes, float* v_scale, float* v_min,
                              void* workspace, size_t workspace_bytes,
                              const cq_opts* opts, void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill: quantization of a visual segment that is written chunk by
 * chunk (a chunked prefill, or video frames appended to the segment).
 * [ART] Method part 1 takes the range per channel over the tokens of one
 * head; minimum and maximum are associative, so the range merged over the
 * chunks is the segment's range, and rows coded on it are exactly the codes
 * cq_quantize_kv gives for the whole segment.  The two calls below need no
 * workspace and no rendezvous between workgroups:
 *
 *   for each chunk [t, t + m) written to the float16/float32 cache x:
 *       cq_kv_range_update(x, .., t0 = t, m, .., reset = (t == 0), grew)
 *   once the segment [0, n) is complete:
 *       cq_quantize_kv_rows(x, .., t0 = 0, m = n, .., n, codes, scale, minv)
 *
 * Codes may also be written as chunks arrive, on the range known so far;
 * a later chunk that widens a unit's range (grew = 1) makes that unit's
 * earlier codes stale, and they are written again with unit_mask = grew.
 * ------------------------------------------------------------------------ */

/* cq_kv_range_update — merge rows [t0, t0 + m) of every (b, h) into a running
 * per-channel range.
 *
 *   x       device, [B][H][x_rows][d] of x_dtype (CQ_F16 or CQ_F32), finite
 *           values; only rows [t0, t0 + m) are read (the cache being filled).
 *           x may point at row s of every (b, h) of a larger cache of x_rows
 *           rows per (b, h) (a segment that starts at row s), provided
 *           s + t0 + m <= x_rows.
 *   mn, mx  device, float32 [B][H][d], in/out: mn = min(mn, rows),
 *           mx = max(mx, rows) per channel.  reset = 1 starts a new range from
 *           the rows (the previous contents are ignored; m >= 1 required).
 *           A zero is stored as +0.
 *   grew    device, uint32 [B][H], or NULL: set to 1 where this call made some
 *           channel's range strictly wider (always 1 under reset), else 0
 *   Requires 0 <= t0, 0 <= m, t0 + m <= x_rows, d == 128 (else UNSUPPORTED).
 *   m == 0 without reset only clears grew.  Calls on the same mn/mx must not
 *   overlap (each call's result is exact whatever its own order of updates).
 */
cq_status cq_kv_range_update(const void* x, cq_dtype x_dtype,
                             int32_t B, int32_t H, int32_t x_rows,
                             int32_t t0, int32_t m, int32_t d,
                             float* mn, float* mx, int32_t reset,
                             uint32_t* grew, void* stream);

/* cq_quantize_kv_rows — codes of rows [t0, t0 + m) of every (b, h) on a GIVEN
 * per-channel range, written into a code buffer laid out for n tokens.
 *
 *   x         device, [B][H][x_rows][d] of x_dtype, finite values; may point
 *             at row s of a larger cache as for cq_kv_range_update
 *   bits, layout  as for cq_quantize_kv
 *   mn, mx    device, float32 [B][H][d]: the range (e.g. from
 *             cq_kv_range_update); a channel with mx <= mn gets code 0 and
 *             scale 0
 *   unit_mask device, uint32 [B][H], or NULL: units with mask 0 are skipped
 *             (none of their words, scale or minv is written)
 *   codes     device, words in `layout` for n tokens per (b, h), as
 *             cq_quantize_kv writes them; only the words of rows
 *             [t0, t0 + m) are written
 *   scale     device, float32 [B][H][d]: (mx - mn)/L correctly rounded
 *   minv      device, float32 [B][H][d]: mn
 *   code(i, j) = round-half-to-even((x_ij - mn_j)*L/(mx_j - mn_j)) decided
 *   exactly and clamped to [0, L] (a value outside the range takes the
 *   nearest end level).  With mn/mx the range of rows [0, n) and t0 = 0,
 *   m = n, the outputs equal cq_quantize_kv's bit for bit.
 *   Requires t0 % 32 == 0, m % 32 == 0 unless t0 + m == n (a V word holds
 *   whole 32-token groups), t0 + m <= n, t0 + m <= x_rows, d*b % 32 == 0,
 *   d == 128 (else UNSUPPORTED).  m == 0 writes nothing.
 */
cq_status cq_quantize_kv_rows(const void* x, cq_dtype x_dtype,
                              int32_t B, int32_t H, int32_t x_rows,
                              int32_t t0, int32_t m, int32_t d, int32_t bits,
                              cq_layout layout,
                              const float* mn, const float* mx,
                              const uint32_t* unit_mask, int32_t n,
                              uint32_t* codes, float* scale, float* minv,
                              void* stream);

/* ------------------------------------------------------------------------
 * cq_decode_attn — one decode step of attention over a quantized visual
 * cache plus a full-precision text tail ([ART] Method parts 2 and 3; only
 * the visual cache is quantized, [ABS]).
 *
 *   q          device, [B][Hq][d] of q_dtype; query head hq reads kv head
 *              hq / (Hq/Hkv)
 *   k_codes    device, CQ_LAYOUT_K words of the visual keys   [B][Hkv][..]
 *   k_scale, k_min  device, float32 [B][Hkv][d]
 *   v_codes    device, CQ_LAYOUT_V words of the visual values [B][Hkv][..]
 *   v_scale, v_min  device, float32 [B][Hkv][d]
 *   k_tail, v_tail  device, [B][Hkv][T][d] of tail_dtype; NULL iff T == 0
 *   sm_scale   softmax scale applied to q.k (e.g. 1/sqrt(d))
 *   calib      host pointer or NULL (= calibration off)
 *   out        device, [B][Hq][d] of out_dtype
 *
 * Computes, per query head, with s_i = sm_scale*(q*k_scale).c_i + sm_scale*q.k_min
 * for visual token i (the post-scaled form of sm_scale*q.k_hat_i),
 * s^t_j = sm_scale*q.kt_j for tail token j, and p = softmax([g(s), s^t]):
 *   out = v_scale * (sum_i p_i c^V_i) + (sum_i p_i)*v_min + sum_j p^t_j vt_j.
 * Accumulation is float32.  Requires n + T >= 1, Hq % Hkv == 0, d == 128.
 * ------------------------------------------------------------------------ */
size_t cq_decode_attn_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n,
                                int32_t T, int32_t d, int32_t bits);

cq_status cq_decode_attn(const void* q, cq_dtype q_dtype,
                         const uint32_t* k_codes, const float* k_scale, const float* k_min,
                         const uint32_t* v_codes, const float* v_scale, const float* v_min,
                         const void* k_tail, const void* v_tail, cq_dtype tail_dtype,
                         int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t T,
                         int32_t d, int32_t bits, float sm_scale,
                         const cq_calib* calib,
                         void* out, cq_dtype out_dtype,
                         void* workspace, size_t workspace_bytes,
                         const cq_opts* opts, void* stream);

/* ------------------------------------------------------------------------
 * cq_decode_attn_noalloc — cq_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * cq_decode_attn with the same opts, minus the workspace: the schedules that
 * need one use a fixed scratch array of CQ_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends.  The
 * call allocates nothing (no hipMalloc, no hipFree); its first call on a
 * device resolves that device's scratch address (the current device must be
 * the stream's).  Calls that need more scratch than the array holds return
 * CQ_ERR_WORKSPACE before enqueuing anything (cq_decode_attn with a
 * workspace takes them).  Every call on a device shares its one array, and
 * the array keeps the last call's contents (no schedule reads scratch it has
 * not written in the same call): calls on one device whose executions
 * overlap (different streams, or different host threads) race and give
 * wrong results; calls in order on one stream are safe.
 * ------------------------------------------------------------------------ */
#define CQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

cq_status cq_decode_attn_noalloc(const void* q, cq_dtype q_dtype,
                                 const uint32_t* k_codes, const float* k_scale, const float* k_min,
                                 const uint32_t* v_codes, const float* v_scale, const float* v_min,
                                 const void* k_tail, const void* v_tail, cq_dtype tail_dtype,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t T,
                                 int32_t d, int32_t bits, float sm_scale,
                                 const cq_calib* calib,
                                 void* out, cq_dtype out_dtype,
                                 const cq_opts* opts, void* stream);

/* ------------------------------------------------------------------------
 * cq_visual_scores — the pre-softmax visual scores of cq_decode_attn on their
 * own, for inspection and diagnostics ([ART] Method part 2; before g):
 *   scores[b][hq][i] = sm_scale*(q*k_scale).c_i + sm_scale*q.k_min,
 * float32, from the packed K codes (any layout-K bit width).
 *
 *   q       device, [B][Hq][d] of q_dtype;  k_codes/k_scale/k_min as for decode
 *   scores  device, float32 [B][Hq][n]
 * Requires n >= 1, Hq % Hkv == 0, Hq/Hkv <= 8, d == 128 (else UNSUPPORTED).
 * ------------------------------------------------------------------------ */
cq_status cq_visual_scores(const void* q, cq_dtype q_dtype,
                           const uint32_t* k_codes, const float* k_scale, const float* k_min,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t d, int32_t bits,
                           float sm_scale, float* scores, void* stream);

/* ------------------------------------------------------------------------
 * cq_calibrate — the calibration map g on its own ([ART] Method part 3):
 * for every row r of scores[R][n], m = min, M = max, and
 * out[r][i] = g(scores[r][i]) as defined for cq_calib (computed in float64,
 * rounded to float32).  calib->enabled == 0 copies the scores.
 *
 *   scores      device, float32 [R][n]
 *   out         device, float32 [R][n]; may alias scores
 *   row_minmax  device, float32 [R][2] receiving (m, M), or NULL
 * Requires n >= 1.
 * ------------------------------------------------------------------------ */
cq_status cq_calibrate(const float* scores, int32_t R, int32_t n,
                       const cq_calib* calib, float* out, float* row_minmax,
                       void* stream);

/* ------------------------------------------------------------------------
 * cq_decode_attn_fp16 — comparison baseline, not part of the method:
 * unquantized softmax decode attention over N fp16 tokens
 * (out = softmax(sm_scale * q.K^T) V per query head, float32 accumulation).
 *
 *   q    device, fp16 [B][Hq][d];   k, v  device, fp16 [B][Hkv][N][d]
 *   out  device, fp16 [B][Hq][d];   workspace >= cq_decode_attn_fp16_workspace
 * Requires N >= 1, Hq % Hkv == 0, d == 128.
 * ------------------------------------------------------------------------ */
size_t cq_decode_attn_fp16_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d);

cq_status cq_decode_attn_fp16(const void* q, const void* k, const void* v,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                              float sm_scale, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* cq_scores_fp16 — the exact counterpart of cq_visual_scores, for the same
 * diagnostics: scores[b][hq][i] = sm_scale * q.k_i (float32 accumulation) over an
 * unquantized fp16 cache k [B][Hkv][N][d].  Requires N >= 1, Hq % Hkv == 0,
 * Hq/Hkv <= 8, d == 128. */
cq_status cq_scores_fp16(const void* q, const void* k, int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                         int32_t d, float sm_scale, float* scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CQ_H */
