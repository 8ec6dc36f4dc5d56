/*
 * fa.h — C ABI of libfa: exact tiled attention for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The textbook attention of the FlashAttention interview
 * canvas (panel 1, "standard attention" box) — scores S = Q K^T scaled by
 * softmax_scale, P = softmax(S) per query row, O = P V — evaluated tile by tile
 * with the online-softmax state (running max m, rescaled sum l, accumulator O;
 * panel 1 "online softmax key state" box and panel 3, Q2) so that the score
 * matrix never reaches device memory.  The tiled result equals the textbook one
 * up to floating-point rounding (panel 1, "one-sentence answer" box).  The
 * forward also returns the per-row statistic LSE_i = ln sum_j exp(s_ij) that a
 * recomputing backward needs (panel 3, Q3).
 *
 * Five entry points do work:
 *   fa_fwd         prefill (KV-cache quantisation overview, section 1, "prefill"):
 *                  every query row of a sequence against its keys, optional
 *                  causal mask, grouped-query heads, optional LSE output;
 *                  fp32, bf16, fp16 or fp8-e4m3 inputs.
 *   fa_decode_kvq  one decode step (same page, section 1, "decode step"): one new
 *                  query token per sequence against the whole cache, read from an
 *                  int8 or fp8-e4m3 cache with per-token-per-head scales and
 *                  dequantised inside the kernel (section 3, "read path"); the
 *                  cache is split into chunks processed in parallel and merged by
 *                  their log-sum-exps.  An optional residual window of recent
 *                  tokens kept in bf16 (section 3, "residual window") joins the
 *                  same softmax.
 *   fa_bwd         the backward of fa_fwd (interview canvas, panel 1 v1 card and
 *                  panel 3, Q3: the backward keeps no score matrix and recomputes
 *                  the local scores and probabilities from O and the per-row
 *                  LSE): dQ, dK, dV for bf16 / fp16.
 *   fa_fp8_quantize  fp8 inputs for fa_fwd with 64-row block scales and an
 *                  optional random-sign Hadamard rotation (FlashAttention-3 page,
 *                  the FP8 path's block quantisation and incoherent processing).
 *   fa_kv_append   the cache's write side (section 3, "before writing the cache"):
 *                  new bf16/fp16 key and value rows are quantised to int8 or
 *                  fp8-e4m3 codes with one fp16 scale per token and head, and
 *                  stored at each sequence's next cache positions.
 *
 * Conventions shared by every call.
 *   - All data pointers are DEVICE pointers (hipMalloc'd or equivalent).  The
 *     caller owns every buffer and the library allocates nothing.  Between
 *     calls it keeps only host-side bookkeeping: the per-thread message of
 *     fa_last_error(), a once-per-device flag for each kernel whose dynamic LDS
 *     limit it has raised, and fa_decode_kvq_noalloc's scratch address per
 *     device (both set up under a lock or once-flag), so calls from several
 *     host threads are safe and no call's result depends on an earlier one.
 *   - With the environment variable FA_LOG set to a value other than "0", every
 *     kernel launch prints one line to stderr before it is enqueued: the
 *     kernel, its grid, block and LDS bytes, and the sizes it was chosen for.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the legacy default
 *     stream) and return after enqueueing.  Nothing synchronises implicitly.
 *   - Parameters are validated on the host before anything is launched; on a
 *     validation error the call returns a negative fa_status and launches
 *     nothing.  A failed launch returns FA_ERR_HIP.  Faults inside a kernel are
 *     reported by the runtime at the caller's next synchronisation.
 *   - fa_last_error() gives a human-readable reason for the last failing call on
 *     the calling thread.
 *   - Tensors are described by element strides for the batch, head and sequence
 *     axes; the head-dimension stride is always 1.  Base pointers must be 16-byte
 *     aligned and the strides must keep every row 16-byte aligned
 *     (FA_ERR_ALIGNMENT otherwise).  Rows of one sequence must not overlap
 *     (sequence stride >= d), one (batch, head) slice must span less than
 *     2^31 bytes, and the sequence stride must be at most 8 MiB per row (the
 *     kernels form row offsets in 32 bits for every row of a tile);
 *     FA_ERR_UNSUPPORTED otherwise.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t passed as an opaque handle, so this header needs no HIP include. */
typedef void *fa_stream_t;

typedef enum {
  FA_F32 = 0,      /* IEEE binary32 */
  FA_F16 = 1,      /* IEEE binary16 */
  FA_BF16 = 2,     /* bfloat16 */
  FA_FP8_E4M3 = 3, /* OCP FP8 E4M3FN (bias 7, max 448, no inf) */
  FA_INT8 = 4      /* signed 8-bit integer codes */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
  FA_ERR_UNSUPPORTED = -2, /* valid but not implemented: head dim, dtype pair, size limit */
  FA_ERR_ALIGNMENT = -3,   /* pointer or stride breaks the 16-byte row alignment */
  FA_ERR_WORKSPACE = -4,   /* workspace missing or too small (decode, backward), or a
                              size beyond fa_decode_kvq_noalloc's fixed scratch */
  FA_ERR_HIP = -5          /* the HIP runtime rejected a launch */
} fa_status;

/*
 * Prefill forward.  Shapes (logical, any strides as described above):
 *   q [B, Hq,  Sq, d]   k, v [B, Hkv, Sk, d]   o [B, Hq, Sq, d]   lse [B, Hq, Sq]
 * Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention;
 * Hq % Hkv == 0).  d is 64 or 128.
 * Dtype pairs (in_dtype -> out_dtype): F32->F32, BF16->BF16, F16->F16,
 * FP8_E4M3->BF16.  For FP8 the true operands are code * descale (one float32
 * descale per tensor, or per 64-row block, see below); the descales are
 * ignored for the other dtypes.
 * causal != 0 masks key j for query i unless j <= i + Sk - Sq (the mask is
 * aligned to the last query and last key; with Sq == Sk it is the usual lower
 * triangle).  A query row that sees no key gets O = 0 and LSE = -inf.
 * lse may be NULL; otherwise it receives float32 natural-log LSE values.
 * softmax_scale multiplies Q K^T before the softmax (1/sqrt(d) for the usual
 * scaled dot-product attention); it must be finite and > 0.
 * FP8 needs d = 128.  For FP8 the probabilities P are rounded once before the
 * P V product (the row sum behind O's normaliser and the LSE uses them
 * unrounded), in the precision fp8_p_bf16 selects:
 *   0  e4m3, and P V runs on fp8 matrix cores (twice the bf16 rate).  Each
 *      probability then carries up to 2^-4 relative rounding, so a row whose
 *      softmax rests on a few keys can be off by up to about 2^-4 max|V|.
 *   1  bf16, with the V codes converted exactly to bf16, and P V runs on bf16
 *      matrix cores (2^-9 relative rounding per probability).
 * fp8_p_bf16 must be 0 for the other input dtypes.
 */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int32_t in_dtype, out_dtype; /* fa_dtype values */
  int32_t B, Hq, Hkv, Sq, Sk, d;
  int64_t q_strides[3]; /* batch, head, sequence — in elements */
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];
  int64_t lse_strides[2]; /* batch, head; the sequence stride is 1 */
  float softmax_scale;
  int32_t causal;
  float q_descale, k_descale, v_descale;
  /* FP8 only, optional: block descales, one float32 per 64 consecutive rows of
   * each (batch, head) slice, [B][H][ceil(S / 64)] contiguous (H = Hq for q,
   * Hkv for k and v), all three or none; when given they replace
   * q/k/v_descale (the FlashAttention-3 page's block quantisation for fp8).
   * They are read on the device, so the host-side checks cannot see them:
   * they must be finite and >= 0 (fa_fp8_quantize writes powers of two).
   * A V tile's descale enters as its ratio to the slice's largest, folded
   * into the probabilities before their rounding (see fp8_p_bf16); a ratio
   * below 2^-20 is taken as 2^-20, which moves the output by at most
   * 2^-19 max|V|.  With fp8_p_bf16 = 0, tiles whose ratio is below about
   * 2^-6 also lose relative precision in e4m3's subnormal range. */
  const float *q_block_descale, *k_block_descale, *v_block_descale;
  int32_t fp8_p_bf16; /* FP8 only: 0 = P in e4m3, 1 = P in bf16 (see above) */
  /* BF16/F16 with d = 128 only, 0 or 1: 1 computes a quarter of the
   * probabilities' exponentials with a polynomial on the FMA pipe instead of
   * the hardware exp2 (the FlashAttention interview canvas, v4 card: software
   * exponentials beside the exponential unit).  Relative error of those
   * exponentials 2^-18.5 (the hardware's is about 2^-22); both are far below
   * the bf16/fp16 rounding of P.  On gfx950 the transcendental instruction
   * shares the vector issue with the FMAs, so this is slower, not faster. */
  int32_t soft_exp2;
} fa_fwd_params;

int fa_fwd(const fa_fwd_params *p, fa_stream_t stream);

/*
 * Backward of fa_fwd by recomputation.  Given the forward's inputs, its output
 * o and natural-log lse (as fa_fwd writes them), and the gradient dout of a
 * loss with respect to o, writes
 *   dq [B, Hq, Sq, d], dk, dv [B, Hkv, Sk, d]
 * the gradients of o = softmax(softmax_scale * q k^T) v (same causal rule, same
 * grouped-query mapping; dk and dv of a key/value head sum the contributions of
 * all the query heads that read it).  The gradient reaches o only: lse is an
 * input, not differentiated.  A query row that sees no key contributes
 * nothing (its lse is -inf).
 * dtype is FA_BF16 or FA_F16 for every tensor but lse (float32); d must be 128.
 * The probabilities and dS are rounded to dtype as matrix-core operands and
 * accumulate in float32.  The caller's workspace (16-byte aligned, at least
 * fa_bwd_workspace_size(B, Hq, Sq) bytes, contents on entry irrelevant) holds
 * the per-row term rowsum(dout * o) in float32.  No atomics: results are
 * bitwise reproducible.  dq, dk, dv must not overlap any input.
 */
typedef struct {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  int32_t dtype; /* fa_dtype: FA_BF16 or FA_F16 */
  int32_t B, Hq, Hkv, Sq, Sk, d;
  int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3], do_strides[3];
  int64_t dq_strides[3], dk_strides[3], dv_strides[3];
  int64_t lse_strides[2];
  float softmax_scale;
  int32_t causal;
  void *workspace;
  size_t workspace_bytes;
  /* 0 or 1: the dK/dV kernel's wave-specialised schedule (FlashAttention-3
   * page, "Hopper asynchrony" section: one group of warps runs its softmax
   * while another runs its matrix products).  The two wavefronts of each SIMD
   * take two roles, the second running the same per-tile phases (S and dP
   * products, softmax gradient, dV and dK products) two phases behind the
   * first, three barriers per tile, so that in two of every three phases one
   * of them issues matrix work while the other does vector work.  Same
   * results, bit for bit; measured 3-10 % slower on this part (each phase
   * slot lasts as long as the longer of its two roles' phases, and the
   * extra barriers cost more than the overlap gains), kept for the
   * comparison.  Any other value is refused with FA_ERR_INVALID_ARG. */
  int32_t wave_pingpong;
} fa_bwd_params;

/* Bytes of workspace fa_bwd needs (0 on invalid sizes). */
size_t fa_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Sq);

int fa_bwd(const fa_bwd_params *p, fa_stream_t stream);

/*
 * fp8 inputs for fa_fwd: block-scaled E4M3FN codes, optionally of rotated rows
 * (FlashAttention-3 page, producer/consumer pseudocode box, "FP8 path": block
 * quantisation of Q/K/V and incoherent processing to keep fp8's error down).
 *   x [B, H, S, d] in_dtype (FA_BF16 or FA_F16), strides x_strides
 *   codes [B, H, S, d] E4M3FN bytes, strides codes_strides
 *   scales [B, H, ceil(S / 64)] float32, contiguous: one per 64-row block
 *   signs [d] float32 of +-1 on the device, or NULL for no rotation
 * Per block: y = x, or y = (x * signs) H / sqrt(d) with H the Sylvester-
 * Hadamard matrix (evaluated in float32 as the fast transform, stages 1, 2, 4,
 * ..., d/2, then one multiply by fp32(1/sqrt(d))); s = the smallest power of
 * two at or above fp32(absmax(y) / 448); code = E4M3FN(clamp(y / s, +-448))
 * rounded to nearest even, or 0 when s == 0.
 * The scales are the block descales fa_fwd takes.  Rotate Q and K with the
 * same signs (Q K^T is unchanged) and leave V unrotated.  d must be 128.
 */
typedef struct {
  const void *x;
  void *codes;
  float *scales;
  const float *signs;
  int32_t in_dtype; /* fa_dtype: FA_BF16 or FA_F16 */
  int32_t B, H, S, d;
  int64_t x_strides[3];     /* batch, head, row — in elements */
  int64_t codes_strides[3]; /* batch, head, row — in bytes */
} fa_fp8_quant_params;

int fa_fp8_quantize(const fa_fp8_quant_params *p, fa_stream_t stream);

/*
 * Cache formats.  Both store one code byte per element and one fp16 scale per
 * (batch, head, token); the value of an element is code * scale (symmetric, no
 * zero point).  The KV-cache quantisation overview lists FP8 and INT8 among the
 * storage forms (section 3, "storage form").
 *   FA_KV_INT8_TOKHEAD_F16SCALE      signed int8 codes in [-127, 127]
 *   FA_KV_FP8_E4M3_TOKHEAD_F16SCALE  OCP FP8 E4M3FN bytes (max 448); the NaN
 *                                    codes 0x7F / 0xFF must not occur
 */
typedef enum { FA_KV_INT8_TOKHEAD_F16SCALE = 0, FA_KV_FP8_E4M3_TOKHEAD_F16SCALE = 1 } fa_kv_format;

/*
 * One-token decode over a quantised cache.
 *   q [B, Hq, d] bf16                         o [B, Hq, d] bf16
 *   k_cache, v_cache [B, Hkv, L, d] codes     lse [B, Hq] float32 (may be NULL)
 *   k_scale, v_scale [B, Hkv, L] fp16 (token stride 1; 2-byte alignment is
 *                    enough; 16-byte aligned scale rows with L a multiple of 4 take the
 *                    faster loads)
 *   seq_lens [B] int32 on the device, or NULL meaning every sequence has L tokens
 * kv_format says how the codes are read (fa_kv_format).  Query head h reads
 * cache head h / (Hq / Hkv).  d must be 128 and Hq / Hkv at most 16.  Each
 * sequence's first seq_lens[b] tokens are attended (0 <= seq_lens[b] <= L; a
 * value outside that range is clamped into it).
 * Residual window (optional, W > 0): k_recent, v_recent [B, Hkv, W, d] bf16
 * (strides recent_strides, shared by both) hold recent tokens unquantised, and
 * recent_lens [B] int32 on the device (NULL = W; clamped into [0, W]) says how
 * many of them each sequence attends; they join the same softmax as the cache
 * tokens.  With W == 0 the window pointers are ignored.  A sequence that attends
 * no token at all gets O = 0 and LSE = -inf.
 * The L positions are cut into num_splits chunks of ceil(L / num_splits)
 * tokens rounded up to a multiple of 32 (1 <= num_splits <= 64; trailing chunks
 * may be empty); every chunk, and the window, yields a normalised partial
 * output and its log-sum-exp, and a second kernel merges them.  The partials
 * live in the caller's workspace, of at least
 * fa_decode_workspace_size(B, Hq, d, num_splits + (W > 0 ? 1 : 0)) bytes
 * (16-byte aligned); its contents on entry do not matter.
 */

typedef struct {
  const void *q;
  const void *k_cache, *v_cache;
  const void *k_scale, *v_scale;
  const int32_t *seq_lens;
  void *o;
  float *lse;
  int32_t B, Hq, Hkv, L, d, num_splits;
  int64_t q_strides[2];     /* batch, head — in elements */
  int64_t kv_strides[3];    /* batch, head, token — shared by k_cache and v_cache */
  int64_t scale_strides[2]; /* batch, head — shared by k_scale and v_scale */
  int64_t o_strides[2];     /* batch, head */
  int64_t lse_strides[2];   /* batch, head */
  int32_t kv_format;        /* fa_kv_format */
  float softmax_scale;
  void *workspace;
  size_t workspace_bytes;
  /* residual window; W == 0 disables it */
  const void *k_recent, *v_recent;
  const int32_t *recent_lens;
  int32_t W;
  int64_t recent_strides[3]; /* batch, head, token — shared by k_recent and v_recent */
} fa_decode_params;

/* Bytes of workspace fa_decode_kvq needs for these sizes (0 on invalid sizes);
 * num_splits counts the window as one more partial when it is used. */
size_t fa_decode_workspace_size(int32_t B, int32_t Hq, int32_t d, int32_t num_splits);

int fa_decode_kvq(const fa_decode_params *p, fa_stream_t stream);

/*
 * fa_decode_kvq for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the split partials kept in a
 * fixed array of FA_DECODE_NOALLOC_MAX_BYTES in the library's own device
 * memory (one per GPU, held until the process ends) instead of a workspace.
 * p->workspace and p->workspace_bytes are ignored.  Sizes whose partials
 * need more than FA_DECODE_NOALLOC_MAX_BYTES (fa_decode_workspace_size(B,
 * Hq, d, num_splits + (W > 0)) bytes) return FA_ERR_WORKSPACE before
 * anything runs.  The call uses the array of the current device, so call it
 * with the stream's device current.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * on it; calls ordered on one stream do not.  Nothing in the array needs to
 * be cleared: each call writes every partial it reads.  The array's address
 * is looked up on the first call on each device.  No memory is allocated.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES (32 * 1024 * 1024)
int fa_decode_kvq_noalloc(const fa_decode_params *p, fa_stream_t stream);

/*
 * Quantise-on-append: the write side of the cache (KV-cache quantisation
 * overview, section 3, "before writing the cache": K/V go from FP16/BF16 to a
 * low-bit form that needs a scale).
 *   k_new, v_new [B, H, T, d] in_dtype (FA_BF16 or FA_F16), strides new_strides
 *   k_cache, v_cache [B, H, L, d] code bytes, strides kv_strides (shared)
 *   k_scale, v_scale [B, H, L] fp16, strides scale_strides (token stride 1)
 *   positions [B] int32 on the device, or NULL meaning 0 for every sequence
 * Row t of sequence b is written to cache slot positions[b] + t; rows whose slot
 * falls outside [0, L) are skipped, and no other slot is touched.  d must be 128.
 * Per row (one token of one head), with QMAX = 127 for int8 and 448 for E4M3FN:
 *   sc   = fp16(min(fp32(absmax / QMAX), 65504)), round to nearest even
 *   code = 0 everywhere if sc == 0, else with y = fp32(x) / fp32(sc) (one
 *          correctly rounded fp32 division):
 *          int8:   clamp(rint(y), -127, 127), ties to even
 *          E4M3FN: the nearest E4M3FN value to clamp(y, -448, 448), ties to even
 * so that dequantising (code * sc) gives back x to within half a code step.
 * The inputs must be finite.  A call writes only the cache slots it addresses;
 * concurrent calls that address the same slot race.
 */
typedef struct {
  const void *k_new, *v_new;
  void *k_cache, *v_cache;
  void *k_scale, *v_scale;
  const int32_t *positions;
  int32_t in_dtype;             /* fa_dtype: FA_BF16 or FA_F16 */
  int32_t kv_format;            /* fa_kv_format */
  int32_t B, H, T, L, d;
  int64_t new_strides[3];       /* batch, head, token — shared by k_new and v_new */
  int64_t kv_strides[3];        /* batch, head, token — shared by k_cache and v_cache */
  int64_t scale_strides[2];     /* batch, head — shared by k_scale and v_scale */
} fa_kv_append_params;

int fa_kv_append(const fa_kv_append_params *p, fa_stream_t stream);

/* Host-only validation used by the calls above; makes no HIP call, so it
 * can run on a machine without a GPU.  Returns FA_OK or a negative fa_status. */
int fa_check_fwd_params(const fa_fwd_params *p);
int fa_check_decode_params(const fa_decode_params *p);
int fa_check_kv_append_params(const fa_kv_append_params *p);
int fa_check_bwd_params(const fa_bwd_params *p);
int fa_check_fp8_quant_params(const fa_fp8_quant_params *p);

/* Static description of a status code. */
const char *fa_status_string(int status);

/* Reason for the last non-FA_OK return on the calling thread ("" if none). */
const char *fa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_MI355X_FA_H */
