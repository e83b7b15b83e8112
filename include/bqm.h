/*
 * bqm.h - C ABI of the MI355X (gfx950) library for the routed-expert MoE layer
 * over frozen 4-bit block-quantized expert weights with a trainable bf16 LoRA.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the comment says "host".  The caller
 *     owns every buffer, including workspaces, and keeps it alive until the
 *     work queued on `stream` has finished.  The library allocates and frees
 *     nothing and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it: no host synchronisation, no
 *     device-to-host copy.
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense
 *     row-major (the last index is contiguous).
 *   - Arguments are checked on the host before anything is launched.  A failed
 *     check returns a negative bqm_status and sets a thread-local message
 *     (bqm_last_error); nothing is enqueued in that case.  A launch failure
 *     returns BQM_ERR_HIP with the HIP error string.  Non-finite input data are
 *     outside the contract and are not scanned for.
 *   - Device pointers must be 16-byte aligned.
 *
 * Page references are to the source pages: "Getting GLM-5.2 NVFP4 Post-Training
 * off the ground" (GLM page), "The 4-bitter Lesson: Balancing Stability and
 * Performance in NVFP4 RL" (4-bitter page) and "nf4moe - QLoRA for a 743B
 * Fused-MoE" (nf4moe page).
 */
#ifndef BQM_H
#define BQM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQM_ABI_VERSION 2

typedef enum {
  BQM_OK = 0,
  BQM_ERR_INVALID_ARG = -1, /* null pointer, bad enum, negative size */
  BQM_ERR_SHAPE = -2,       /* sizes that break a block or tile rule */
  BQM_ERR_ALIGN = -3,       /* a device pointer not 16-byte aligned */
  BQM_ERR_UNSUPPORTED = -4, /* a valid request the library does not implement */
  BQM_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  BQM_ERR_HIP = -6          /* a HIP launch or runtime error */
} bqm_status;

typedef enum { BQM_FMT_NVFP4 = 1, BQM_FMT_NF4 = 2 } bqm_format;
typedef enum { BQM_SCALE_PER_TENSOR = 0, BQM_SCALE_PER_ROW = 1 } bqm_scale_mode;

/* A rowwise-quantized stack [n_mat, rows, cols]; blocks run along cols (the
 * input dimension of a weight), the only copy ever stored (GLM page, section
 * "The 4-bit base that was actually using 8-bit memory": the columnwise copy is
 * dropped and the backward reads this one transposed).
 *   codes : uint8 [n_mat, rows, cols/2]; element 2j is the low nibble of byte j,
 *           element 2j+1 the high nibble.  NVFP4: E2M1 with the sign in bit 3.
 *           NF4: index 0..15 into the NormalFloat codebook.
 *   scales: NVFP4: uint8 E4M3FN bits [n_mat, rows, cols/16];
 *           NF4: float absmax [n_mat, rows, cols/64];
 *           NF4 nested: uint8 E4M3FN bits [n_mat, rows, cols/64] (see below).
 *   s_dec : NVFP4: float [n_mat] (per tensor) or [n_mat*rows] (per row);
 *           the value of an element is e2m1(code) * e4m3(scale) * s_dec.
 *           NF4: NULL.  NF4 nested: float [n_mat, 1 + G], G = ceil(rows*cols/64/256):
 *           per matrix the offset, then the scale of each group of 256 blocks.
 *   four_over_six: the mode the stack was quantized with (metadata).
 *   nested: NF4 only.  1: the absmax is double-quantized (the nested code of
 *           bnb's quant state that the nf4moe page names; read here as QLoRA's
 *           double quantization): block b of a matrix (row-major block order)
 *           has absmax' = fl(fl(e4m3(scales[b]) * s_dec[1 + b/256]) + s_dec[0]),
 *           and an element decodes to bf16(fl(level[code] * absmax')). */
typedef struct {
  int32_t fmt; /* bqm_format */
  int32_t scale_mode; /* bqm_scale_mode (NVFP4) */
  int64_t n_mat, rows, cols;
  uint8_t *codes;
  void *scales;
  float *s_dec;
  int32_t four_over_six;
  int32_t nested;
} bqm_qtensor;

/* ABI version of the loaded library (BQM_ABI_VERSION). */
int bqm_abi_version(void);

/* Message for the last non-OK status returned on this host thread ("" if none).
 * The string is owned by the library and valid until the next call on this thread. */
const char *bqm_last_error(void);

/* ---------------------------------------------------------------------------
 * NVFP4 quantization with the Four-Over-Six block-scale choice.
 * 4-bitter page, sections "Method" and "Four-Over-Six for RL Weights and
 * Activations"; GLM page, section "Why can't we just transpose the one copy?".
 *
 * x: bf16 [n_mat, rows, cols], cols % 16 == 0.  out->fmt must be BQM_FMT_NVFP4
 * and out->n_mat/rows/cols must equal the input sizes; out->codes, out->scales
 * and out->s_dec receive the result, out->scale_mode selects
 *   BQM_SCALE_PER_TENSOR: one FP32 scale per 2-D matrix (weights): A = max|x|
 *                         over the matrix, s_dec = A / (6*M);
 *   BQM_SCALE_PER_ROW:    one per row (per-token activation scales).
 * M = 256 with four_over_six != 0 (then each 16-block tries the scale t/6 and
 * t/4 and keeps the one with the lower FP32 squared error, ties keeping t/6),
 * M = 448 otherwise.  four_over_six = 1 measures that error in the scaled domain
 * (the target scaled down once by 1/s_dec, against q*sb: the page's fast path);
 * four_over_six = 2 uses the strict FP32 reference instead (each candidate scaled
 * back up, fl(fl(q*sb)*s_dec), against the original x); codes and candidate
 * scales are computed the same way, only the choice may differ (at near-ties).
 * out->four_over_six records the mode.  s_dec_in (nullable, same shape as out->s_dec) replaces
 * the amax-derived scale.  All rounding is round-to-nearest-even, E4M3 and E2M1
 * saturate.  Result codes and scales are deterministic bit patterns.
 * ws: per-tensor mode without s_dec_in needs bqm_quantize_nvfp4_workspace_size()
 * bytes of device scratch (the running amax of each matrix; the call clears it
 * on its stream, so calls sharing one ws must not overlap); per-row mode and
 * s_dec_in need none (ws may be NULL). */
size_t bqm_quantize_nvfp4_workspace_size(int64_t n_mat, int64_t rows, int64_t cols,
                                         int32_t scale_mode);
bqm_status bqm_quantize_nvfp4(const uint16_t *x, int32_t four_over_six, const float *s_dec_in,
                              bqm_qtensor *out /* host struct */, void *ws, size_t ws_bytes,
                              void *stream);

/* The same quantization for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): it takes no
 * workspace and allocates nothing.  Per-tensor mode without s_dec_in keeps the
 * running amax of each matrix in a static device array of the library (65536
 * matrices, 256 KiB per GPU, held until the process ends); a call with more
 * matrices returns BQM_ERR_WORKSPACE before anything is launched.  The array is
 * cleared by a kernel at the start of every call that uses it.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  The
 * stream must belong to the current device.  Results are bit-identical to
 * bqm_quantize_nvfp4's. */
bqm_status bqm_quantize_nvfp4_noalloc(const uint16_t *x, int32_t four_over_six, const float *s_dec_in,
                                      bqm_qtensor *out /* host struct */, void *stream);

/* NF4 quantization, blocksize 64 along cols, FP32 absmax per block: each
 * element is multiplied by the FP32 reciprocal of its block's absmax and takes
 * the nearest of the 16 NormalFloat levels, ties going to the lower level.
 * nf4moe page, section "The fix: dequant-on-forward for routed experts".
 * x: bf16 [n_mat, rows, cols], cols % 64 == 0; out->fmt == BQM_FMT_NF4. */
bqm_status bqm_quantize_nf4(const uint16_t *x, bqm_qtensor *out /* host struct */, void *stream);

/* Nested (double-quantized) absmax of an NF4 stack (the nested code of bnb's
 * quant state, nf4moe page, section "The fix: dequant-on-forward for routed
 * experts"; the page gives no
 * details, so this is QLoRA's published double quantization with E4M3 as the
 * 8-bit float).  Per matrix, over its absmax in row-major block order:
 *   offset = fl32(fl64(sum) / nb) (nb blocks; fl64(sum) is the exact sum of the
 *   matrix's absmax rounded once to the nearest double), d = fl(absmax - offset),
 *   per group of 256 blocks s2 = fl(max|d| / 448) and codes e4m3_rne_sat(fl(d / s2))
 *   (sign bit for d < 0; s2 = 0 gives codes 0).
 * plain: an NF4 stack with FP32 absmax (as bqm_quantize_nf4 writes; read only).
 * nested: the same shape, fmt BQM_FMT_NF4 and nested = 1; its scales (uint8
 * [n_mat, rows, cols/64]) and s_dec (float [n_mat, 1 + G]) are written, and its
 * codes get the plain codes (copied unless the two pointers are equal).  The
 * sum is exact (integer fixed point) before its one rounding, so the result does
 * not depend on the order of the additions; at most 2^31 blocks per matrix. */
bqm_status bqm_nf4_nest(const bqm_qtensor *plain, bqm_qtensor *nested, void *stream);

/* Dequantize a stack to bf16 [n_mat, rows, cols] (the DQ of DQ(Q(W)): GLM page,
 * section "The 4-bit base that was actually using 8-bit memory", where the one
 * rowwise copy is dequantized to bf16 for the backward; 4-bitter page, section
 * "Improving Gradient Stability", where the backward consumes DQ(Q(w));
 * nf4moe page, section "The fix: dequant-on-forward for routed experts", for NF4):
 *   NVFP4: bf16_rne(fl32(e2m1(code) * e4m3(scale)) * s_dec)  (one FP32 rounding)
 *   NF4:   bf16_rne(fl32(level[code] * absmax)), absmax' when nested
 * q: a stack as bqm_quantize_nvfp4 / bqm_quantize_nf4 / bqm_nf4_nest wrote it
 * (read only); y: bf16 [n_mat, rows, cols], written.  Errors: a bad format, a
 * NULL or unaligned pointer, or cols not a multiple of the block size.
 * The same values (without the s_dec factor, which the GEMMs apply to their
 * FP32 accumulators) are what the MoE GEMMs multiply. */
bqm_status bqm_dequantize(const bqm_qtensor *q /* host struct */, uint16_t *y, void *stream);

/* ---------------------------------------------------------------------------
 * Routing (nf4moe page, the expert module's forward receives top_k_index and
 * top_k_weights [T, k]).  Softmax over the E fp32 logits of each token, the k
 * largest logits chosen in descending order, equal logits going to the lower
 * expert index; weights are the chosen softmax probabilities (divided by their
 * sum if renorm != 0).  logits f32 [T, E] -> topk_idx i32 [T, k], topk_w f32
 * [T, k].  1 <= k <= E <= 1024, k <= 16.  T == 0 is a no-op. */
bqm_status bqm_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renorm,
                     int32_t *topk_idx, float *topk_w, void *stream);

/* Stable counting sort of the R = T*k routed pairs f = t*k + j by expert (the
 * order in which the nf4moe module visits them: expert, then token, then slot;
 * nf4moe page, section "The fix: dequant-on-forward for routed experts").
 * perm i32 [R]: perm[pos] = f.  inv i32 [R]: inv[f] = pos.  offsets i32 [E+1]:
 * exclusive prefix sum of per-expert counts.  Bit-exact, no atomics on the
 * result order.  A pair whose index lies outside [0, E) belongs to no expert:
 * it is placed after every expert's rows (offsets[E] <= pos < R, in f order), so
 * offsets[E] < R tells the caller that such pairs were dropped; the MoE calls
 * treat their expert output and gradient as zero (dtopk_w 0).
 * ws: bqm_permute_workspace_size() bytes. */
size_t bqm_permute_workspace_size(int64_t T, int32_t E, int32_t k);
bqm_status bqm_permute(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k, int32_t *perm,
                       int32_t *inv, int32_t *offsets, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The MoE layer.  Expert weights are stacks w_gu [E, 2I, H] (gate rows 0..I-1,
 * up rows I..2I-1, the chunk(2, -1) split of the nf4moe module) and w_dn
 * [E, H, I], both rowwise quantized (NVFP4 per-tensor, or NF4).  LoRA per
 * expert in bf16: A_gu [E, r, H], B_gu [E, 2I, r], A_dn [E, r, I], B_dn [E, H, r]
 * (all NULL when r == 0).  H % 64 == 0, I % 64 == 0, 1 <= k <= min(E, 16),
 * 0 <= r <= 128.  act_quant = 1 selects the W4A4 path: the base GEMMs multiply
 * per-token NVFP4 (Four-Over-Six) activations while LoRA reads bf16 ones
 * (4-bitter page, section "Method"); NVFP4 weights only.  The quantized rows are
 * expanded once into the workspace as bf16 val * sb (exact) and their per-row
 * s_dec multiplies the FP32 accumulator.
 */
/* Stages of the layer, for optional per-stage timing (stage_events below). */
typedef enum {
  BQM_STAGE_PERMUTE = 0,     /* counting sort of routed rows by expert */
  BQM_STAGE_ACT_QUANT_X,     /* W4A4: per-token NVFP4 of x */
  BQM_STAGE_LORA_A_GU,       /* U_gu = s x A_gu^T */
  BQM_STAGE_GATE_UP_FWD,     /* h, a = SwiGLU(x W_gu^T + U_gu B_gu^T) */
  BQM_STAGE_ACT_QUANT_A,     /* W4A4: per-token NVFP4 of a */
  BQM_STAGE_LORA_A_DN,       /* U_dn = s a A_dn^T */
  BQM_STAGE_DOWN_FWD,        /* y = a W_dn^T + U_dn B_dn^T */
  BQM_STAGE_COMBINE_FWD,     /* out = sum_j w y */
  BQM_STAGE_DTOPK,           /* d topk_w */
  BQM_STAGE_LORA_B_DN,       /* V_dn = s dy B_dn */
  BQM_STAGE_DOWN_DGRAD,      /* dh = SwiGLU'(w (dy W_dn + V_dn A_dn)) */
  BQM_STAGE_LORA_B_GU,       /* V_gu = s dh B_gu */
  BQM_STAGE_GATE_UP_DGRAD,   /* dX rows = dh W_gu + V_gu A_gu */
  BQM_STAGE_COMBINE_DGRAD,   /* dx = sum_j dX rows */
  BQM_STAGE_LORA_GRAD,       /* the four LoRA weight gradients */
  BQM_STAGE_COUNT
} bqm_stage;

typedef struct {
  int64_t T, H, I;
  int32_t E, k, r;
  int32_t act_quant;
  float lora_scale;
  /* 0: per-expert LoRA-A stacks A_gu [E, r, H], A_dn [E, r, I].  1: one LoRA-A
   * common to all experts, A_gu [r, H] and A_dn [r, I], with per-expert B (the
   * adapter layout of the GLM page, "Getting GLM-5.2 NVFP4 Post-Training off
   * the ground": its serving part, the paragraph on the non-fused NVFP4 MoE-LoRA
   * path, which names a shared LoRA-A and per-expert LoRA-B).  Other values:
   * BQM_ERR_INVALID_ARG. */
  int32_t lora_shared_a;
  bqm_qtensor w_gu;
  bqm_qtensor w_dn;
  /* bf16 LoRA matrices (NULL when r == 0): A_gu, B_gu [E, 2I, r], A_dn, B_dn
   * [E, H, r]; the A shapes follow lora_shared_a. */
  const uint16_t *A_gu, *B_gu, *A_dn, *B_dn;
  /* Optional (NULL: no timing).  Host array of 2*BQM_STAGE_COUNT hipEvent_t
   * handles created by the caller; every stage that runs records events
   * [2*stage] before and [2*stage+1] after its kernels on the call's stream. */
  void *const *stage_events;
} bqm_moe_desc;

/* Bytes of the workspace shared by bqm_moe_fwd, bqm_moe_dgrad and
 * bqm_lora_grad for this descriptor (host only).  The forward saves the
 * routing permutation, the gate/up activations h [R, 2I], a [R, I], the LoRA
 * intermediates and the expert outputs y [R, H] in it; the dgrad adds
 * dh [R, 2I] and its LoRA intermediates for bqm_lora_grad, which uses the rest
 * for partial sums (the row chunks of experts with more than 2048 rows). */
size_t bqm_moe_workspace_size(const bqm_moe_desc *d);

/* Forward: out[t] = sum_j topk_w[t,j] * y(t,j) with, for expert e = topk_idx[t,j],
 *   h = X~ DQ(W_gu[e])^T + s (X A_gu[e]^T) B_gu[e]^T,  a = silu(h[:, :I]) * h[:, I:],
 *   y = a~ DQ(W_dn[e])^T + s (a A_dn[e]^T) B_dn[e]^T
 * (nf4moe page, the QuantizedNaiveMoe forward; only experts that receive tokens
 * are read; A_gu[e], A_dn[e] stand for the one shared A with lora_shared_a; the
 * weights are NVFP4 or NF4, plain or nested).  x bf16 [T, H], topk_idx i32 [T, k], topk_w f32 [T, k], y bf16
 * [T, H] (the layer output).  Accumulation is FP32; the workspace keeps h in FP32 and
 * a (the down projection's bf16 operand) and the routed rows y in bf16, as the pages'
 * bf16 module does; the combine sums the k rows of a token in FP32. */
bqm_status bqm_moe_fwd(const bqm_moe_desc *d, const uint16_t *x, const int32_t *topk_idx,
                       const float *topk_w, uint16_t *out, void *ws, size_t ws_bytes,
                       void *stream);

/* Input gradient through DQ(Q(W)) (GLM page, section "The 4-bit base that was
 * actually using 8-bit memory": dX = dY W contracts the output dimension, read
 * from the single rowwise copy transposed, in bf16; 4-bitter page, section
 * "Improving Gradient Stability").  Must follow bqm_moe_fwd with the same
 * descriptor and workspace.  dy bf16 [T, H] -> dx bf16 [T, H] and, if
 * dtopk_w != NULL, f32 [T, k] with dtopk_w[t,j] = <dy[t], y(t,j)>.
 * Activation quantizers (W4A4) are the identity in this pass. */
bqm_status bqm_moe_dgrad(const bqm_moe_desc *d, const uint16_t *dy, void *ws, size_t ws_bytes,
                         uint16_t *dx, float *dtopk_w, void *stream);

/* The same input gradient over a second, columnwise quantization of the weights
 * (the two-copy scheme the GLM page's section "Why can't we just transpose the
 * one copy?" describes for FP4 tensor cores; a comparison variant here): w_gu_col
 * = Q(W_gu^T) [E, H, 2I] and w_dn_col = Q(W_dn^T) [E, I, H], NVFP4 with per-tensor
 * scales, each blocked along the dgrad's contraction axis and read K-major.  The
 * base GEMMs then use DQ(Q(W^T))^T, not the forward's DQ(Q(W)).  The copies must
 * carry the same per-tensor s_dec as d->w_gu and d->w_dn (quantizing W^T from its
 * own amax gives exactly that: transposition keeps the amax), because
 * bqm_lora_grad rescales by the rowwise s_dec.  Otherwise as bqm_moe_dgrad; the
 * copies are caller-owned and read only. */
bqm_status bqm_moe_dgrad_colwise(const bqm_moe_desc *d, const bqm_qtensor *w_gu_col,
                                 const bqm_qtensor *w_dn_col, const uint16_t *dy, void *ws,
                                 size_t ws_bytes, uint16_t *dx, float *dtopk_w, void *stream);

/* LoRA weight gradients (the adapter is the trained part; per-expert A/B on
 * the 3-D stacks, nf4moe page, section "Does it actually train?"), from the
 * state bqm_moe_fwd and bqm_moe_dgrad left in ws plus the two layer inputs the
 * library does not keep: x bf16 [T, H] (the forward input) and dy bf16 [T, H]
 * (the dgrad input).  With s = lora_scale and w the routing weight of a row:
 *   dB_gu = s dh^T (X A_gu^T)      dA_gu = s (dh B_gu)^T X
 *   dB_dn = s (w dy)^T (a A_dn^T)  dA_dn = s (w dy B_dn)^T a
 * summed over each expert's rows, FP32 accumulation.  f32 outputs dA_gu
 * [E, r, H], dB_gu [E, 2I, r], dA_dn [E, r, I], dB_dn [E, H, r]; experts
 * without rows get zeros.  An expert's rows are summed in chunks of 2048 whose
 * FP32 partial sums are added in chunk order.  With lora_shared_a, dA_gu [r, H]
 * and dA_dn [r, I] are sums over all routed rows of every expert (the gradient
 * of the one shared matrix), added in a fixed order; either way repeated calls
 * give identical bits.  Requires r > 0. */
bqm_status bqm_lora_grad(const bqm_moe_desc *d, const uint16_t *x, const uint16_t *dy, void *ws,
                         size_t ws_bytes, float *dA_gu, float *dB_gu, float *dA_dn, float *dB_dn,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BQM_H */
