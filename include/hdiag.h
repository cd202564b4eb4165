/*
 * hdiag.h - C ABI of the MI355X (gfx950) block-scale quantiser library
 * (libhdiag.so).
 *
 * For every contiguous block of B weights along K in each row of W [N, K] the
 * library picks one scale from a quantised grid and encodes the block to an
 * element format, as the qwantize "Results" page describes it (sections
 * "INT8 (FP8 E4M3 scales)", "NVFP4 (FP8 E4M3 scales)" and "MXFP4 (UE8M0
 * power-of-2 scales)"), following the generic microscaling quantiser of
 * "Is Finer Better? The Limits of Microscaling Formats in LLMs", §2.1:
 * s = Q_scale(x_max / C), q_i = Q_elem(x_i / s), x^_i = s q_i.
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller, 16-byte
 *     aligned, row-major and densely packed.  The library allocates nothing;
 *     calls that need scratch memory take a caller-owned workspace whose size
 *     the matching *_workspace_size() function returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     calls only enqueue work on that stream and return; results (including the
 *     double scalars written by the error metrics) are valid once the stream has
 *     been synchronised.  Calls on different streams may run concurrently as
 *     long as they do not share output or workspace memory.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns an error and touches no memory.  Nothing is printed
 *     and no exception crosses the ABI.  hdiag_last_error() returns a
 *     thread-local description of the last failure on the calling thread.
 *   - Inputs must be finite; NaN / Inf inputs give unspecified (but
 *     memory-safe) codes.
 *   - Sizes of 0 (N, K or M) are valid and enqueue nothing, except where a
 *     metric would divide by zero (see the metric functions).
 */
#ifndef HDIAG_H
#define HDIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HD_OK = 0,
    HD_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment, enum or block size */
    HD_ERR_UNSUPPORTED = -2, /* a valid but unimplemented combination */
    HD_ERR_HIP = -3          /* the HIP runtime reported an error (see hdiag_last_error) */
} hd_status;

typedef enum { HD_F32 = 0, HD_BF16 = 1 } hd_dtype;

/* Scale choice (qwantize "Results", all three format tables):
 *   HD_NAIVE     - amax of the block snapped onto the scale grid;
 *   HD_SSE_OPT   - the candidate minimising sum_j (w_j - s Q(w_j / s))^2;
 *   HD_H_OPT     - the candidate minimising sum_j h_j (w_j - s Q(w_j / s))^2,
 *                  the diagonal-Hessian form of the output error (quantisation
 *                  algorithms note, §1);
 *   HD_NAIVE_OCP - power-of-two grids only (HD_MXFP4, HD_MXFP8): the OCP MX
 *                  rule s = 2^(floor(log2 amax) - emax), emax the exponent of
 *                  the largest element (2 for E2M1, 8 for E4M3), clamped to
 *                  E8M0's range; amax = 0 gives code 0 ("Is Finer Better?"
 *                  §2.1 cites the OCP specification that defines it).
 * The search methods evaluate every candidate of the grid and return the first
 * (lowest) scale code among equal minima.  On the FP16 scale grids
 * (HD_FP4_F16, HD_INT4_F16) they alternate instead (see hd_format). */
typedef enum { HD_NAIVE = 0, HD_SSE_OPT = 1, HD_H_OPT = 2, HD_NAIVE_OCP = 3 } hd_method;

/* Element format x scale grid.
 *   HD_INT8_E4M3 - symmetric INT8 elements in [-127, 127]; the block's amax is
 *                  stored as an E4M3 code and the effective scale is
 *                  fl32(val(code) / 127) (qwantize "Results", INT8 section).
 *   HD_NVFP4     - E2M1 elements {0,.5,1,1.5,2,3,4,6}, E4M3 scale ("Is Finer
 *                  Better?" §2.1, NVFP4 with a UE4M3 scale; any B here).
 *   HD_MXFP4     - E2M1 elements, E8M0 power-of-two scale (OCP MX, §2.1).
 *   HD_MXFP8     - E4M3 elements, E8M0 scale.
 *   HD_FP8_E4M3S - E4M3 elements, E4M3 scale.
 *   HD_NVFP4_UE4M4 - E2M1 elements, unsigned UE4M4 scale (4 exponent bits,
 *                  bias 7, 4 mantissa bits, every code finite: 0x01..0xFF,
 *                  2^-10 .. 496) (qwantize "Results", Exotic Scales).
 *   HD_NVFP4_UE5M3 - E2M1 elements, unsigned UE5M3 scale (bias 15, 3 mantissa
 *                  bits: 2^-17 .. 122880) (same section; "Is Finer Better?"
 *                  §5.2).
 *   HD_NVINT4    - symmetric INT4 elements [-7, 7] (two's complement nibbles,
 *                  element 2i in the low nibble), E4M3 scale
 *                  s = Q_E4M3(amax / 7) (the NVINT4 rows of the qwantize
 *                  "Results" GPTQ tables, read with the generic rule of "Is
 *                  Finer Better?" §2.1).
 *   HD_FP4_F16   - E2M1 elements with a binary16 (FP16 E5M10) block scale, and
 *   HD_INT4_F16  - INT4 elements [-7, 7] with a binary16 block scale
 *                  (qwantize "Results", "Larger blocks: bs=64 (E4M3 scales) and
 *                  bs=128 (FP16 scales)").  Scales are stored as 2-byte
 *                  binary16 bit patterns; only 0x0000 .. 0x7BFF (0 .. 65504)
 *                  are produced or accepted.  Naive: s = fp16(fl32(amax / C)),
 *                  round to nearest even, saturating at 65504.  SSE / H-Optimal
 *                  alternate, from the Naive scale, between encoding the block
 *                  at the current scale and the least-squares scale of that
 *                  assignment, s* = sum w q / sum q^2 (weighted by h for
 *                  H-Optimal, in float64) snapped to FP16; they stop at a
 *                  fixed point, at an all-zero assignment or the zero scale,
 *                  or after 32 rounds, and keep the scale with the smallest
 *                  objective among those visited (the earliest on ties).
 * Search candidates: the 126 positive finite E4M3 codes 0x01..0x7E (E4M3 and
 * INT8 grids; max 448), all 255 finite E8M0 codes 0x00..0xFE (2^-127 ..
 * 2^127), or the 255 positive UE4M4 / UE5M3 codes.  Naive may also return E4M3 code 0 (the zero scale: every element
 * encodes to 0), when amax / C rounds into the zero bin ("Is Finer Better?",
 * App. F.3). */
typedef enum {
    HD_INT8_E4M3 = 0,
    HD_NVFP4 = 1,
    HD_MXFP4 = 2,
    HD_MXFP8 = 3,
    HD_FP8_E4M3S = 4,
    HD_NVFP4_UE4M4 = 5,
    HD_NVFP4_UE5M3 = 6,
    HD_NVINT4 = 7,
    HD_FP4_F16 = 8,
    HD_INT4_F16 = 9
} hd_format;

/* ------------------------------------------------------------- schedule --- */

/* Process-wide schedule settings of kernels whose work split does not change
 * what they compute, only the order of floating-point partial sums or the
 * tile shape of an intermediate product.  Value 0 (the initial state) is the
 * automatic choice.  Meant for tests and tuning; a setting applies to calls
 * made after it on any thread.
 *   HD_SCHED_GRAM_GANGS - output_error_gram(_batch): g > 0 runs the C E^T walk
 *                         as g gangs of one workgroup per 256-row tile of E
 *                         instead of its per-XCD schedule (the order of the
 *                         float64 partial sums changes);
 *   HD_SCHED_GPTQ_TILE  - gptq_*: 64 or 128 forces the tile width of the
 *                         factorisation's matrix-core products;
 *   HD_SCHED_GRAM_BANDS - output_error_gram(_batch): a > 0 runs the per-XCD
 *                         walk with a bands of C per panel and
 *                         max(1, CUs / 8 / a) tiles of E per group (ignored
 *                         while HD_SCHED_GRAM_GANGS is set; the order of the
 *                         float64 partial sums changes).
 * Errors: HD_ERR_INVALID_ARG for an unknown setting or value. */
typedef enum {
    HD_SCHED_GRAM_GANGS = 0,
    HD_SCHED_GPTQ_TILE = 1,
    HD_SCHED_GRAM_BANDS = 2,
    HD_SCHED_COUNT = 3
} hd_schedule;
hd_status hdiag_set_schedule(hd_schedule knob, int32_t value);

/* ---------------------------------------------------------------- hdiag --- */

/* Bytes of workspace hdiag() needs for X [M, K]. */
size_t hdiag_workspace_size(int64_t M, int64_t K);

/* h[j] = sum_{t<M} X[t][j]^2: the diagonal of X^T X, i.e. the per-input-channel
 * weight of the H-Optimal objective (quantisation algorithms note, §1, which
 * writes it as the mean E[x_j^2]; the sum differs by the factor M, which does
 * not move the argmin).  X: [M, K] of dtype xt.  h: [K] float32 output.
 * Summed in float64 (squares are exact), rounded once to float32.
 * workspace: ws_bytes >= hdiag_workspace_size(M, K).
 * Errors: HD_ERR_INVALID_ARG for NULL X / h (when M*K > 0), M or K < 0, a bad
 * dtype, a misaligned pointer or a short workspace. */
hd_status hdiag(const void *X, hd_dtype xt, int64_t M, int64_t K, float *h, void *ws,
                size_t ws_bytes, void *stream);

/* Bytes of the static device scratch behind hdiag_noalloc(). */
#define HD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* hdiag() for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as hdiag() (bit for bit), but the float64
 * row-chunk partials go to a static __device__ scratch array of
 * HD_NOALLOC_SCRATCH_BYTES held by every GPU the library runs on until the
 * process ends, so no workspace is passed and nothing is allocated
 * (no hipMalloc / hipFree, no allocating library call).  The device is the
 * stream's (the current device for the null stream); the first call on a
 * device looks up that device's scratch address once.
 * Limit: hdiag_workspace_size(M, K) <= HD_NOALLOC_SCRATCH_BYTES (every M for
 * K up to about 10^6 columns); larger shapes return HD_ERR_UNSUPPORTED and
 * launch nothing.
 * Concurrency: every call on one GPU shares that GPU's scratch.  Calls that
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and give undefined h; calls on one stream are ordered and
 * safe.  No part of the scratch must start at zero: each call writes every
 * partial it reads.
 * Errors: those of hdiag(), plus HD_ERR_UNSUPPORTED for a shape beyond the
 * limit and HD_ERR_HIP if the scratch address cannot be looked up. */
hd_status hdiag_noalloc(const void *X, hd_dtype xt, int64_t M, int64_t K, float *h, void *stream);

/* ------------------------------------------------------ quantize_blocks --- */

/* Choose the scale of every block and encode W with it.
 *   W      : [N, K] of dtype wt (float32 or bfloat16).
 *   B      : block size along K, one of 8, 16, 32, 64, 128, 256; K % B == 0.
 *            B = 4 (the smallest block of "Is Finer Better?" App. F) is
 *            accepted by the Naive methods, encode_blocks, dequantize and the
 *            per-tensor-scaled pair, with K % 8 == 0; every other call
 *            returns HD_ERR_UNSUPPORTED for it.
 *   h      : [K] float32, required for HD_H_OPT.  For HD_NAIVE it only weights
 *            the reported block objective (NULL: unweighted); ignored by
 *            HD_SSE_OPT.
 *   codes  : element codes.  HD_INT8_E4M3: [N, K] int8 two's complement.
 *            HD_MXFP8 / HD_FP8_E4M3S: [N, K] E4M3 bytes (sign bit 7).
 *            HD_NVFP4 / HD_MXFP4 / HD_NVFP4_UE4M4 / HD_NVFP4_UE5M3 /
 *            HD_FP4_F16: [N, K/2] bytes of two E2M1 nibbles (sign bit 3),
 *            element 2i in the low nibble.  HD_NVINT4 / HD_INT4_F16: [N, K/2]
 *            bytes of two INT4 two's complement nibbles, same order.  A negative input that rounds to
 *            zero keeps its sign bit (E2M1 0x8, E4M3 0x80).
 *   scales : [N, K/B] scale codes: one byte each (E4M3, E8M0, UE4M4, UE5M3),
 *            or two (little-endian binary16 bits, 2-byte aligned) for
 *            HD_FP4_F16 / HD_INT4_F16.
 *   block_obj: optional [N, K/B] float32: the block's objective at the chosen
 *            scale (weighted by h when h is used), computed in float64 and
 *            rounded; may be NULL.
 * Encoding: q = RNE_T(fl32(|w| / s)) onto the element table T with ties to the
 * even code and saturation at the largest element; dequantised value
 * fl32(s * val(q)).  Division is IEEE round-to-nearest (qwantize "Results",
 * Correctness notes, on why a reciprocal-multiply moves boundary ties).
 * Errors: HD_ERR_INVALID_ARG for NULL W / codes / scales (when N*K > 0), bad
 * enums, an unsupported B, K % B != 0, N or K < 0, H_OPT without h,
 * HD_NAIVE_OCP on a grid that is not E8M0, misaligned pointers. */
hd_status quantize_blocks(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt,
                          int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                          float *block_obj, void *stream);

/* quantize_blocks() with instrumentation, for measurement and tests: when
 * `evaluated` (device uint64, 8-byte aligned, may be NULL) is given, the
 * SSE / H-Optimal searches of the 8-bit scale grids add to it the number of
 * (weight, candidate) pairs they evaluated (every candidate a block's lanes
 * walk, repeats at the grid ends included; the zero tail the search proves
 * tied is not walked).  The caller clears it; Naive and the FP16-scale
 * alternation add nothing.  Results are those of quantize_blocks(). */
hd_status quantize_blocks_instrumented(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt,
                                       int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                                       float *block_obj, uint64_t *evaluated, void *stream);

/* Encode W with caller-given scale codes (the encode step alone).  Arguments
 * as quantize_blocks; scales_in [N, K/B] is read, not written.  A NaN scale
 * code (E4M3 0x7F..., E8M0 0xFF, binary16 above 0x7BFF) encodes its block
 * with the zero scale. */
hd_status encode_blocks(hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N, int64_t K,
                        const uint8_t *scales_in, const float *h, uint8_t *codes, float *block_obj,
                        void *stream);

/* ----------------------------------------------------------- dequantize --- */

/* Wq[n][k] = sign * fl32(s_block * val(q)) ("Is Finer Better?" §2.1,
 * x^ = s q), written as float32 or as bfloat16 (round-to-nearest-even of the
 * float32 value).  codes / scales laid out as quantize_blocks writes them.
 * Invalid codes (INT8 -128, E4M3 0x7F / 0xFF, E8M0 0xFF, INT4 -8, binary16
 * scales above 0x7BFF) decode to 0. */
hd_status dequantize(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales,
                     int64_t N, int64_t K, void *Wq, hd_dtype out_t, void *stream);

/* --------------------------------------------------------------- errors --- */

/* Weight error ||Wq - W||_F / ||W||_F (qwantize "Results", metric
 * definitions), in float64, written to the device scalar *out.
 * sums (optional, device, 2 doubles): {sum (Wq-W)^2, sum W^2}.
 * If ||W||_F = 0 the result is the IEEE quotient (NaN or Inf). */
size_t weight_error_workspace_size(int64_t N, int64_t K);
hd_status weight_error(const void *W, hd_dtype wt, const void *Wq, hd_dtype qt, int64_t N, int64_t K,
                       double *out, double *sums, void *ws, size_t ws_bytes, void *stream);

/* dequantize() and weight_error() in one pass ("Is Finer Better?" §2.1 for
 * the dequantised values; qwantize "Results", metric definitions, for the
 * ratio): Wq is written exactly as dequantize(fmt, B, codes, scales, N, K,
 * Wq, out_t) writes it, and *out / sums are exactly what weight_error(W, wt,
 * Wq, out_t, N, K, ...) gives for that Wq (the same partial sums in the same
 * order), while the codes and W are read once and Wq is not read back.
 * B as for dequantize (4 included); K % 8 == 0; W [N, K] float32 or
 * bfloat16; workspace: ws_bytes >= weight_error_workspace_size(N, K).
 * N * K = 0 writes nothing to Wq and gives the IEEE quotient 0 / 0. */
hd_status dequantize_weight_error(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales,
                                  int64_t N, int64_t K, void *Wq, hd_dtype out_t, const void *W, hd_dtype wt,
                                  double *out, double *sums, void *ws, size_t ws_bytes, void *stream);

/* Output error ||X Wq^T - X W^T||_F / ||X W^T||_F (qwantize "Results", metric
 * definitions), written to the device scalar *out (float64).
 * sums (optional, device, 2 doubles): {||X (Wq-W)^T||^2, ||X W^T||^2}.
 * With X and W in bfloat16 and K % 32 == 0 the products run on the bf16 MFMA
 * units with float32 accumulation: Y = X W^T and D = X dW^T with
 * dW = fl32(Wq - W) split into two bfloat16 terms hi + lo (the difference, not
 * Wq, is rounded, so INT8 codes that bf16 cannot hold do not move the metric);
 * the squares of each output tile are summed in float64.  Other inputs use a
 * float32 vector path.
 * workspace: ws_bytes >= output_error_workspace_size(M, N, K). */
size_t output_error_workspace_size(int64_t M, int64_t N, int64_t K);
hd_status output_error(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt,
                       const void *Wq, hd_dtype qt, int64_t N, int64_t K, double *out, double *sums,
                       void *ws, size_t ws_bytes, void *stream);

/* output_error with ||X W^T||_F^2 already known: ysq is a device double
 * holding it (e.g. sums[1] of an earlier output_error on the same X and W).
 * Only D = X dW^T is computed (two of the three bf16 products); the result is
 * sqrt(sum D^2) / sqrt(*ysq), and sums (optional) receives {sum D^2, *ysq}.
 * Arguments, workspace and errors as output_error, plus HD_ERR_INVALID_ARG for
 * a NULL ysq.  For callers that score several quantisations of one W against
 * the same X. */
hd_status output_error_given_ref(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt,
                                 const void *Wq, hd_dtype qt, int64_t N, int64_t K, const double *ysq,
                                 double *out, double *sums, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------- output error against a reference --- */

/* For callers that score several quantisations of one W against one X: the
 * output error of each quantisation then costs one MFMA product instead of two.
 *
 * output_reference() fills a caller-allocated device buffer `ref` of at least
 * output_reference_size(M, N, K) bytes (16-byte aligned) with:
 *   byte 0                : double ||X W^T||_F^2;
 *   byte HD_REF_Y_OFFSET  : float Y[M][N] = X W^T (row-major), products of the
 *                           bf16 inputs accumulated in float32 on the MFMA units;
 *   after Y               : data private to the library (a float16 copy of X
 *                           with one power-of-two scale per row, used for INT8).
 * X and W must be bfloat16 (HD_ERR_UNSUPPORTED otherwise: use output_error);
 * K % 8 == 0.  The buffer stays valid as long as X and W are unchanged.
 *
 * output_error_codes() returns ||X Wq^T - X W^T||_F / ||X W^T||_F for
 * Wq = dequantize(fmt, B, codes, scales) without forming Wq:
 *   - E2M1 / E4M3 elements: the dequantised values s val(q) are exact in
 *     bfloat16, so X Wq^T is one bf16 MFMA product (float32 accumulation);
 *   - INT8: val(a8) q (E4M3 scale value times the integer code) is exact in
 *     float16 and is multiplied with the float16 copy of X; the factor
 *     2^e_row / 127 is applied in float64 afterwards.  This uses val q / 127
 *     for fl32(fl32(val / 127) q), a difference of at most two float32
 *     roundings (2^-23 relative) per weight;
 *   - D = X Wq^T - Y is formed and squared in float64, so D is carried to
 *     float32 accumulation accuracy relative to Y (about 1e-6 of ||Y|| per
 *     element): the metric is accurate to ~1e-4 relative while it is above
 *     ~1e-3.  output_error() computes D directly and has no such floor.
 * X is the same bfloat16 [M, K] given to output_reference, ref its buffer.
 * sums (optional, device, 2 doubles): {||D||^2, ||X W^T||^2}.
 * workspace: ws_bytes >= output_error_codes_workspace_size(M, N, K).
 * Errors: HD_ERR_INVALID_ARG as quantize_blocks for fmt / B / N / K, NULL or
 * misaligned pointers, a short ref or workspace; HD_ERR_UNSUPPORTED for a
 * float32 X and for the FP16-scale formats (s val(q) needs up to 14
 * significant bits there: use dequantize + output_error).  Calls that share `ref` may run concurrently (it is only read);
 * each needs its own workspace. */
#define HD_REF_Y_OFFSET 256
size_t output_reference_size(int64_t M, int64_t N, int64_t K);
hd_status output_reference(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt, int64_t N,
                           int64_t K, void *ref, size_t ref_bytes, void *stream);
size_t output_error_codes_workspace_size(int64_t M, int64_t N, int64_t K);
hd_status output_error_codes(hd_format fmt, int32_t B, const void *X, hd_dtype xt, int64_t M,
                             const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                             const void *ref, size_t ref_bytes, double *out, double *sums, void *ws,
                             size_t ws_bytes, void *stream);

/* ----------------------------------------- output error through X^T X --- */

/* The output error of qwantize "Results" (metric definitions), computed from
 * the Gram matrix G = X^T X: ||X D^T||_F^2 = sum_n d_n^T G d_n for the rows
 * d_n of D = Wq - W (and of W itself for ||X W^T||_F^2), an identity of the
 * definition.  G depends on X alone, so once it is formed each quantisation
 * costs about N K^2 multiply-adds (the symmetry of G halves N K K) instead of
 * the 2 M N K of two products with X: the cheaper order whenever several
 * quantisations of weights of width K are scored against more than about K/2
 * rows of X.
 *
 * output_gram() fills a caller-allocated device buffer `gram` of at least
 * output_gram_size(K) bytes (16-byte aligned) with data private to the
 * library: h = diag(G), and C = G / sqrt(h_j h_k) off the diagonal (0 where h
 * is 0), as float16, one triangle only.  X: bfloat16 [M, K], K % 8 == 0;
 * the products run on the bf16 MFMA units with float32 accumulation.
 * h (optional, device, float [K]): hdiag(X) already computed on the same X;
 * NULL computes it here.  The buffer stays valid as long as X is unchanged.
 * workspace: ws_bytes >= output_gram_workspace_size(M, K) (hdiag's partial
 * sums when h is NULL; X itself is read in place).
 *
 * output_reference_gram() writes ||X W^T||_F^2 (double) to the device scalar
 * *ysq; output_error_gram() writes ||X Wq^T - X W^T||_F / sqrt(*ysq) to *out,
 * for Wq = dequantize(fmt, B, codes, scales) (every format, FP16 scales
 * included) without forming Wq, and sums (optional, device, 3 doubles) gets
 * {t = ||X (Wq - W)^T||_F^2, *ysq, b = sum_n sum_j d_nj^2 h_j}.  W: bfloat16
 * or float32 [N, K], the weights the codes quantise.
 * Accuracy: with e_n = d_n sqrt(h), d^T G d = sum_j d_j^2 h_j + e^T C e; the
 * diagonal sum b is taken in float64 from float32 d and h, the off-diagonal
 * part t - b is the float16 MFMA product of e (one power-of-two scale per
 * row, rounded to 11 significant bits) with the float16 C (|C| <= 1), in
 * float32 accumulation.  Those roundings are relative to the off-diagonal
 * terms, whose size is set by b, not by t, so the metric's relative error
 * grows with b / t: on Gaussian X with outlier channels (b / t about 1) it
 * is about 1e-6; where the error cancels across correlated channels (as
 * GPTQ's compensation makes it do) it reaches about 4e-5 (b / t) in the
 * worst constructions tested (channel pairs of correlation 0.5 ... 0.999
 * with errors of opposite sign, K = 16 ... 1024), so it meets a 1e-4 bar for
 * b / t <= 2.  sums[2] / sums[0] reports b / t; above 2, use
 * output_error_codes() or output_error(), which form X Wq^T itself.
 * workspace: ws_bytes >= output_error_gram_workspace_size(N, K); each call
 * needs its own.  Calls that share `gram` may run concurrently (it is only
 * read).
 * Schedule: HD_SCHED_GRAM_GANGS and HD_SCHED_GRAM_BANDS (hdiag_set_schedule)
 * change only the order of the float64 partial sums.
 * Errors: HD_ERR_INVALID_ARG as quantize_blocks for fmt / B / N / K, NULL or
 * misaligned pointers, a short buffer or workspace, K % 8 != 0 for
 * output_gram; HD_ERR_UNSUPPORTED for a float32 X. */
size_t output_gram_size(int64_t K);
size_t output_gram_workspace_size(int64_t M, int64_t K);
hd_status output_gram(const void *X, hd_dtype xt, int64_t M, int64_t K, const float *h, void *gram,
                      size_t gram_bytes, void *ws, size_t ws_bytes, void *stream);
size_t output_error_gram_workspace_size(int64_t N, int64_t K);
hd_status output_reference_gram(const void *W, hd_dtype wt, int64_t N, int64_t K, const void *gram,
                                size_t gram_bytes, double *ysq, void *ws, size_t ws_bytes, void *stream);
hd_status output_error_gram(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales, const void *W,
                            hd_dtype wt, int64_t N, int64_t K, const void *gram, size_t gram_bytes,
                            const double *ysq, double *out, double *sums, void *ws, size_t ws_bytes, void *stream);

/* output_error_gram for count quantisations of the same W [N, K] in one call:
 * fmts[q], Bs[q], codes[q], scales[q] (q < count) are HOST arrays holding,
 * for each quantisation, its format, block size and the device pointers of
 * its codes and scales (each as for output_error_gram).  out: device
 * double[count], out[q] = ||X Wq_q^T - X W^T||_F / sqrt(*ysq); sums (optional,
 * device, 3 count doubles): {t_q, *ysq, b_q} for each q, as output_error_gram's.
 * The results are those of count output_error_gram calls up to the order of
 * the float64 partial sums; one MFMA walk over the stacked operand of several
 * quantisations reads each C block for all of them at once, and a batch is
 * cut into walks of as many quantisations as fit the Infinity Cache together
 * with C (two for K = 9728; the whole batch when C alone does not fit).
 * workspace: ws_bytes >= output_error_gram_batch_workspace_size(count, N, K)
 * (count x the single call's operand).  1 <= count <= 4096.  Errors as
 * output_error_gram, for each q. */
size_t output_error_gram_batch_workspace_size(int32_t count, int64_t N, int64_t K);
hd_status output_error_gram_batch(int32_t count, const hd_format *fmts, const int32_t *Bs,
                                  const uint8_t *const *codes, const uint8_t *const *scales, const void *W,
                                  hd_dtype wt, int64_t N, int64_t K, const void *gram, size_t gram_bytes,
                                  const double *ysq, double *out, double *sums, void *ws, size_t ws_bytes,
                                  void *stream);

/* ------------------------------------------------ per-tensor scaling --- */

/* Two-level scales for the E4M3 block-scale formats (HD_INT8_E4M3, HD_NVFP4,
 * HD_FP8_E4M3S, HD_NVINT4): "Is Finer Better?" §5.1 and Table 1 (UE4M3-S,
 * per-tensor scaling on top of UE4M3 block scales; the page's formula for the
 * tensor scale is not legible, the reading here is the one documented):
 *   s_T = fl32(amax_T / (C * 448)), C the element maximum (6 E2M1, 7 INT4,
 *   448 E4M3; 1 for INT8, whose block scale is amax itself), 1 for an all-zero
 *   tensor - the largest block scale lands on the top of the E4M3 grid;
 *   the blocks quantise W' = fl32(W / s_T) exactly as quantize_blocks does
 *   (codes, scales and block_obj refer to W');
 *   dequantize_tensor_scaled gives x^ = fl32(s_T * fl32(s * val(q))).
 * tensor_scale: one device float (written by quantize, read by dequantize).
 * Workspace: quantize_blocks_tensor_scaled_workspace_size(N, K) bytes (W' is
 * staged there in float32).  Errors as quantize_blocks / dequantize, plus
 * HD_ERR_INVALID_ARG for a format without E4M3 block scales and for
 * HD_NAIVE_OCP. */
size_t quantize_blocks_tensor_scaled_workspace_size(int64_t N, int64_t K);
hd_status quantize_blocks_tensor_scaled(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt,
                                        int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                                        float *tensor_scale, float *block_obj, void *ws, size_t ws_bytes,
                                        void *stream);
hd_status dequantize_tensor_scaled(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales,
                                   const float *tensor_scale, int64_t N, int64_t K, void *Wq, hd_dtype out_t,
                                   void *stream);

/* ----------------------------------------------------------------- GPTQ --- */

/* GPTQ on top of a scale choice (qwantize "Results", "GPTQ Quantization": GPTQ
 * of Frantar et al. with its block size equal to the quantisation block size;
 * the quantisation-algorithms note, §1: H = X^T X + lambda I, columns
 * quantised in sequence with each residual propagated through H^-1).
 *
 * gptq_hessian: H = X^T X, float32 [K, K] row-major, for bfloat16 X [M, K]
 * (products exact, float32 accumulation on the MFMA units; for K % 8 == 0 the
 * lower triangle is computed and mirrored, so H is exactly symmetric).
 * Workspace: gptq_hessian_workspace_size(M, K) bytes (256 when K % 8 == 0, X
 * being read in place; otherwise X^T is staged there).  Errors:
 * HD_ERR_UNSUPPORTED for float32 X; HD_ERR_INVALID_ARG for K > 65535, NULL or
 * misaligned pointers, a short workspace.
 *
 * gptq_quantize: codes / scales as quantize_blocks writes them, for W [N, K]
 * quantised with `method` inside the GPTQ column loop:
 *   - h_j = H_jj weights H-Optimal; lambda = damp * mean_j H_jj (1 if that mean
 *     is 0; the usual damp is 0.01) is added to the diagonal;
 *   - ordered == 0 (GPTQ-Seq): block columns left to right; ordered != 0
 *     (GPTQ-Ord): by descending Hessian-weighted loss sum_n sum_{j in b}
 *     h_j (w - q)^2 of the method's own quantisation of W (ties: lower block
 *     first); block_order (optional, device int32 [K/B]) receives the
 *     processing order as original block indices;
 *   - with U the upper Cholesky factor of (H + lambda I)^-1 in processing
 *     order, each block's scales are chosen by `method` from the block's
 *     current (compensated) values, then its columns are encoded in order and
 *     each error (w_c - q_c) / U_cc is subtracted, times U_ck, from every later
 *     column k (scales and codes are taken from the working values rounded to
 *     float32, the quantiser's input; the working weights, the errors, the
 *     factor and the updates are float64, so decisions follow a float64
 *     computation of the loop);
 *   - info (optional, device int32): 0, or 1 + the first pivot at which the
 *     damped Hessian was not positive definite (that pivot is replaced by 1).
 * Workspace: gptq_workspace_size(B, N, K) bytes, about 3.8 K^2 doubles +
 * 8 N K bytes (3.1 GB for K = 9728, N = 2560).  Errors as
 * quantize_blocks, plus K > 65535 and a negative or non-finite damp.
 * Schedule: HD_SCHED_GPTQ_TILE (hdiag_set_schedule) = 64 or 128 fixes the
 * output tile width of the factorisation's float64
 * matrix-core products of 256 rows and columns and up; otherwise 128 is used
 * when it gives at least two rounds of workgroups.  Results agree to float64
 * rounding either way. */
size_t gptq_hessian_workspace_size(int64_t M, int64_t K);
hd_status gptq_hessian(const void *X, hd_dtype xt, int64_t M, int64_t K, float *H, void *ws, size_t ws_bytes,
                       void *stream);
size_t gptq_workspace_size(int32_t B, int64_t N, int64_t K);
hd_status gptq_quantize(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N, int64_t K,
                        const float *H, double damp, int32_t ordered, uint8_t *codes, uint8_t *scales,
                        int32_t *block_order, int32_t *info, void *ws, size_t ws_bytes, void *stream);

/* GPTQ-Seq with the factor made once: the column loop of sequential-order
 * GPTQ reads only V = (L^-1)^T of the damped Hessian H + lambda I (lambda as
 * gptq_quantize takes it from damp), which depends on H and damp alone, so
 * every call on one layer (any format, block size and method) can share it.
 * gptq_factor() writes it, with the factorisation's status, to a caller
 * buffer of gptq_factor_size(K) bytes (16-byte aligned; workspace
 * gptq_factor_workspace_size(K)); info (optional, device int32) gets the
 * status as gptq_quantize reports it.  gptq_quantize_factored() is
 * gptq_quantize(..., ordered = 0) with the factor's V in place of its own
 * factorisation: the same codes, scales, block_order and info bit for bit.
 * H is still read (its diagonal weights H-Optimal); workspace as
 * gptq_quantize.  Errors as gptq_quantize, plus HD_ERR_INVALID_ARG for a
 * short factor buffer. */
size_t gptq_factor_size(int64_t K);
size_t gptq_factor_workspace_size(int64_t K);
hd_status gptq_factor(const float *H, int64_t K, double damp, void *factor, size_t factor_bytes, int32_t *info,
                      void *ws, size_t ws_bytes, void *stream);
hd_status gptq_quantize_factored(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N,
                                 int64_t K, const float *H, const void *factor, size_t factor_bytes, uint8_t *codes,
                                 uint8_t *scales, int32_t *block_order, int32_t *info, void *ws, size_t ws_bytes,
                                 void *stream);

/* ------------------------------------------------------------ utilities --- */

/* Static description of a status code. */
const char *hdiag_strerror(hd_status s);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *hdiag_last_error(void);

/* Format facts: bits of one element code, bits of one scale, number of search
 * candidates (for the FP16 scale grids: the 31743 positive finite values the
 * alternation may land on), and total bits per weight = elem_bits +
 * scale_bits / B (qwantize "Results", "Larger blocks" layout table: 4.5 /
 * 4.25 / 4.125 for FP4 with an 8-bit scale at B = 16 / 32 / 64, and 4.125
 * with an FP16 scale at B = 128).  Any output pointer may be
 * NULL.  Host-only; needs no GPU. */
hd_status hdiag_format_info(hd_format fmt, int32_t B, int *elem_bits, int *scale_bits,
                            int *n_candidates, double *bits_per_weight);

/* Library version string.  Host-only. */
const char *hdiag_version(void);

/* ---------------------------------------------------------- measurement --- */

/* Streaming probes: kernels with the memory access patterns of the
 * HBM-bound stages and next to no arithmetic, for measuring the bandwidth a
 * kernel with those loads and stores reaches at best (no passage of the
 * pages defines them; they serve the measurement of the stages against the
 * HBM roofline).  n counts 16-bit elements, n % 8192 == 0; every buffer is
 * device memory, 16-byte aligned (out1 of ENCODE and in1 of DEQUANT:
 * 4-byte), and caller-allocated:
 *   HD_PROBE_READ:    in0 = n bf16 read; out0 = n / 8192 uint32, word w the
 *                     XOR of the 32-bit words of elements 8192 w .. + 8191;
 *   HD_PROBE_ENCODE:  in0 = n bf16; out0 = n / 2 bytes, one 32-bit word per
 *                     8 elements (the XOR of their four words); out1 = n / 16
 *                     bytes, per 16 elements the low byte of the first
 *                     8-element word (the NVFP4 B = 16 encode's byte mix);
 *   HD_PROBE_WRITE:   out0 = n bf16, 32-bit word i = i;
 *   HD_PROBE_DEQUANT: in0 = n / 2 bytes (a 32-bit word c per 8 elements), in1
 *                     = n / 16 bytes (a byte s per 16 elements); out0 = n bf16,
 *                     per 8 elements the words {c ^ s, c + s, 3 c, c >> 3} (the
 *                     dequantize-to-bfloat16 byte mix).
 * Errors: HD_ERR_INVALID_ARG for an unknown kind, n < 0, n % 8192 != 0, or a
 * NULL or misaligned buffer the kind uses. */
typedef enum { HD_PROBE_READ = 0, HD_PROBE_ENCODE = 1, HD_PROBE_WRITE = 2, HD_PROBE_DEQUANT = 3 } hd_probe;
hd_status hdiag_stream_probe(hd_probe kind, int64_t n, const void *in0, const void *in1, void *out0, void *out1,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HDIAG_H */
