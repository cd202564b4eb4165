// kernels.hpp - launchers behind the C ABI (arguments already validated).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace hd {

// Current value of a schedule setting (hdiag_set_schedule; 0 = automatic).
int schedule_setting(int knob);

// Naive scale + encode (scales_in == NULL), or encode with given scale codes.
// ocp != 0 (E8M0 grids): the OCP MX floor rule instead of the Naive snap.
hipError_t launch_encode(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                         const uint8_t *scales_in, uint8_t *codes, uint8_t *scales, float *block_obj, int ocp,
                         hipStream_t st);

// SSE-Optimal (h == NULL) or H-Optimal search + encode.  evals (optional,
// device): incremented by the number of (weight, candidate) pairs evaluated.
hipError_t launch_search(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                         uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals,
                         hipStream_t st);
// per element family (one translation unit each)
hipError_t launch_search_int_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                   uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals,
                                   hipStream_t st);
hipError_t launch_search_e2m1_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                    uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals,
                                    hipStream_t st);
hipError_t launch_search_e4m3_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                    uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals,
                                    hipStream_t st);

// SSE-Optimal (h == NULL) or H-Optimal binary16 block scales by alternation
// (HD_FP4_F16, HD_INT4_F16) + encode.
hipError_t launch_alt_f16(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                          uint8_t *codes, uint8_t *scales, float *block_obj, hipStream_t st);

// tscale (device float, may be NULL): a per-tensor scale multiplying every value.
hipError_t launch_dequant(int fmt, int B, const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                          void *out, int out_t, const float *tscale, hipStream_t st);

size_t weight_error_ws(int64_t N, int64_t K);
hipError_t launch_weight_error(const void *W, int wdt, const void *Wq, int qdt, int64_t N, int64_t K,
                               double *out, double *sums, void *ws, hipStream_t st);
// dequantize and weight error in one pass (workspace: weight_error_ws)
hipError_t launch_dequant_weight_error(int fmt, int B, const uint8_t *codes, const uint8_t *scales, int64_t N,
                                       int64_t K, void *Wq, int out_t, const void *W, int wdt, double *out,
                                       double *sums, void *ws, hipStream_t st);

size_t hdiag_ws(int64_t M, int64_t K);
hipError_t launch_hdiag(const void *X, int xdt, int64_t M, int64_t K, float *h, void *ws, hipStream_t st);
// hdiag_noalloc's static scratch: its size in bytes, and its device address on
// the device of `st` (the current device for the null stream), looked up once
// per device.
size_t hdiag_noalloc_limit();
hipError_t hdiag_scratch_address(hipStream_t st, void **ptr);

size_t output_error_ws(int64_t M, int64_t N, int64_t K, bool mfma);
bool output_error_uses_mfma(int xdt, int wdt, int64_t K);
// ysq: optional device double holding ||X W^T||^2; when given, Y is not computed.
hipError_t launch_output_error(const void *X, int xdt, int64_t M, const void *W, int wdt, const void *Wq,
                               int qdt, int64_t N, int64_t K, const double *ysq, double *out, double *sums,
                               void *ws, hipStream_t st);

// Output error against a stored reference (outref.hip).  The reference buffer
// holds, at these byte offsets: ||X W^T||^2 (double, offset 0), Y = X W^T
// (float [M][N], offset y), the per-row exponents of X' (int [M], offset e),
// X' (fp16 [M][K], offset x) and the GEMM's workgroup partials (offset part).
struct RefLayout {
    int64_t y, e, x, part, bytes;
};
RefLayout output_reference_layout(int64_t M, int64_t N, int64_t K);
hipError_t launch_output_reference(const void *X, int64_t M, const void *W, int64_t N, int64_t K, void *ref,
                                   hipStream_t st);
size_t output_error_codes_ws(int64_t M, int64_t N, int64_t K);
hipError_t launch_output_error_codes(int fmt, int B, const void *X, int64_t M, const uint8_t *codes,
                                     const uint8_t *scales, int64_t N, int64_t K, const void *ref, double *out,
                                     double *sums, void *ws, hipStream_t st);

// Output error through G = X^T X (outref.hip).  The gram buffer holds, at
// these byte offsets: h (float [K]), sqrt(h) (sq), 1/sqrt(h) or 0 (r) and the
// lower block triangle of C = G / sqrt(h h^T) with zero diagonal, off-diagonal
// 256 x 256 blocks doubled (float16 [K][K], offset c).
struct GramLayout {
    int64_t h, sq, r, c, bytes;
};
GramLayout output_gram_layout(int64_t K);
size_t output_gram_ws(int64_t M, int64_t K);
// h: float [K] = hdiag(X), or NULL to compute it here.
hipError_t launch_output_gram(const void *X, int64_t M, int64_t K, const float *h, void *gram, void *ws,
                              hipStream_t st);
size_t output_error_gram_ws(int64_t count, int64_t N, int64_t K);
// count quantisations (host arrays fmt, B, codes, scales) of one W:
// out[q] = ||X (Wq_q - W)^T|| / sqrt(*ysq); fmt == NULL: ysq_out[0] = ||X W^T||^2.
hipError_t launch_output_error_gram(int count, const int *fmt, const int *B, const uint8_t *const *codes,
                                    const uint8_t *const *scales, const void *W, int wdt, int64_t N, int64_t K,
                                    const void *gram, const double *ysq, double *ysq_out, double *out, double *sums,
                                    void *ws, hipStream_t st);

// Y = A B^T (bf16 A [M][K], B [N][K], float32 Y [M][N]) on the MFMA product of
// outref.hip; part: output_gemm_parts_bytes(M, N) bytes of scratch.
int64_t output_gemm_parts_bytes(int64_t M, int64_t N);
hipError_t launch_gram_store(const void *X, int64_t M, int64_t K, float *H, hipStream_t st);
hipError_t launch_gemm_store(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K, float *Y,
                             double *part, hipStream_t st);

// GPTQ (gptq.hip): H = X^T X (bf16 X), and the column loop on top of a scale
// choice; info (device int, may be NULL) gets 1 + the index of the first
// non-positive pivot of the damped Hessian's factorisation, else 0.
int64_t gptq_hessian_ws(int64_t M, int64_t K);
hipError_t launch_gptq_hessian(const void *X, int64_t M, int64_t K, float *H, void *ws, hipStream_t st);
int64_t gptq_ws(int B, int64_t N, int64_t K);
hipError_t launch_gptq(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *H,
                       double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int *info,
                       void *ws, hipStream_t st);
// The sequential order's factor, made once per (H, damp), and GPTQ-Seq from it.
int64_t gptq_factor_bytes(int64_t K);
int64_t gptq_factor_ws(int64_t K);
hipError_t launch_gptq_factor(const float *H, int64_t K, double damp, void *factor, int *info, void *ws,
                              hipStream_t st);
hipError_t launch_gptq_factored(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                                const float *H, const void *factor, uint8_t *codes, uint8_t *scales,
                                int32_t *block_order, int *info, void *ws, hipStream_t st);

// Per-tensor scaling over E4M3 block scales (tscale.hip): the tensor scale
// into *tscale and W / tscale (float32 [N][K]) into Wp.
hipError_t launch_tensor_scale(int fmt, const void *W, int wdt, int64_t N, int64_t K, float *tscale, float *Wp,
                               void *ws, hipStream_t st);

// measurement probes (probe.hip)
hipError_t launch_stream_probe(int kind, int64_t n, const void *in0, const void *in1, void *out0, void *out1,
                               hipStream_t st);

}  // namespace hd
