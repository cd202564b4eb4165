// abi.cpp - the C ABI of libhdiag.so: argument validation, error reporting and
// dispatch to the kernel launchers.  Nothing here allocates device memory.
#include <atomic>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "hdiag.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

hd_status fail(hd_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

hd_status ok()
{
    g_last_error[0] = '\0';
    return HD_OK;
}

hd_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(HD_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_dtype(int d) { return d == HD_F32 || d == HD_BF16; }
bool valid_fmt(int f) { return f >= HD_INT8_E4M3 && f <= HD_INT4_F16; }
bool valid_block(int32_t B) { return B == 8 || B == 16 || B == 32 || B == 64 || B == 128 || B == 256; }
// B = 4 (two blocks per 8-weight lane chunk): Naive, encode and dequantize only
bool valid_block4(int32_t B) { return B == 4 || valid_block(B); }
bool is_4bit(int f)
{
    return f == HD_NVFP4 || f == HD_MXFP4 || f == HD_NVFP4_UE4M4 || f == HD_NVFP4_UE5M3 || f == HD_NVINT4 ||
           f == HD_FP4_F16 || f == HD_INT4_F16;
}
bool is_e8m0(int f) { return f == HD_MXFP4 || f == HD_MXFP8; }
bool is_f16(int f) { return f == HD_FP4_F16 || f == HD_INT4_F16; }

#define HD_REQUIRE(cond, ...) \
    do {                      \
        if (!(cond)) return fail(HD_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

hd_status check_ptr(const void *p, const char *name, bool needed)
{
    if (!needed) return HD_OK;
    if (p == nullptr) return fail(HD_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(HD_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return HD_OK;
}

#define HD_CHECK_PTR(p, needed)                                       \
    do {                                                              \
        hd_status s_ = check_ptr((const void *)(p), #p, (needed));    \
        if (s_ != HD_OK) return s_;                                   \
    } while (0)

hd_status check_quant_shape(int fmt, int32_t B, int64_t N, int64_t K, bool naive_path = false)
{
    HD_REQUIRE(valid_fmt(fmt), "unknown format %d", fmt);
    if (B == 4 && !naive_path)
        return fail(HD_ERR_UNSUPPORTED, "block size 4 is supported by Naive scales, encode_blocks and dequantize only");
    HD_REQUIRE(valid_block4(B), "block size %d is not one of 4, 8, 16, 32, 64, 128, 256", (int)B);
    HD_REQUIRE(B != 4 || K % 8 == 0, "block size 4 needs K %% 8 == 0 (K=%lld)", (long long)K);
    HD_REQUIRE(N >= 0 && K >= 0, "negative size N=%lld K=%lld", (long long)N, (long long)K);
    HD_REQUIRE(K % B == 0, "K=%lld is not a multiple of B=%d", (long long)K, (int)B);
    HD_REQUIRE(N <= (int64_t)1 << 40 && K <= (int64_t)1 << 31, "size too large");
    HD_REQUIRE(N * K / B <= (int64_t)1 << 40, "size too large");
    return HD_OK;
}

std::atomic<int> g_schedule[HD_SCHED_COUNT];

}  // namespace

int hd::schedule_setting(int knob)
{
    return knob >= 0 && knob < HD_SCHED_COUNT ? g_schedule[knob].load(std::memory_order_relaxed) : 0;
}

extern "C" {

hd_status hdiag_set_schedule(hd_schedule knob, int32_t value)
{
    HD_REQUIRE(knob >= 0 && knob < HD_SCHED_COUNT, "unknown schedule setting %d", (int)knob);
    HD_REQUIRE(value >= 0, "schedule value %d is negative", (int)value);
    if (knob == HD_SCHED_GPTQ_TILE)
        HD_REQUIRE(value == 0 || value == 64 || value == 128, "GPTQ tile %d is not 0, 64 or 128", (int)value);
    g_schedule[knob].store(value, std::memory_order_relaxed);
    return ok();
}

const char *hdiag_version(void) { return "hdiag 0.1 (gfx950)"; }

const char *hdiag_strerror(hd_status s)
{
    switch (s) {
    case HD_OK: return "success";
    case HD_ERR_INVALID_ARG: return "invalid argument";
    case HD_ERR_UNSUPPORTED: return "unsupported combination";
    case HD_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *hdiag_last_error(void) { return g_last_error; }

hd_status hdiag_format_info(hd_format fmt, int32_t B, int *elem_bits, int *scale_bits, int *n_candidates,
                            double *bits_per_weight)
{
    HD_REQUIRE(valid_fmt(fmt), "unknown format %d", (int)fmt);
    HD_REQUIRE(B > 0, "block size must be positive");
    const int eb = is_4bit(fmt) ? 4 : 8;
    const int sb = is_f16(fmt) ? 16 : 8;
    const int nc = is_f16(fmt) ? 0x7BFF : (is_e8m0(fmt) || fmt == HD_NVFP4_UE4M4 || fmt == HD_NVFP4_UE5M3) ? 255 : 126;
    if (elem_bits) *elem_bits = eb;
    if (scale_bits) *scale_bits = sb;
    if (n_candidates) *n_candidates = nc;
    if (bits_per_weight) *bits_per_weight = (double)eb + (double)sb / (double)B;
    return ok();
}

hd_status hdiag_stream_probe(hd_probe kind, int64_t n, const void *in0, const void *in1, void *out0, void *out1,
                             void *stream)
{
    HD_REQUIRE(kind >= HD_PROBE_READ && kind <= HD_PROBE_DEQUANT, "unknown probe kind %d", (int)kind);
    HD_REQUIRE(n >= 0 && n % 8192 == 0, "n=%lld is not a non-negative multiple of 8192", (long long)n);
    if (n == 0) return ok();
    HD_CHECK_PTR(in0, kind != HD_PROBE_WRITE);
    HD_CHECK_PTR(out0, true);
    if (kind == HD_PROBE_ENCODE)
        HD_REQUIRE(out1 != nullptr && ((uintptr_t)out1 & 3u) == 0, "out1 is NULL or not 4-byte aligned");
    if (kind == HD_PROBE_DEQUANT) HD_REQUIRE(in1 != nullptr, "in1 is NULL");
    return hip_status(hd::launch_stream_probe(kind, n, in0, in1, out0, out1, (hipStream_t)stream),
                      "hdiag_stream_probe");
}

size_t hdiag_workspace_size(int64_t M, int64_t K)
{
    if (M < 0 || K <= 0) return 0;
    return hd::hdiag_ws(M, K);
}

hd_status hdiag(const void *X, hd_dtype xt, int64_t M, int64_t K, float *h, void *ws, size_t ws_bytes,
                void *stream)
{
    HD_REQUIRE(valid_dtype(xt), "unknown dtype %d", (int)xt);
    HD_REQUIRE(M >= 0 && K >= 0, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K == 0) return ok();
    HD_CHECK_PTR(h, true);
    HD_CHECK_PTR(X, M > 0);
    HD_CHECK_PTR(ws, true);
    const size_t need = hd::hdiag_ws(M, K);
    HD_REQUIRE(ws_bytes >= need, "workspace of %zu bytes is short of %zu", ws_bytes, need);
    return hip_status(hd::launch_hdiag(X, xt, M, K, h, ws, (hipStream_t)stream), "hdiag");
}

hd_status hdiag_noalloc(const void *X, hd_dtype xt, int64_t M, int64_t K, float *h, void *stream)
{
    HD_REQUIRE(valid_dtype(xt), "unknown dtype %d", (int)xt);
    HD_REQUIRE(M >= 0 && K >= 0, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K == 0) return ok();
    HD_CHECK_PTR(h, true);
    HD_CHECK_PTR(X, M > 0);
    const size_t need = hd::hdiag_ws(M, K), have = hd::hdiag_noalloc_limit();
    if (need > have)
        return fail(HD_ERR_UNSUPPORTED, "hdiag_noalloc: X [%lld, %lld] needs %zu bytes of partials, beyond the %zu-byte static scratch; use hdiag() with a workspace",
                    (long long)M, (long long)K, need, have);
    void *ws = nullptr;
    hd_status s = hip_status(hd::hdiag_scratch_address((hipStream_t)stream, &ws), "hdiag_noalloc (scratch address)");
    if (s != HD_OK) return s;
    return hip_status(hd::launch_hdiag(X, xt, M, K, h, ws, (hipStream_t)stream), "hdiag_noalloc");
}

hd_status quantize_blocks(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N,
                          int64_t K, const float *h, uint8_t *codes, uint8_t *scales, float *block_obj,
                          void *stream)
{
    return quantize_blocks_instrumented(method, fmt, B, W, wt, N, K, h, codes, scales, block_obj, nullptr, stream);
}

hd_status quantize_blocks_instrumented(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt,
                                       int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                                       float *block_obj, uint64_t *evaluated, void *stream)
{
    if (evaluated != nullptr && ((uintptr_t)evaluated & 7u))
        return fail(HD_ERR_INVALID_ARG, "evaluated is not 8-byte aligned");
    HD_REQUIRE(method >= HD_NAIVE && method <= HD_NAIVE_OCP, "unknown method %d", (int)method);
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    hd_status s = check_quant_shape(fmt, B, N, K, method == HD_NAIVE || method == HD_NAIVE_OCP);
    if (s != HD_OK) return s;
    HD_REQUIRE(method != HD_H_OPT || h != nullptr, "H-Optimal needs h");
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(W, true);
    HD_CHECK_PTR(codes, true);
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if ((uintptr_t)scales & 3u) return fail(HD_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    if (h != nullptr && !aligned16(h)) return fail(HD_ERR_INVALID_ARG, "h is not 16-byte aligned");
    if (block_obj != nullptr && ((uintptr_t)block_obj & 3u)) return fail(HD_ERR_INVALID_ARG, "block_obj misaligned");
    hipStream_t st = (hipStream_t)stream;
    HD_REQUIRE(method != HD_NAIVE_OCP || is_e8m0(fmt), "the OCP rule needs a power-of-two (E8M0) scale grid");
    if (method == HD_NAIVE || method == HD_NAIVE_OCP)
        return hip_status(hd::launch_encode(fmt, B, W, wt, N, K, h, nullptr, codes, scales, block_obj,
                                            method == HD_NAIVE_OCP, st),
                          "quantize_blocks(naive)");
    const float *hh = method == HD_H_OPT ? h : nullptr;
    if (is_f16(fmt))
        return hip_status(hd::launch_alt_f16(fmt, B, W, wt, N, K, hh, codes, scales, block_obj, st),
                          "quantize_blocks(alternation)");
    return hip_status(hd::launch_search(fmt, B, W, wt, N, K, hh, codes, scales, block_obj,
                                        reinterpret_cast<unsigned long long *>(evaluated), st),
                      "quantize_blocks(search)");
}

hd_status encode_blocks(hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N, int64_t K,
                        const uint8_t *scales_in, const float *h, uint8_t *codes, float *block_obj, void *stream)
{
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    hd_status s = check_quant_shape(fmt, B, N, K, true);
    if (s != HD_OK) return s;
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(W, true);
    HD_CHECK_PTR(codes, true);
    if (scales_in == nullptr) return fail(HD_ERR_INVALID_ARG, "scales_in is NULL");
    if (is_f16(fmt) && ((uintptr_t)scales_in & 1u)) return fail(HD_ERR_INVALID_ARG, "scales_in is not 2-byte aligned");
    if (h != nullptr && !aligned16(h)) return fail(HD_ERR_INVALID_ARG, "h is not 16-byte aligned");
    if (block_obj != nullptr && ((uintptr_t)block_obj & 3u)) return fail(HD_ERR_INVALID_ARG, "block_obj misaligned");
    return hip_status(hd::launch_encode(fmt, B, W, wt, N, K, h, scales_in, codes, nullptr, block_obj, 0,
                                        (hipStream_t)stream),
                      "encode_blocks");
}

hd_status dequantize(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                     void *Wq, hd_dtype out_t, void *stream)
{
    HD_REQUIRE(valid_dtype(out_t), "unknown dtype %d", (int)out_t);
    hd_status s = check_quant_shape(fmt, B, N, K, true);
    if (s != HD_OK) return s;
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(codes, true);
    HD_CHECK_PTR(Wq, true);
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if (is_f16(fmt) && ((uintptr_t)scales & 1u)) return fail(HD_ERR_INVALID_ARG, "scales is not 2-byte aligned");
    return hip_status(hd::launch_dequant(fmt, B, codes, scales, N, K, Wq, out_t, nullptr, (hipStream_t)stream),
                      "dequantize");
}

size_t weight_error_workspace_size(int64_t N, int64_t K) { return hd::weight_error_ws(N, K); }

hd_status weight_error(const void *W, hd_dtype wt, const void *Wq, hd_dtype qt, int64_t N, int64_t K, double *out,
                       double *sums, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(valid_dtype(wt) && valid_dtype(qt), "unknown dtype");
    HD_REQUIRE(N >= 0 && K >= 0, "negative size");
    HD_REQUIRE(K % 8 == 0, "K=%lld must be a multiple of 8", (long long)K);
    HD_REQUIRE(out != nullptr, "out is NULL");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::weight_error_ws(N, K), "workspace too small");
    HD_CHECK_PTR(W, N * K > 0);
    HD_CHECK_PTR(Wq, N * K > 0);
    return hip_status(hd::launch_weight_error(W, wt, Wq, qt, N, K, out, sums, ws, (hipStream_t)stream),
                      "weight_error");
}

hd_status dequantize_weight_error(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales, int64_t N,
                                  int64_t K, void *Wq, hd_dtype out_t, const void *W, hd_dtype wt, double *out,
                                  double *sums, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(valid_dtype(out_t) && valid_dtype(wt), "unknown dtype");
    hd_status s = check_quant_shape(fmt, B, N, K, true);
    if (s != HD_OK) return s;
    HD_REQUIRE(K % 8 == 0, "K=%lld must be a multiple of 8", (long long)K);
    HD_REQUIRE(out != nullptr, "out is NULL");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::weight_error_ws(N, K), "workspace too small");
    const bool any = N * K > 0;
    HD_CHECK_PTR(codes, any);
    HD_CHECK_PTR(Wq, any);
    HD_CHECK_PTR(W, any);
    if (any && scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if (any && is_f16(fmt) && ((uintptr_t)scales & 1u)) return fail(HD_ERR_INVALID_ARG, "scales is not 2-byte aligned");
    return hip_status(hd::launch_dequant_weight_error(fmt, B, codes, scales, N, K, Wq, out_t, W, wt, out, sums, ws,
                                                      (hipStream_t)stream),
                      "dequantize_weight_error");
}

size_t output_error_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    // the larger of the two paths, so a caller need not know which one runs
    const size_t a = hd::output_error_ws(M, N, K, true), b = hd::output_error_ws(M, N, K, false);
    return a > b ? a : b;
}

static hd_status output_error_common(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt,
                                     const void *Wq, hd_dtype qt, int64_t N, int64_t K, const double *ysq,
                                     double *out, double *sums, void *ws, size_t ws_bytes, void *stream,
                                     const char *what)
{
    HD_REQUIRE(valid_dtype(xt) && valid_dtype(wt) && valid_dtype(qt), "unknown dtype");
    HD_REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    HD_REQUIRE(K % 8 == 0, "K=%lld must be a multiple of 8", (long long)K);
    HD_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31, "size too large");
    HD_REQUIRE(out != nullptr, "out is NULL");
    HD_CHECK_PTR(ws, true);
    const bool mfma = hd::output_error_uses_mfma(xt, wt, K);
    HD_REQUIRE(ws_bytes >= hd::output_error_ws(M, N, K, mfma), "workspace too small");
    HD_CHECK_PTR(X, M * K > 0);
    HD_CHECK_PTR(W, N * K > 0);
    HD_CHECK_PTR(Wq, N * K > 0);
    return hip_status(
        hd::launch_output_error(X, xt, M, W, wt, Wq, qt, N, K, ysq, out, sums, ws, (hipStream_t)stream), what);
}

hd_status output_error(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt, const void *Wq,
                       hd_dtype qt, int64_t N, int64_t K, double *out, double *sums, void *ws, size_t ws_bytes,
                       void *stream)
{
    return output_error_common(X, xt, M, W, wt, Wq, qt, N, K, nullptr, out, sums, ws, ws_bytes, stream,
                               "output_error");
}

hd_status output_error_given_ref(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt,
                                 const void *Wq, hd_dtype qt, int64_t N, int64_t K, const double *ysq,
                                 double *out, double *sums, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(ysq != nullptr, "ysq is NULL");
    return output_error_common(X, xt, M, W, wt, Wq, qt, N, K, ysq, out, sums, ws, ws_bytes, stream,
                               "output_error_given_ref");
}

size_t output_reference_size(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    return (size_t)hd::output_reference_layout(M, N, K).bytes;
}

hd_status output_reference(const void *X, hd_dtype xt, int64_t M, const void *W, hd_dtype wt, int64_t N, int64_t K,
                           void *ref, size_t ref_bytes, void *stream)
{
    HD_REQUIRE(valid_dtype(xt) && valid_dtype(wt), "unknown dtype");
    HD_REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    HD_REQUIRE(K % 8 == 0, "K=%lld must be a multiple of 8", (long long)K);
    HD_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= (int64_t)1 << 31, "size too large");
    if (xt != HD_BF16 || wt != HD_BF16)
        return fail(HD_ERR_UNSUPPORTED, "output_reference needs bfloat16 X and W (output_error takes float32)");
    HD_CHECK_PTR(ref, true);
    HD_REQUIRE(ref_bytes >= (size_t)hd::output_reference_layout(M, N, K).bytes, "reference buffer too small");
    HD_CHECK_PTR(X, M * K > 0);
    HD_CHECK_PTR(W, N * K > 0);
    return hip_status(hd::launch_output_reference(X, M, W, N, K, ref, (hipStream_t)stream), "output_reference");
}

size_t output_error_codes_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    return hd::output_error_codes_ws(M, N, K);
}

hd_status output_error_codes(hd_format fmt, int32_t B, const void *X, hd_dtype xt, int64_t M, const uint8_t *codes,
                             const uint8_t *scales, int64_t N, int64_t K, const void *ref, size_t ref_bytes,
                             double *out, double *sums, void *ws, size_t ws_bytes, void *stream)
{
    hd_status s = check_quant_shape(fmt, B, N, K);
    if (s != HD_OK) return s;
    HD_REQUIRE(valid_dtype(xt), "unknown dtype %d", (int)xt);
    HD_REQUIRE(M >= 0, "negative size");
    HD_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= (int64_t)1 << 31, "size too large");
    if (xt != HD_BF16) return fail(HD_ERR_UNSUPPORTED, "output_error_codes needs bfloat16 X");
    if (is_f16(fmt))
        return fail(HD_ERR_UNSUPPORTED, "output_error_codes: FP16 block scales do not give an exact 16-bit operand "
                                        "(use dequantize + output_error)");
    HD_REQUIRE(out != nullptr, "out is NULL");
    HD_CHECK_PTR(ref, true);
    HD_REQUIRE(ref_bytes >= (size_t)hd::output_reference_layout(M, N, K).bytes, "reference buffer too small");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::output_error_codes_ws(M, N, K), "workspace too small");
    HD_CHECK_PTR(X, M * K > 0);
    HD_CHECK_PTR(codes, N * K > 0);
    if (N * K > 0 && scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    return hip_status(hd::launch_output_error_codes(fmt, B, X, M, codes, scales, N, K, ref, out, sums, ws,
                                                    (hipStream_t)stream),
                      "output_error_codes");
}

size_t output_gram_size(int64_t K)
{
    if (K < 0) return 0;
    return (size_t)hd::output_gram_layout(K).bytes;
}

size_t output_gram_workspace_size(int64_t M, int64_t K)
{
    if (M < 0 || K < 0) return 0;
    return hd::output_gram_ws(M, K);
}

hd_status output_gram(const void *X, hd_dtype xt, int64_t M, int64_t K, const float *h, void *gram,
                      size_t gram_bytes, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(valid_dtype(xt), "unknown dtype %d", (int)xt);
    HD_REQUIRE(M >= 0 && K >= 0, "negative size");
    HD_REQUIRE(M <= (int64_t)1 << 31 && K <= (int64_t)1 << 17, "size too large");
    HD_REQUIRE(K % 8 == 0, "K=%lld is not a multiple of 8", (long long)K);
    if (xt != HD_BF16) return fail(HD_ERR_UNSUPPORTED, "output_gram needs bfloat16 X (the MFMA product)");
    HD_CHECK_PTR(gram, true);
    HD_REQUIRE(gram_bytes >= (size_t)hd::output_gram_layout(K).bytes, "gram buffer too small");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::output_gram_ws(M, K), "workspace too small");
    HD_CHECK_PTR(X, M * K > 0);
    HD_CHECK_PTR(h, h != nullptr);
    return hip_status(hd::launch_output_gram(X, M, K, h, gram, ws, (hipStream_t)stream), "output_gram");
}

size_t output_error_gram_workspace_size(int64_t N, int64_t K)
{
    if (N < 0 || K < 0) return 0;
    return hd::output_error_gram_ws(1, N, K);
}

size_t output_error_gram_batch_workspace_size(int32_t count, int64_t N, int64_t K)
{
    if (count < 1 || N < 0 || K < 0) return 0;
    return hd::output_error_gram_ws(count, N, K);
}

hd_status output_reference_gram(const void *W, hd_dtype wt, int64_t N, int64_t K, const void *gram,
                                size_t gram_bytes, double *ysq, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    HD_REQUIRE(N >= 0 && K >= 0, "negative size");
    HD_REQUIRE(N <= (int64_t)1 << 31 && K <= (int64_t)1 << 17, "size too large");
    HD_REQUIRE(K % 8 == 0, "K=%lld is not a multiple of 8", (long long)K);
    HD_REQUIRE(ysq != nullptr, "ysq is NULL");
    HD_CHECK_PTR(gram, true);
    HD_REQUIRE(gram_bytes >= (size_t)hd::output_gram_layout(K).bytes, "gram buffer too small");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::output_error_gram_ws(1, N, K), "workspace too small");
    HD_CHECK_PTR(W, N * K > 0);
    return hip_status(hd::launch_output_error_gram(1, nullptr, nullptr, nullptr, nullptr, W, wt, N, K, gram, nullptr,
                                                   ysq, nullptr, nullptr, ws, (hipStream_t)stream),
                      "output_reference_gram");
}

hd_status output_error_gram_batch(int32_t count, const hd_format *fmts, const int32_t *Bs,
                                  const uint8_t *const *codes, const uint8_t *const *scales, const void *W,
                                  hd_dtype wt, int64_t N, int64_t K, const void *gram, size_t gram_bytes,
                                  const double *ysq, double *out, double *sums, void *ws, size_t ws_bytes,
                                  void *stream)
{
    HD_REQUIRE(count >= 1 && count <= 4096, "count=%d is not in 1..4096", (int)count);
    HD_REQUIRE(fmts != nullptr && Bs != nullptr && codes != nullptr && scales != nullptr,
               "fmts, Bs, codes and scales must be host arrays of count entries");
    int f[4096], b[4096];
    for (int32_t q = 0; q < count; ++q) {
        hd_status s = check_quant_shape(fmts[q], Bs[q], N, K);
        if (s != HD_OK) return s;
        f[q] = (int)fmts[q];
        b[q] = (int)Bs[q];
        HD_CHECK_PTR(codes[q], N * K > 0);
        if (N * K > 0 && scales[q] == nullptr) return fail(HD_ERR_INVALID_ARG, "scales[%d] is NULL", (int)q);
    }
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    HD_REQUIRE(N <= (int64_t)1 << 31 && K <= (int64_t)1 << 17, "size too large");
    HD_REQUIRE(out != nullptr, "out is NULL");
    HD_REQUIRE(ysq != nullptr, "ysq is NULL");
    HD_CHECK_PTR(gram, true);
    HD_REQUIRE(gram_bytes >= (size_t)hd::output_gram_layout(K).bytes, "gram buffer too small");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= hd::output_error_gram_ws(count, N, K), "workspace too small");
    HD_CHECK_PTR(W, N * K > 0);
    return hip_status(hd::launch_output_error_gram(count, f, b, codes, scales, W, wt, N, K, gram, ysq, nullptr, out,
                                                   sums, ws, (hipStream_t)stream),
                      "output_error_gram_batch");
}

hd_status output_error_gram(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales, const void *W,
                            hd_dtype wt, int64_t N, int64_t K, const void *gram, size_t gram_bytes,
                            const double *ysq, double *out, double *sums, void *ws, size_t ws_bytes, void *stream)
{
    if (codes == nullptr && N * K > 0) return fail(HD_ERR_INVALID_ARG, "codes is NULL");
    const uint8_t *cs[1] = {codes}, *ss[1] = {scales};
    const hd_format fs[1] = {fmt};
    const int32_t bs[1] = {B};
    return output_error_gram_batch(1, fs, bs, cs, ss, W, wt, N, K, gram, gram_bytes, ysq, out, sums, ws, ws_bytes,
                                   stream);
}

size_t gptq_factor_size(int64_t K)
{
    if (K < 0) return 0;
    return (size_t)hd::gptq_factor_bytes(K);
}

size_t gptq_factor_workspace_size(int64_t K)
{
    if (K < 0) return 0;
    return (size_t)hd::gptq_factor_ws(K);
}

hd_status gptq_factor(const float *H, int64_t K, double damp, void *factor, size_t factor_bytes, int32_t *info,
                      void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(K >= 0 && K <= 65535, "size too large (K <= 65535)");
    HD_REQUIRE(damp >= 0.0 && damp < 1e300, "damp must be a finite non-negative number");
    if (K == 0) return ok();
    HD_CHECK_PTR(H, true);
    HD_CHECK_PTR(factor, true);
    HD_REQUIRE(factor_bytes >= (size_t)hd::gptq_factor_bytes(K), "factor buffer too small");
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(ws_bytes >= (size_t)hd::gptq_factor_ws(K), "workspace too small");
    if (info != nullptr && ((uintptr_t)info & 3u)) return fail(HD_ERR_INVALID_ARG, "info misaligned");
    return hip_status(hd::launch_gptq_factor(H, K, damp, factor, info, ws, (hipStream_t)stream), "gptq_factor");
}

hd_status gptq_quantize_factored(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N,
                                 int64_t K, const float *H, const void *factor, size_t factor_bytes, uint8_t *codes,
                                 uint8_t *scales, int32_t *block_order, int32_t *info, void *ws, size_t ws_bytes,
                                 void *stream)
{
    HD_REQUIRE(method >= HD_NAIVE && method <= HD_NAIVE_OCP, "unknown method %d", (int)method);
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    hd_status s = check_quant_shape(fmt, B, N, K);
    if (s != HD_OK) return s;
    HD_REQUIRE(K <= 65535 && N <= (int64_t)1 << 31, "size too large (K <= 65535)");
    HD_REQUIRE(method != HD_NAIVE_OCP || is_e8m0(fmt), "the OCP rule needs a power-of-two (E8M0) scale grid");
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(W, true);
    HD_CHECK_PTR(H, true);
    HD_CHECK_PTR(factor, true);
    HD_REQUIRE(factor_bytes >= (size_t)hd::gptq_factor_bytes(K), "factor buffer too small");
    HD_CHECK_PTR(codes, true);
    HD_CHECK_PTR(ws, true);
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if ((uintptr_t)scales & 3u) return fail(HD_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    if (block_order != nullptr && ((uintptr_t)block_order & 3u)) return fail(HD_ERR_INVALID_ARG, "block_order misaligned");
    if (info != nullptr && ((uintptr_t)info & 3u)) return fail(HD_ERR_INVALID_ARG, "info misaligned");
    HD_REQUIRE(ws_bytes >= (size_t)hd::gptq_ws(B, N, K), "workspace too small");
    return hip_status(hd::launch_gptq_factored(method, fmt, B, W, wt, N, K, H, factor, codes, scales, block_order,
                                               info, ws, (hipStream_t)stream),
                      "gptq_quantize_factored");
}

bool is_e4m3_scaled(int f) { return f == HD_INT8_E4M3 || f == HD_NVFP4 || f == HD_FP8_E4M3S || f == HD_NVINT4; }

size_t quantize_blocks_tensor_scaled_workspace_size(int64_t N, int64_t K)
{
    if (N < 0 || K < 0) return 0;
    return (size_t)(256 + ((N * K * 4 + 255) / 256) * 256);
}

hd_status quantize_blocks_tensor_scaled(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt,
                                        int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                                        float *tensor_scale, float *block_obj, void *ws, size_t ws_bytes,
                                        void *stream)
{
    HD_REQUIRE(method >= HD_NAIVE && method <= HD_H_OPT, "unknown method %d (the OCP rule needs E8M0 scales)",
               (int)method);
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    hd_status s = check_quant_shape(fmt, B, N, K, method == HD_NAIVE);
    if (s != HD_OK) return s;
    HD_REQUIRE(is_e4m3_scaled(fmt), "per-tensor scaling needs an E4M3 block-scale format");
    HD_REQUIRE(method != HD_H_OPT || h != nullptr, "H-Optimal needs h");
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(W, true);
    HD_CHECK_PTR(codes, true);
    HD_CHECK_PTR(ws, true);
    HD_REQUIRE(tensor_scale != nullptr && ((uintptr_t)tensor_scale & 3u) == 0, "tensor_scale is NULL or misaligned");
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if ((uintptr_t)scales & 3u) return fail(HD_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    if (h != nullptr && !aligned16(h)) return fail(HD_ERR_INVALID_ARG, "h is not 16-byte aligned");
    if (block_obj != nullptr && ((uintptr_t)block_obj & 3u)) return fail(HD_ERR_INVALID_ARG, "block_obj misaligned");
    HD_REQUIRE(ws_bytes >= quantize_blocks_tensor_scaled_workspace_size(N, K), "workspace too small");
    hipStream_t st = (hipStream_t)stream;
    float *Wp = reinterpret_cast<float *>(static_cast<char *>(ws) + 256);
    hipError_t e = hd::launch_tensor_scale(fmt, W, wt, N, K, tensor_scale, Wp, ws, st);
    if (e != hipSuccess) return hip_status(e, "quantize_blocks_tensor_scaled(scale)");
    if (method == HD_NAIVE)
        return hip_status(hd::launch_encode(fmt, B, Wp, HD_F32, N, K, h, nullptr, codes, scales, block_obj, 0, st),
                          "quantize_blocks_tensor_scaled(naive)");
    const float *hh = method == HD_H_OPT ? h : nullptr;
    return hip_status(hd::launch_search(fmt, B, Wp, HD_F32, N, K, hh, codes, scales, block_obj, nullptr, st),
                      "quantize_blocks_tensor_scaled(search)");
}

hd_status dequantize_tensor_scaled(hd_format fmt, int32_t B, const uint8_t *codes, const uint8_t *scales,
                                   const float *tensor_scale, int64_t N, int64_t K, void *Wq, hd_dtype out_t,
                                   void *stream)
{
    HD_REQUIRE(valid_dtype(out_t), "unknown dtype %d", (int)out_t);
    hd_status s = check_quant_shape(fmt, B, N, K, true);
    if (s != HD_OK) return s;
    HD_REQUIRE(is_e4m3_scaled(fmt), "per-tensor scaling needs an E4M3 block-scale format");
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(codes, true);
    HD_CHECK_PTR(Wq, true);
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    HD_REQUIRE(tensor_scale != nullptr && ((uintptr_t)tensor_scale & 3u) == 0, "tensor_scale is NULL or misaligned");
    return hip_status(hd::launch_dequant(fmt, B, codes, scales, N, K, Wq, out_t, tensor_scale, (hipStream_t)stream),
                      "dequantize_tensor_scaled");
}

size_t gptq_hessian_workspace_size(int64_t M, int64_t K)
{
    if (M < 0 || K < 0) return 0;
    return (size_t)hd::gptq_hessian_ws(M, K);
}

hd_status gptq_hessian(const void *X, hd_dtype xt, int64_t M, int64_t K, float *H, void *ws, size_t ws_bytes,
                       void *stream)
{
    HD_REQUIRE(valid_dtype(xt), "unknown dtype %d", (int)xt);
    HD_REQUIRE(M >= 0 && K >= 0, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    HD_REQUIRE(M <= (int64_t)1 << 31 && K <= 65535, "size too large (K <= 65535)");
    if (xt != HD_BF16) return fail(HD_ERR_UNSUPPORTED, "gptq_hessian needs bfloat16 X (the MFMA product)");
    if (K == 0) return ok();
    HD_CHECK_PTR(H, true);
    HD_CHECK_PTR(ws, true);
    HD_CHECK_PTR(X, M > 0);
    HD_REQUIRE(ws_bytes >= (size_t)hd::gptq_hessian_ws(M, K), "workspace too small");
    return hip_status(hd::launch_gptq_hessian(X, M, K, H, ws, (hipStream_t)stream), "gptq_hessian");
}

size_t gptq_workspace_size(int32_t B, int64_t N, int64_t K)
{
    if (!valid_block(B) || N < 0 || K < 0 || K % B) return 0;
    return (size_t)hd::gptq_ws(B, N, K);
}

hd_status gptq_quantize(hd_method method, hd_format fmt, int32_t B, const void *W, hd_dtype wt, int64_t N, int64_t K,
                        const float *H, double damp, int32_t ordered, uint8_t *codes, uint8_t *scales,
                        int32_t *block_order, int32_t *info, void *ws, size_t ws_bytes, void *stream)
{
    HD_REQUIRE(method >= HD_NAIVE && method <= HD_NAIVE_OCP, "unknown method %d", (int)method);
    HD_REQUIRE(valid_dtype(wt), "unknown dtype %d", (int)wt);
    hd_status s = check_quant_shape(fmt, B, N, K);
    if (s != HD_OK) return s;
    HD_REQUIRE(K <= 65535 && N <= (int64_t)1 << 31, "size too large (K <= 65535)");
    HD_REQUIRE(method != HD_NAIVE_OCP || is_e8m0(fmt), "the OCP rule needs a power-of-two (E8M0) scale grid");
    HD_REQUIRE(damp >= 0.0 && damp < 1e300, "damp must be a finite non-negative number");
    if (N == 0 || K == 0) return ok();
    HD_CHECK_PTR(W, true);
    HD_CHECK_PTR(H, true);
    HD_CHECK_PTR(codes, true);
    HD_CHECK_PTR(ws, true);
    if (scales == nullptr) return fail(HD_ERR_INVALID_ARG, "scales is NULL");
    if ((uintptr_t)scales & 3u) return fail(HD_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    if (block_order != nullptr && ((uintptr_t)block_order & 3u)) return fail(HD_ERR_INVALID_ARG, "block_order misaligned");
    if (info != nullptr && ((uintptr_t)info & 3u)) return fail(HD_ERR_INVALID_ARG, "info misaligned");
    HD_REQUIRE(ws_bytes >= (size_t)hd::gptq_ws(B, N, K), "workspace too small");
    return hip_status(hd::launch_gptq(method, fmt, B, W, wt, N, K, H, damp, ordered != 0, codes, scales, block_order,
                                      info, ws, (hipStream_t)stream),
                      "gptq_quantize");
}

}  // extern "C"

namespace hd {

hipError_t launch_search(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                         uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals,
                         hipStream_t st)
{
    switch (fmt) {
    case HD_INT8_E4M3:
    case HD_NVINT4: return launch_search_int_elems(fmt, B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_NVFP4:
    case HD_MXFP4:
    case HD_NVFP4_UE4M4:
    case HD_NVFP4_UE5M3: return launch_search_e2m1_elems(fmt, B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_MXFP8:
    case HD_FP8_E4M3S: return launch_search_e4m3_elems(fmt, B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hd
