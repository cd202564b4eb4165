/*
 * Block-scale quantiser oracle: a plain, slow, obviously correct CPU model of
 * the hot path (hdiag -> scale choice -> encode -> dequantize -> errors).
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
 * baseline of the benchmark are the only callers.  It shares no source, header,
 * table or constant with the GPU library; each side derives its own tables.
 *
 * What each part follows (page, then section / table / equation):
 *   - number formats: LLM-FP4 summary page, "Floating-Point Quantization
 *     Mechanics" (value of an EeMm code, Q_max); qwantize "Results" page,
 *     "Exotic Scales" (E4M3 has 126 positive values, the E2M1 codebook);
 *     "Is Finer Better?" §2.1 (E8M0 power-of-two scales, UE4M3 for NVFP4).
 *   - element rounding: quantisation-algorithms note, §2 (sorted FP32 codepoint
 *     table + binary search for the two neighbouring codepoints), rounded to
 *     nearest with ties to the even code, saturating at the largest code.
 *   - Naive scale: "Is Finer Better?" §2.1 (s = Q_scale(x_max / C),
 *     q = Q_elem(x / s), x^ = s q), App. F.3 (the zero-scale bin); qwantize
 *     "Results", "INT8 (FP8 E4M3 scales)" (amax stored as E4M3, effective scale
 *     amax_fp8 / 127 divided in float32).
 *   - SSE-Optimal / H-Optimal: qwantize "Results", INT8 / NVFP4 / MXFP4 tables
 *     and "Why NVFP4 benefits much more from Hessian-awareness"; the weighted
 *     objective sum_j h_j (w_j - s Q(w_j / s))^2 with h_j the diagonal of X^T X
 *     is the diagonal form in the quantisation-algorithms note, §1.  The oracle
 *     takes the plain definition: the exact argmin over every candidate of the
 *     scale grid, objective in float64 summed in element order, the first
 *     (lowest) code on ties.
 *   - metrics: qwantize "Results", the weight-error and output-error
 *     definitions at the top of the page.
 *
 *   - more grids (qwantize "Results", "Exotic Scales"; "Is Finer Better?"
 *     §5.2): the unsigned UE4M4 (bias 7) and UE5M3 (bias 15) scale grids,
 *     every code finite, 255 positive values, with E2M1 elements; NVINT4
 *     (the "GPTQ Quantization" tables) read as symmetric INT4 elements
 *     [-7, 7] with an E4M3 block scale s = Q_E4M3(amax / 7), the generic
 *     rule of "Is Finer Better?" §2.1 with C = 7; the OCP MX rule for
 *     power-of-two scales, 2^(floor(log2 amax) - emax_elem) (the OCP
 *     microscaling specification the same section cites), as an alternative
 *     Naive for MXFP4 / MXFP8.
 *   - FP16 scales (qwantize "Results", "Larger blocks: bs=64 (E4M3 scales) and
 *     bs=128 (FP16 scales)"): FP4 (E2M1) or INT4 elements with a binary16
 *     (E5M10, bias 15, top exponent reserved) block scale; Naive is
 *     fp16(fl32(amax / C)); SSE-Optimal / H-Optimal are found by alternating
 *     element assignment and the closed-form least-squares scale snapped to
 *     FP16 (f16_alternation below; its readings are listed there).
 *   - per-tensor scaling over E4M3 block scales ("Is Finer Better?" §5.1,
 *     UE4M3-S; orc_quantize_tensor_scaled, its reading is listed there).
 *   - GPTQ (qwantize "Results", "GPTQ Quantization"; quantisation-algorithms
 *     note, §1): H = X^T X (orc_xtx), damped, the upper Cholesky factor of its
 *     inverse, and the column loop of Frantar et al. with the GPTQ block equal
 *     to the quantisation block, in natural or loss order (orc_gptq; its
 *     readings are listed there).
 *
 * Readings where the pages are silent (also listed in the design notes):
 *   E8M0 Naive snap = nearest power of two in the linear domain, ties upward
 *   (parity unpinned beyond self-consistency); negative inputs that round to
 *   zero keep their sign bit in E2M1/E4M3 codes (a convention, parity
 *   unpinned); E2M1 codes pack element 2i in the low nibble (a convention);
 *   INT4 codes are two's complement nibbles, packed the same way.
 *
 * Build: -O2 -ffp-contract=off, no fast-math, so every float expression below
 * is one IEEE binary32 operation rounded to nearest-even (fl32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* format ids (same numbering as the public library, kept independently) */
enum { F_INT8_E4M3 = 0, F_NVFP4 = 1, F_MXFP4 = 2, F_MXFP8 = 3, F_FP8_E4M3S = 4,
       F_NVFP4_UE4M4 = 5, F_NVFP4_UE5M3 = 6, F_NVINT4 = 7, F_FP4_F16 = 8, F_INT4_F16 = 9,
       F_COUNT = 10 };
enum { M_NAIVE = 0, M_SSE = 1, M_H = 2, M_NAIVE_OCP = 3 };
enum { DT_F32 = 0, DT_BF16 = 1 };

/* element kinds */
enum { E_INT8 = 0, E_E2M1 = 1, E_E4M3 = 2, E_INT4 = 3 };
/* scale kinds */
enum { S_E4M3_OF_AMAX_DIV127 = 0, S_E4M3 = 1, S_E8M0 = 2, S_UE4M4 = 3, S_UE5M3 = 4, S_F16 = 5 };

/* rounds of the FP16-scale alternation before it stops without a fixed point */
#define F16_ALT_MAX_ROUNDS 32

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* Non-negative values of a sign-magnitude binary float format EeMm with
 * exponent bias `bias`, in increasing bit-pattern order (code k = p*2^m + d).
 * Exponent field p >= 1 gives 2^(p-bias) * (1 + d/2^m); p = 0 gives the
 * subnormals 2^(1-bias) * (d/2^m).  reserve = 0: every code is finite;
 * 1: only the all-ones pattern is NaN (OCP E4M3FN); 2: the whole top exponent
 * is Inf/NaN (IEEE style).  Returns the count, or ORC_EINVAL if cap is short. */
int orc_fp_table(int ebits, int mbits, int bias, int reserve, double *out, int cap)
{
    int np = 1 << ebits, nd = 1 << mbits, n = 0;
    for (int p = 0; p < np; p++) {
        if (reserve == 2 && p == np - 1)
            break;
        for (int d = 0; d < nd; d++) {
            if (reserve == 1 && p == np - 1 && d == nd - 1)
                break;
            double frac = (double)d / (double)nd;
            double v = (p == 0) ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, p - bias);
            if (n >= cap)
                return ORC_EINVAL;
            out[n++] = v;
        }
    }
    return n;
}

/* E8M0: 255 finite codes c = 0..254 with value 2^(c-127); 0xFF is NaN. */
int orc_e8m0_table(double *out, int cap)
{
    if (cap < 255)
        return ORC_EINVAL;
    for (int c = 0; c < 255; c++)
        out[c] = ldexp(1.0, c - 127);
    return 255;
}

static double T_E2M1[8];
static double T_E4M3[127];
static double T_INT8[128];
static double T_INT4[8];
static double T_UE4M4[256];
static double T_UE5M3[256];
static double T_F16[31744];
static int tables_ready = 0;

static void init_tables(void)
{
    if (tables_ready)
        return;
    orc_fp_table(2, 1, 1, 0, T_E2M1, 8);      /* {0,.5,1,1.5,2,3,4,6} */
    orc_fp_table(4, 3, 7, 1, T_E4M3, 127);    /* 0 .. 448, 0x7F is NaN */
    orc_fp_table(4, 4, 7, 0, T_UE4M4, 256);   /* unsigned, every code finite: 0 .. 496 */
    orc_fp_table(5, 3, 15, 0, T_UE5M3, 256);  /* unsigned, every code finite: 0 .. 122880 */
    orc_fp_table(5, 10, 15, 2, T_F16, 31744); /* FP16 E5M10, top exponent Inf/NaN: 0 .. 65504 */
    for (int i = 0; i < 128; i++)
        T_INT8[i] = (double)i;                /* symmetric INT8 magnitudes */
    for (int i = 0; i < 8; i++)
        T_INT4[i] = (double)i;                /* symmetric INT4 magnitudes 0..7 */
    tables_ready = 1;
}

/* Round a >= 0 onto the sorted table T[0..n-1] (T[0] = 0): saturate at the
 * top; otherwise take the nearer of T[i] <= a < T[i+1], an exact tie going to
 * the even index.  The differences are exact in float64 for these tables. */
int orc_rne_index(const double *T, int n, double a)
{
    if (!(a < T[n - 1]))
        return n - 1;
    int lo = 0, hi = n - 1; /* T[lo] <= a < T[hi] */
    while (hi - lo > 1) {
        int mid = lo + (hi - lo) / 2;
        if (T[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dl = a - T[lo], dh = T[hi] - a;
    if (dl < dh)
        return lo;
    if (dh < dl)
        return hi;
    return (lo % 2 == 0) ? lo : hi;
}

void orc_rne_index_batch(const double *T, int n, const float *x, int64_t count, int32_t *idx)
{
    for (int64_t i = 0; i < count; i++)
        idx[i] = orc_rne_index(T, n, (double)x[i]);
}

static int elem_kind(int fmt)
{
    switch (fmt) {
    case F_INT8_E4M3: return E_INT8;
    case F_NVFP4: case F_MXFP4: case F_NVFP4_UE4M4: case F_NVFP4_UE5M3: case F_FP4_F16: return E_E2M1;
    case F_NVINT4: case F_INT4_F16: return E_INT4;
    default: return E_E4M3;
    }
}

static int scale_kind(int fmt)
{
    switch (fmt) {
    case F_INT8_E4M3: return S_E4M3_OF_AMAX_DIV127;
    case F_NVFP4: case F_FP8_E4M3S: case F_NVINT4: return S_E4M3;
    case F_NVFP4_UE4M4: return S_UE4M4;
    case F_NVFP4_UE5M3: return S_UE5M3;
    case F_FP4_F16: case F_INT4_F16: return S_F16;
    default: return S_E8M0;
    }
}

/* bytes per stored scale: 2 for FP16 scales (little-endian binary16 bits), else 1 */
static int scale_bytes(int fmt) { return scale_kind(fmt) == S_F16 ? 2 : 1; }

static int get_scale(int fmt, const uint8_t *scales, int64_t i)
{
    if (scale_bytes(fmt) == 2)
        return scales[2 * i] | (scales[2 * i + 1] << 8);
    return scales[i];
}

static void put_scale(int fmt, uint8_t *scales, int64_t i, int code)
{
    if (scale_bytes(fmt) == 2) {
        scales[2 * i] = (uint8_t)(code & 0xFF);
        scales[2 * i + 1] = (uint8_t)(code >> 8);
    } else {
        scales[i] = (uint8_t)code;
    }
}

/* elements stored as 4-bit codes, two per byte */
static int four_bit(int fmt) { return elem_kind(fmt) == E_E2M1 || elem_kind(fmt) == E_INT4; }

static const double *elem_table(int fmt, int *n)
{
    switch (elem_kind(fmt)) {
    case E_INT8: *n = 128; return T_INT8;
    case E_INT4: *n = 8; return T_INT4;
    case E_E2M1: *n = 8; return T_E2M1;
    default: *n = 127; return T_E4M3;
    }
}

/* largest element magnitude C of the Naive rule s = Q_scale(amax / C) */
static float elem_cmax(int fmt)
{
    switch (elem_kind(fmt)) {
    case E_E2M1: return 6.0f;
    case E_INT4: return 7.0f;
    default: return 448.0f;
    }
}

/* Candidate scale codes of the search, ascending: the 126 positive E4M3 codes
 * 0x01..0x7E, all 255 finite E8M0 codes, or the 255 positive UE4M4 / UE5M3
 * codes 0x01..0xFF. */
int orc_candidates(int fmt, int *first, int *last)
{
    init_tables();
    if (fmt < 0 || fmt >= F_COUNT)
        return ORC_EINVAL;
    if (scale_kind(fmt) == S_E8M0) {
        *first = 0;
        *last = 254;
    } else if (scale_kind(fmt) == S_UE4M4 || scale_kind(fmt) == S_UE5M3) {
        *first = 1;
        *last = 255;
    } else if (scale_kind(fmt) == S_F16) {
        *first = 1;
        *last = 0x7BFF; /* every positive finite binary16 value */
    } else {
        *first = 1;
        *last = 126;
    }
    return *last - *first + 1;
}

/* The fp32 scale a scale code stands for.  INT8: fl32(val_E4M3(code) / 127);
 * E4M3 grids: val_E4M3(code) (code 0 is the zero scale); E8M0: 2^(code-127)
 * (2^-127 is an fp32 subnormal and exact).  Returns NAN for a NaN code. */
float orc_scale_value(int fmt, int code)
{
    init_tables();
    switch (scale_kind(fmt)) {
    case S_E4M3_OF_AMAX_DIV127:
        if (code < 0 || code > 126) return NAN;
        return (float)T_E4M3[code] / 127.0f;
    case S_E4M3:
        if (code < 0 || code > 126) return NAN;
        return (float)T_E4M3[code];
    case S_UE4M4:
        if (code < 0 || code > 255) return NAN;
        return (float)T_UE4M4[code];
    case S_UE5M3:
        if (code < 0 || code > 255) return NAN;
        return (float)T_UE5M3[code];
    case S_F16:
        if (code < 0 || code > 0x7BFF) return NAN; /* Inf, NaN and negative scales are invalid */
        return (float)T_F16[code];
    default:
        if (code < 0 || code > 254) return NAN;
        return (float)ldexp(1.0, code - 127);
    }
}

/* Naive scale code of a block with max |w| = amax. */
int orc_naive_scale_code(int fmt, float amax)
{
    init_tables();
    int sk = scale_kind(fmt);
    if (sk == S_E4M3_OF_AMAX_DIV127)
        return orc_rne_index(T_E4M3, 127, (double)amax); /* amax itself, saturating at 448 */
    float C = elem_cmax(fmt); /* largest element magnitude */
    float v = amax / C;       /* fl32 */
    if (sk == S_E4M3)
        return orc_rne_index(T_E4M3, 127, (double)v);
    if (sk == S_UE4M4)
        return orc_rne_index(T_UE4M4, 256, (double)v);
    if (sk == S_UE5M3)
        return orc_rne_index(T_UE5M3, 256, (double)v);
    if (sk == S_F16)
        return orc_rne_index(T_F16, 31744, (double)v); /* RNE, saturating at 65504 */
    /* E8M0: nearest power of two in the linear domain, ties upward */
    if (v == 0.0f)
        return 0;
    int e;
    double f = frexp((double)v, &e); /* v = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                   /* v = (2f) * 2^E, 2f in [1, 2) */
    if (2.0 * f >= 1.5)
        E += 1;
    if (E < -127)
        E = -127;
    if (E > 127)
        E = 127;
    return E + 127;
}

/* OCP MX rule for power-of-two scales: 2^(floor(log2 amax) - emax), emax the
 * exponent of the largest element (E2M1: 6 = 1.5 * 2^2; E4M3: 448 = 1.75 * 2^8),
 * clamped to the E8M0 range; an all-zero block gets code 0.  -1 for a format
 * without E8M0 scales. */
int orc_naive_ocp_code(int fmt, float amax)
{
    init_tables();
    if (fmt < 0 || fmt >= F_COUNT || scale_kind(fmt) != S_E8M0)
        return -1;
    if (amax == 0.0f)
        return 0;
    int e;
    frexp((double)amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
    int emax = (elem_kind(fmt) == E_E2M1) ? 2 : 8;
    int E = e - 1 - emax;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E + 127;
}

/* Encode one element with scale s; returns the code byte (INT8 two's
 * complement, E2M1 sign<<3 | index, E4M3 sign<<7 | index) and writes the
 * dequantised value fl32(s * val(q)) with the element's sign. */
static int enc_elem(int fmt, float s, float w, float *wq)
{
    int n;
    const double *T = elem_table(fmt, &n);
    int neg = signbit(w) != 0;
    float a = fabsf(w);
    int idx = 0;
    if (s != 0.0f) {
        float x = a / s; /* fl32 IEEE division (may overflow to +inf: saturates) */
        idx = orc_rne_index(T, n, (double)x);
    }
    float mag = s * (float)T[idx]; /* fl32 */
    *wq = neg ? -mag : mag;
    switch (elem_kind(fmt)) {
    case E_INT8: return (uint8_t)(int8_t)(neg ? -idx : idx);
    case E_INT4: return (neg ? -idx : idx) & 0xF; /* two's complement nibble */
    case E_E2M1: return (neg << 3) | idx;
    default: return (neg << 7) | idx;
    }
}

/* Decode one element code to (sign, index); -1 for an invalid code. */
static int dec_elem(int fmt, int code, int *neg)
{
    switch (elem_kind(fmt)) {
    case E_INT8: {
        int v = (int8_t)(uint8_t)code;
        if (v == -128) return -1;
        *neg = v < 0;
        return v < 0 ? -v : v;
    }
    case E_INT4: {
        int v = code & 0xF;
        if (v >= 8) v -= 16;
        if (v == -8) return -1;
        *neg = v < 0;
        return v < 0 ? -v : v;
    }
    case E_E2M1:
        *neg = (code >> 3) & 1;
        return code & 7;
    default:
        *neg = (code >> 7) & 1;
        if ((code & 0x7F) == 0x7F) return -1;
        return code & 0x7F;
    }
}

/* Objective of one block at scale s: sum_j om_j (w_j - wq_j)^2 in float64,
 * j ascending (om == NULL means every om_j = 1). */
static double block_objective(int fmt, float s, const float *w, const double *om, int B)
{
    double obj = 0.0;
    for (int j = 0; j < B; j++) {
        float wq;
        enc_elem(fmt, s, w[j], &wq);
        double d = (double)w[j] - (double)wq;
        obj += (om ? om[j] : 1.0) * (d * d);
    }
    return obj;
}

/* Binary16 code of v >= 0: round to nearest, ties to the even code,
 * saturating at 65504 (the FP16 scale snap). */
int orc_f16_code(double v)
{
    init_tables();
    return orc_rne_index(T_F16, 31744, v);
}

/* FP16-scale alternation (qwantize "Results", "Larger blocks: bs=64 (E4M3
 * scales) and bs=128 (FP16 scales)").  For a fixed element assignment q the
 * objective sum_j om_j (w_j - s q_j)^2 is a quadratic in s with its minimum at
 * s* = sum_j om_j w_j q_j / sum_j om_j q_j^2 (least squares); the page
 * alternates between q (encode at the current scale) and s (s* snapped to
 * FP16).  Readings: the walk starts at the Naive scale; it stops at a fixed
 * point (the snapped s* is the current scale), when every om_j q_j^2 is 0 (s*
 * undefined), at the zero scale, or after F16_ALT_MAX_ROUNDS rounds; the scale
 * returned is the iterate with the smallest objective, the earliest on ties,
 * so the result is never worse than Naive.  Sums in float64, j ascending; each
 * product om_j * w_j * q_j is exact in float64 (24 + 24 + 3 bits). */
static int f16_alternation(int fmt, const float *w, const double *om, int B, float amax, double *best_out)
{
    int n_t;
    const double *T = elem_table(fmt, &n_t);
    int code = orc_naive_scale_code(fmt, amax);
    int best_code = code;
    double best = block_objective(fmt, (float)T_F16[code], w, om, B);
    for (int round = 0; round < F16_ALT_MAX_ROUNDS && code != 0; round++) {
        float s = (float)T_F16[code];
        double num = 0.0, den = 0.0;
        for (int j = 0; j < B; j++) {
            float wq;
            int neg = 0;
            int idx = dec_elem(fmt, enc_elem(fmt, s, w[j], &wq), &neg);
            double q = neg ? -T[idx] : T[idx];
            double o = om ? om[j] : 1.0;
            num += o * (double)w[j] * q;
            den += o * q * q;
        }
        if (den == 0.0)
            break;
        int next = orc_rne_index(T_F16, 31744, num / den);
        if (next == code)
            break;
        code = next;
        double obj = block_objective(fmt, (float)T_F16[code], w, om, B);
        if (obj < best) {
            best = obj;
            best_code = code;
        }
    }
    *best_out = best;
    return best_code;
}

static float widen(const void *p, int dt, int64_t i)
{
    if (dt == DT_F32)
        return ((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int orc_max_threads(void) { return set_threads(0); }

/* Every candidate's objective for one block (for brute-force checks).
 * obj_out / code_out hold orc_candidates() entries. */
int orc_block_all_objectives(int fmt, int B, const float *w, const float *h, double *obj_out,
                             int32_t *code_out)
{
    init_tables();
    int c0, c1;
    if (orc_candidates(fmt, &c0, &c1) < 0 || B <= 0)
        return ORC_EINVAL;
    double *om = NULL;
    if (h) {
        om = (double *)malloc(sizeof(double) * (size_t)B);
        if (!om) return ORC_ENOMEM;
        for (int j = 0; j < B; j++) om[j] = (double)h[j];
    }
    for (int c = c0; c <= c1; c++) {
        obj_out[c - c0] = block_objective(fmt, orc_scale_value(fmt, c), w, om, B);
        code_out[c - c0] = c;
    }
    free(om);
    return c1 - c0 + 1;
}

static int check_common(int fmt, int B, int64_t N, int64_t K)
{
    if (fmt < 0 || fmt >= F_COUNT || B <= 0 || N < 0 || K < 0 || (K > 0 && K % B != 0))
        return ORC_EINVAL;
    if (four_bit(fmt) && (K % 2) != 0)
        return ORC_EINVAL;
    return ORC_OK;
}

static void put_code(int fmt, uint8_t *codes, int64_t N, int64_t K, int64_t n, int64_t k, int code)
{
    (void)N;
    if (four_bit(fmt)) {
        uint8_t *p = codes + n * (K / 2) + k / 2;
        if (k % 2 == 0)
            *p = (uint8_t)((*p & 0xF0) | (code & 0xF));
        else
            *p = (uint8_t)((*p & 0x0F) | ((code & 0xF) << 4));
    } else {
        codes[n * K + k] = (uint8_t)code;
    }
}

static int get_code(int fmt, const uint8_t *codes, int64_t K, int64_t n, int64_t k)
{
    if (four_bit(fmt)) {
        uint8_t b = codes[n * (K / 2) + k / 2];
        return (k % 2 == 0) ? (b & 0xF) : (b >> 4);
    }
    return codes[n * K + k];
}

/* The scale code a method picks for one block w[0..B-1] with max |w| = amax,
 * and its objective (weighted by om, or unweighted if om == NULL): Naive or
 * the OCP rule; the exact argmin over the scale grid in ascending code order
 * (the first strict minimum); or, for FP16 scales, the alternation. */
static int choose_scale(int method, int fmt, const float *w, const double *om, int B, float amax, double *best)
{
    if (method == M_NAIVE || method == M_NAIVE_OCP) {
        int code = method == M_NAIVE ? orc_naive_scale_code(fmt, amax) : orc_naive_ocp_code(fmt, amax);
        *best = block_objective(fmt, orc_scale_value(fmt, code), w, om, B);
        return code;
    }
    if (scale_kind(fmt) == S_F16)
        return f16_alternation(fmt, w, om, B, amax, best);
    int c0, c1;
    orc_candidates(fmt, &c0, &c1);
    int code = c0;
    double b0 = block_objective(fmt, orc_scale_value(fmt, c0), w, om, B);
    for (int c = c0 + 1; c <= c1; c++) {
        double o = block_objective(fmt, orc_scale_value(fmt, c), w, om, B);
        if (o < b0) {
            b0 = o;
            code = c;
        }
    }
    *best = b0;
    return code;
}

/* quantize_blocks.  method: Naive / SSE-Optimal / H-Optimal (the exact argmin
 * over the scale grid; for FP16 scales the alternation above).  scales_in, when
 * not NULL, fixes every block's scale code (encode only: method is ignored).
 * h is required for H-Optimal; for Naive and for a fixed scale it only weights
 * the reported objective.  codes: [N][K] bytes (INT8, E4M3) or [N][K/2]
 * (E2M1, INT4: element 2k in the low nibble); scales: [N][K/B] codes, one byte
 * each, or two (little-endian binary16 bits) for FP16 scales; block_obj:
 * [N][K/B] float64 or NULL. */
int orc_quantize(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                 const float *h, const uint8_t *scales_in, uint8_t *codes, uint8_t *scales,
                 double *block_obj, int nthreads)
{
    init_tables();
    if (check_common(fmt, B, N, K) != ORC_OK || (wdt != DT_F32 && wdt != DT_BF16))
        return ORC_EINVAL;
    if (!scales_in && method == M_H && !h)
        return ORC_EINVAL;
    if (!scales_in && (method < M_NAIVE || method > M_NAIVE_OCP))
        return ORC_EINVAL;
    if (!scales_in && method == M_NAIVE_OCP && scale_kind(fmt) != S_E8M0)
        return ORC_EINVAL;
    if (N == 0 || K == 0)
        return ORC_OK;
    const int64_t nb = K / B;
    int use_h = h != NULL && (scales_in != NULL || method != M_SSE);
    double *om_all = NULL;
    if (use_h) {
        om_all = (double *)malloc(sizeof(double) * (size_t)K);
        if (!om_all) return ORC_ENOMEM;
        for (int64_t k = 0; k < K; k++) om_all[k] = (double)h[k];
    }
    int err = ORC_OK;
    int nt = set_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)B);
        if (!w) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; n++) {
            if (!w) continue;
            for (int64_t b = 0; b < nb; b++) {
                const double *om = use_h ? om_all + b * B : NULL;
                float amax = 0.0f;
                for (int j = 0; j < B; j++) {
                    w[j] = widen(W, wdt, n * K + b * B + j);
                    float a = fabsf(w[j]);
                    if (a > amax) amax = a;
                }
                int code;
                double best;
                if (scales_in) {
                    code = get_scale(fmt, scales_in, n * nb + b);
                    float s = orc_scale_value(fmt, code);
                    if (isnan(s)) {
#pragma omp atomic write
                        err = ORC_EINVAL;
                        continue;
                    }
                    best = block_objective(fmt, s, w, om, B);
                } else {
                    code = choose_scale(method, fmt, w, om, B, amax, &best);
                }
                float s = orc_scale_value(fmt, code);
                if (scales) put_scale(fmt, scales, n * nb + b, code);
                if (block_obj) block_obj[n * nb + b] = best;
                if (codes) {
                    for (int j = 0; j < B; j++) {
                        float wq;
                        int cb = enc_elem(fmt, s, w[j], &wq);
                        put_code(fmt, codes, N, K, n, b * B + j, cb);
                    }
                }
            }
        }
        free(w);
    }
    free(om_all);
    return err;
}

/* dequantize: Wq[n][k] = sign * fl32(s_block * val(index)) as float32. */
int orc_dequantize(int fmt, int B, const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                   float *out, int nthreads)
{
    init_tables();
    if (check_common(fmt, B, N, K) != ORC_OK)
        return ORC_EINVAL;
    int n_t;
    const double *T = elem_table(fmt, &n_t);
    const int64_t nb = K / B;
    int err = ORC_OK;
    int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            float s = orc_scale_value(fmt, get_scale(fmt, scales, n * nb + k / B));
            int neg = 0;
            int idx = dec_elem(fmt, get_code(fmt, codes, K, n, k), &neg);
            if (isnan(s) || idx < 0) {
#pragma omp atomic write
                err = ORC_EINVAL;
                continue;
            }
            float mag = s * (float)T[idx];
            out[n * K + k] = neg ? -mag : mag;
        }
    }
    return err;
}

/* Per-block objective of W at the given scale codes (om = h, or 1 if NULL). */
int orc_objectives_at(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                      const uint8_t *scales_in, double *obj_out, int nthreads)
{
    return orc_quantize(M_NAIVE, fmt, B, W, wdt, N, K, h, scales_in, NULL, NULL, obj_out, nthreads);
}

/* hdiag: h_j = sum_t x_tj^2, summed in float64 in row order, stored as fp32. */
int orc_hdiag(const void *X, int xdt, int64_t M, int64_t K, float *h, int nthreads)
{
    if (M < 0 || K < 0 || (xdt != DT_F32 && xdt != DT_BF16))
        return ORC_EINVAL;
    double *acc = (double *)calloc((size_t)(K ? K : 1), sizeof(double));
    if (!acc) return ORC_ENOMEM;
    int nt = set_threads(nthreads);
    const int64_t chunk = 64;
    const int64_t nchunks = (K + chunk - 1) / chunk;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t c = 0; c < nchunks; c++) {
        int64_t j0 = c * chunk, j1 = j0 + chunk < K ? j0 + chunk : K;
        for (int64_t t = 0; t < M; t++)
            for (int64_t j = j0; j < j1; j++) {
                double x = (double)widen(X, xdt, t * K + j);
                acc[j] += x * x;
            }
    }
    for (int64_t j = 0; j < K; j++)
        h[j] = (float)acc[j];
    free(acc);
    return ORC_OK;
}

/* Weight error ||Wq - W||_F / ||W||_F in float64 (row partials summed in row
 * order).  Also returns the two sums of squares when the pointers are set. */
double orc_weight_error(const void *W, int wdt, const void *Wq, int qdt, int64_t N, int64_t K,
                        double *num_out, double *den_out, int nthreads)
{
    double *rn = (double *)calloc((size_t)(N ? N : 1), sizeof(double));
    double *rd = (double *)calloc((size_t)(N ? N : 1), sizeof(double));
    if (!rn || !rd) {
        free(rn);
        free(rd);
        return NAN;
    }
    int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double a = 0.0, b = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double w = (double)widen(W, wdt, n * K + k);
            double q = (double)widen(Wq, qdt, n * K + k);
            a += (q - w) * (q - w);
            b += w * w;
        }
        rn[n] = a;
        rd[n] = b;
    }
    double num = 0.0, den = 0.0;
    for (int64_t n = 0; n < N; n++) {
        num += rn[n];
        den += rd[n];
    }
    free(rn);
    free(rd);
    if (num_out) *num_out = num;
    if (den_out) *den_out = den;
    return sqrt(num) / sqrt(den);
}

/* Output error ||X Wq^T - X W^T||_F / ||X W^T||_F in float64:
 * Y = X W^T and D = X (Wq - W)^T from the exact inputs, every dot product
 * summed in k order, squares summed per row of X and then in row order. */
double orc_output_error(const void *X, int xdt, int64_t M, const void *W, int wdt, const void *Wq,
                        int qdt, int64_t N, int64_t K, double *dsq_out, double *ysq_out, int nthreads)
{
    const size_t nk = (size_t)(N * K) + 1;
    double *Wd = (double *)malloc(sizeof(double) * nk);
    double *Dd = (double *)malloc(sizeof(double) * nk);
    double *rd = (double *)calloc((size_t)(M ? M : 1), sizeof(double));
    double *ry = (double *)calloc((size_t)(M ? M : 1), sizeof(double));
    if (!Wd || !Dd || !rd || !ry) {
        free(Wd); free(Dd); free(rd); free(ry);
        return NAN;
    }
    for (int64_t i = 0; i < N * K; i++) {
        double w = (double)widen(W, wdt, i);
        Wd[i] = w;
        Dd[i] = (double)widen(Wq, qdt, i) - w;
    }
    int nt = set_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(K ? K : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < M; t++) {
            if (!x) continue;
            for (int64_t k = 0; k < K; k++)
                x[k] = (double)widen(X, xdt, t * K + k);
            double sd = 0.0, sy = 0.0;
            for (int64_t n = 0; n < N; n++) {
                const double *wr = Wd + n * K, *dr = Dd + n * K;
                double y = 0.0, d = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    y += x[k] * wr[k];
                    d += x[k] * dr[k];
                }
                sy += y * y;
                sd += d * d;
            }
            rd[t] = sd;
            ry[t] = sy;
        }
        free(x);
    }
    double dsq = 0.0, ysq = 0.0;
    for (int64_t t = 0; t < M; t++) {
        dsq += rd[t];
        ysq += ry[t];
    }
    free(Wd); free(Dd); free(rd); free(ry);
    if (dsq_out) *dsq_out = dsq;
    if (ysq_out) *ysq_out = ysq;
    return sqrt(dsq) / sqrt(ysq);
}

/* Y = X W^T in float64 from the exact inputs, each entry summed in k order
 * (the product behind the output error's reference term ||X W^T||). */
void orc_matmul_nt(const void *X, int xdt, int64_t M, const void *W, int wdt, int64_t N, int64_t K, double *Y,
                   int nthreads)
{
    int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t t = 0; t < M; t++) {
        for (int64_t n = 0; n < N; n++) {
            double y = 0.0;
            for (int64_t k = 0; k < K; k++)
                y += (double)widen(X, xdt, t * K + k) * (double)widen(W, wdt, n * K + k);
            Y[t * N + n] = y;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* GPTQ                                                                      */
/* ------------------------------------------------------------------------ */

/* H = X^T X, K x K row-major in float64: H[i][j] = sum_t x_ti x_tj, t in
 * order (products of bf16 / fp32 values are exact in float64). */
int orc_xtx(const void *X, int xdt, int64_t M, int64_t K, double *H, int nthreads)
{
    if (M < 0 || K < 0 || (xdt != DT_F32 && xdt != DT_BF16))
        return ORC_EINVAL;
    int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t i = 0; i < K; i++) {
        for (int64_t j = 0; j <= i; j++) {
            double acc = 0.0;
            for (int64_t t = 0; t < M; t++)
                acc += (double)widen(X, xdt, t * K + i) * (double)widen(X, xdt, t * K + j);
            H[i * K + j] = acc;
            H[j * K + i] = acc;
        }
    }
    return ORC_OK;
}

/* Lower Cholesky factor of the symmetric positive definite A (n x n), in
 * place of L (may alias nothing); returns ORC_EINVAL if A is not positive
 * definite in float64. */
static int cholesky_lower(const double *A, double *L, int64_t n)
{
    memset(L, 0, sizeof(double) * (size_t)(n * n));
    for (int64_t j = 0; j < n; j++) {
        double d = A[j * n + j];
        for (int64_t k = 0; k < j; k++)
            d -= L[j * n + k] * L[j * n + k];
        if (!(d > 0.0))
            return ORC_EINVAL;
        const double ljj = sqrt(d);
        L[j * n + j] = ljj;
        for (int64_t i = j + 1; i < n; i++) {
            double v = A[i * n + j];
            for (int64_t k = 0; k < j; k++)
                v -= L[i * n + k] * L[j * n + k];
            L[i * n + j] = v / ljj;
        }
    }
    return ORC_OK;
}

/* U with H^-1 = U^T U, U upper triangular with positive diagonal, for the
 * symmetric positive definite H (n x n): the sequence GPTQ (Frantar et al.)
 * uses - L = chol(H), H^-1 = L^-T L^-1, then the Cholesky factor of H^-1. */
static int inverse_upper_factor(const double *H, double *U, int64_t n)
{
    double *L = (double *)malloc(sizeof(double) * (size_t)(n * n));
    double *Li = (double *)calloc((size_t)(n * n), sizeof(double));
    double *Hi = (double *)malloc(sizeof(double) * (size_t)(n * n));
    int rc = (L && Li && Hi) ? ORC_OK : ORC_ENOMEM;
    if (rc == ORC_OK)
        rc = cholesky_lower(H, L, n);
    if (rc == ORC_OK) {
        /* L^-1 column by column: forward substitution on the unit vectors */
        for (int64_t c = 0; c < n; c++) {
            for (int64_t i = c; i < n; i++) {
                double v = (i == c) ? 1.0 : 0.0;
                for (int64_t k = c; k < i; k++)
                    v -= L[i * n + k] * Li[k * n + c];
                Li[i * n + c] = v / L[i * n + i];
            }
        }
        /* H^-1 = L^-T L^-1: (i, j) = sum_k Li[k][i] Li[k][j], k >= max(i, j) */
        for (int64_t i = 0; i < n; i++) {
            for (int64_t j = 0; j <= i; j++) {
                double v = 0.0;
                for (int64_t k = i; k < n; k++)
                    v += Li[k * n + i] * Li[k * n + j];
                Hi[i * n + j] = v;
                Hi[j * n + i] = v;
            }
        }
        rc = cholesky_lower(Hi, L, n); /* H^-1 = L2 L2^T, U = L2^T */
        if (rc == ORC_OK)
            for (int64_t i = 0; i < n; i++)
                for (int64_t j = 0; j < n; j++)
                    U[i * n + j] = (j >= i) ? L[j * n + i] : 0.0;
    }
    free(L);
    free(Li);
    free(Hi);
    return rc;
}

/* GPTQ on top of a scale choice (qwantize "Results", "GPTQ Quantization": GPTQ
 * of Frantar et al. with its block size equal to the quantisation block size;
 * the quantisation-algorithms note, §1: H = X^T X + lambda I, columns quantised
 * in sequence, each residual propagated through H^-1).
 *
 *   H       : X^T X, K x K (orc_xtx); h_j = fl32(H_jj) weights H-Optimal, as
 *             hdiag would give it.
 *   damping : lambda = damp * mean_j H_jj (1 if that mean is 0), H + lambda I.
 *   order   : ordered == 0 (GPTQ-Seq): block columns left to right.
 *             ordered != 0 (GPTQ-Ord): block columns by descending
 *             Hessian-weighted loss sum_n sum_{j in b} h_j (w_nj - q_nj)^2 of
 *             the method's quantisation of W without GPTQ, ties in column
 *             order; W's and H's columns are permuted by whole blocks.
 *   loop    : U = the upper Cholesky factor of (H + lambda I)^-1 in the
 *             processing order.  For each block column in order, every row's
 *             scale is chosen by `method` from that row's current (already
 *             compensated) block, rounded to fp32 as the quantiser's input;
 *             then the block's columns j are encoded one by one at that scale
 *             and the error e = (w_j - q_j) / U_jj is propagated to every
 *             later column k: w_k -= e U_jk.  Working weights are float64.
 * Outputs codes / scales in the original column order; block_order[i] is the
 * original index of the i-th block column processed (may be NULL). */
/* Precision experiment (test infrastructure, not a reference): GPTQ as
 * orc_gptq, with selected quantities carried in float32 or perturbed, to
 * measure how far the column loop's decisions move under rounding alone.
 *   GPTQ_EMUL_H32  : H rounded to float32 (an H formed in float32);
 *   GPTQ_EMUL_U32  : the factor U rounded to float32;
 *   GPTQ_EMUL_W32  : working weights stored in float32 after every update,
 *                    the propagated error e and each product e U_ck in float32;
 *   GPTQ_EMUL_HULP : every off-diagonal H_ij with i + j odd moved by one
 *                    float64 ulp (a float64 computation in another order). */
enum { GPTQ_EMUL_H32 = 1, GPTQ_EMUL_U32 = 2, GPTQ_EMUL_W32 = 4, GPTQ_EMUL_HULP = 8 };
static int gptq_impl(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const double *H,
                     double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int nthreads,
                     int emul);

int orc_gptq(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const double *H,
             double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int nthreads)
{
    return gptq_impl(method, fmt, B, W, wdt, N, K, H, damp, ordered, codes, scales, block_order, nthreads, 0);
}

int orc_gptq_emulated(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const double *H,
                      double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int nthreads,
                      int emul)
{
    return gptq_impl(method, fmt, B, W, wdt, N, K, H, damp, ordered, codes, scales, block_order, nthreads, emul);
}

static int gptq_impl(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const double *H,
                     double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int nthreads,
                     int emul)
{
    init_tables();
    if (check_common(fmt, B, N, K) != ORC_OK || (wdt != DT_F32 && wdt != DT_BF16) || !H || damp < 0.0 || B > 256)
        return ORC_EINVAL;
    if (method < M_NAIVE || method > M_NAIVE_OCP || (method == M_NAIVE_OCP && scale_kind(fmt) != S_E8M0))
        return ORC_EINVAL;
    if (N == 0 || K == 0)
        return ORC_OK;
    const int64_t nb = K / B;
    int nt = set_threads(nthreads);
    int rc = ORC_OK;
    float *h = (float *)malloc(sizeof(float) * (size_t)K);
    int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)nb); /* processing slot -> block */
    int64_t *col = (int64_t *)malloc(sizeof(int64_t) * (size_t)K);   /* processed column -> original */
    double *Hp = (double *)malloc(sizeof(double) * (size_t)(K * K));
    double *U = (double *)malloc(sizeof(double) * (size_t)(K * K));
    double *Wc = (double *)malloc(sizeof(double) * (size_t)(N * K));
    double *om = (double *)malloc(sizeof(double) * (size_t)K);
    if (!h || !perm || !col || !Hp || !U || !Wc || !om) {
        rc = ORC_ENOMEM;
        goto done;
    }
    double mean = 0.0;
    for (int64_t j = 0; j < K; j++) {
        h[j] = (float)H[j * K + j];
        mean += H[j * K + j];
    }
    mean /= (double)K;
    const double lambda = mean > 0.0 ? damp * mean : 1.0;

    for (int64_t b = 0; b < nb; b++)
        perm[b] = b;
    if (ordered) {
        /* Hessian-weighted loss of each block column without GPTQ */
        double *loss = (double *)calloc((size_t)nb, sizeof(double));
        double *bo = (double *)malloc(sizeof(double) * (size_t)(N * nb));
        if (!loss || !bo) {
            free(loss);
            free(bo);
            rc = ORC_ENOMEM;
            goto done;
        }
        uint8_t *sc = (uint8_t *)malloc((size_t)(N * nb) * (size_t)scale_bytes(fmt));
        rc = sc ? orc_quantize(method, fmt, B, W, wdt, N, K, h, NULL, NULL, sc, NULL, nthreads) : ORC_ENOMEM;
        if (rc == ORC_OK)
            rc = orc_quantize(M_NAIVE, fmt, B, W, wdt, N, K, h, sc, NULL, NULL, bo, nthreads);
        if (rc == ORC_OK) {
            for (int64_t n = 0; n < N; n++)
                for (int64_t b = 0; b < nb; b++)
                    loss[b] += bo[n * nb + b];
            /* stable insertion sort by descending loss */
            for (int64_t i = 1; i < nb; i++) {
                int64_t v = perm[i], k = i;
                while (k > 0 && loss[perm[k - 1]] < loss[v]) {
                    perm[k] = perm[k - 1];
                    k--;
                }
                perm[k] = v;
            }
        }
        free(sc);
        free(loss);
        free(bo);
        if (rc != ORC_OK)
            goto done;
    }
    for (int64_t i = 0; i < nb; i++)
        for (int j = 0; j < B; j++)
            col[i * B + j] = perm[i] * B + j;
    if (block_order)
        for (int64_t i = 0; i < nb; i++)
            block_order[i] = (int32_t)perm[i];
    for (int64_t i = 0; i < K; i++) {
        for (int64_t j = 0; j < K; j++) {
            double v = H[col[i] * K + col[j]];
            if (emul & GPTQ_EMUL_H32)
                v = (double)(float)v;
            if ((emul & GPTQ_EMUL_HULP) && col[i] != col[j] && ((col[i] + col[j]) & 1))
                v = nextafter(v, v > 0.0 ? INFINITY : -INFINITY);
            Hp[i * K + j] = v;
        }
        Hp[i * K + i] += lambda;
        om[i] = (double)h[col[i]];
    }
    rc = inverse_upper_factor(Hp, U, K);
    if (rc != ORC_OK)
        goto done;
    if (emul & GPTQ_EMUL_U32)
        for (int64_t i = 0; i < K * K; i++)
            U[i] = (double)(float)U[i];
    for (int64_t n = 0; n < N; n++)
        for (int64_t i = 0; i < K; i++)
            Wc[n * K + i] = (double)widen(W, wdt, n * K + col[i]);

#pragma omp parallel num_threads(nt)
    {
        float w[256];
        const double *omw;
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; n++) {
            double *wr = Wc + n * K;
            for (int64_t i = 0; i < nb; i++) {
                const int64_t cs = i * B;
                float amax = 0.0f;
                for (int j = 0; j < B; j++) {
                    w[j] = (float)wr[cs + j];
                    if (fabsf(w[j]) > amax) amax = fabsf(w[j]);
                }
                omw = (method == M_SSE) ? NULL : om + cs;
                double obj;
                const int code = choose_scale(method, fmt, w, omw, B, amax, &obj);
                const float s = orc_scale_value(fmt, code);
                put_scale(fmt, scales, n * nb + perm[i], code);
                for (int j = 0; j < B; j++) {
                    const int64_t c = cs + j;
                    float wq;
                    const int cb = enc_elem(fmt, s, (float)wr[c], &wq);
                    put_code(fmt, codes, N, K, n, col[c], cb);
                    const double e = (wr[c] - (double)wq) / U[c * K + c];
                    if (emul & GPTQ_EMUL_W32) {
                        const float ef = (float)e;
                        for (int64_t k = c + 1; k < K; k++)
                            wr[k] = (double)((float)wr[k] - ef * (float)U[c * K + k]);
                    } else {
                        for (int64_t k = c + 1; k < K; k++)
                            wr[k] -= e * U[c * K + k];
                    }
                }
            }
        }
    }
done:
    free(h);
    free(perm);
    free(col);
    free(Hp);
    free(U);
    free(Wc);
    free(om);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Per-tensor scaling on top of E4M3 block scales                            */
/* ------------------------------------------------------------------------ */

/* "Is Finer Better?" §5.1 / Table 1 (UE4M3-S: per-tensor scaling + UE4M3
 * block scales; the page's formula for the tensor scale is not legible in
 * our copy).  Reading: s_T = fl32(amax_T / (C_T * 448)) maps the tensor's
 * largest block scale onto the top of the E4M3 grid (C_T = the element
 * maximum, or 1 for INT8, whose block scale is amax itself); 1 when the tensor
 * is all zero.  The blocks then quantise W' = fl32(W / s_T) exactly as the
 * format does, and x^ = fl32(s_T * fl32(s q)).  E4M3-scale formats only. */
float orc_tensor_scale(int fmt, const void *W, int wdt, int64_t n)
{
    init_tables();
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        const float a = fabsf(widen(W, wdt, i));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f)
        return 1.0f;
    const float ct = (scale_kind(fmt) == S_E4M3_OF_AMAX_DIV127) ? 1.0f : elem_cmax(fmt);
    return amax / (ct * 448.0f); /* ct * 448 is exact */
}

int orc_quantize_tensor_scaled(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                               const float *h, uint8_t *codes, uint8_t *scales, float *tensor_scale,
                               double *block_obj, int nthreads)
{
    init_tables();
    if (fmt < 0 || fmt >= F_COUNT || (scale_kind(fmt) != S_E4M3 && scale_kind(fmt) != S_E4M3_OF_AMAX_DIV127))
        return ORC_EINVAL;
    if (wdt != DT_F32 && wdt != DT_BF16)
        return ORC_EINVAL;
    const float st = orc_tensor_scale(fmt, W, wdt, N * K);
    float *Wp = (float *)malloc(sizeof(float) * (size_t)(N * K > 0 ? N * K : 1));
    if (!Wp)
        return ORC_ENOMEM;
    for (int64_t i = 0; i < N * K; i++)
        Wp[i] = widen(W, wdt, i) / st; /* fl32 IEEE division */
    const int rc = orc_quantize(method, fmt, B, Wp, DT_F32, N, K, h, NULL, codes, scales, block_obj, nthreads);
    free(Wp);
    if (tensor_scale)
        *tensor_scale = st;
    return rc;
}

int orc_dequantize_tensor_scaled(int fmt, int B, const uint8_t *codes, const uint8_t *scales, float tensor_scale,
                                 int64_t N, int64_t K, float *out, int nthreads)
{
    const int rc = orc_dequantize(fmt, B, codes, scales, N, K, out, nthreads);
    if (rc == ORC_OK)
        for (int64_t i = 0; i < N * K; i++)
            out[i] = tensor_scale * out[i]; /* fl32 */
    return rc;
}
