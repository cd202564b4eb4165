// formats.hpp - number formats, scale grids and exact rounding for the gfx950
// kernels of libhdiag.so.
//
// Element formats: INT8 [-127, 127]; INT4 [-7, 7] (the NVINT4 rows of the
// qwantize "Results" tables, read as symmetric INT4); E2M1
// {0,.5,1,1.5,2,3,4,6} (qwantize "Results", Exotic Scales); OCP E4M3 (126
// positive finite codes, max 448; 0x7F/0xFF NaN).  Scale grids: E4M3 codes
// 0x01..0x7E; INT8's fl32(E4M3 / 127) (qwantize "Results", INT8 section); E8M0
// 2^(c-127), c = 0..254 ("Is Finer Better?" §2.1); the unsigned UE4M4 (bias 7)
// and UE5M3 (bias 15) grids of the "Exotic Scales" section, every code finite
// (0x01..0xFF positive); binary16 (FP16 E5M10, 0x0000..0x7BFF) block scales
// found by alternation (qwantize "Results", "Larger blocks: bs=64 (E4M3 scales)
// and bs=128 (FP16 scales)").  Values follow the EeMm formula of the LLM-FP4
// summary page ("Floating-Point Quantization Mechanics").
//
// Rounding: q = RNE(fl32(|w| / s)) onto the element grid, ties to the even
// code, saturating.  Every helper here is exact in IEEE binary32 with
// round-to-nearest-even and preserved denormals (the HIP default on gfx950);
// the library is built with -ffp-contract=off so no expression is fused behind
// our back.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "hdiag.h"

namespace hd {

enum ElemKind { ELEM_INT8 = 0, ELEM_E2M1 = 1, ELEM_E4M3 = 2, ELEM_INT4 = 3 };
enum ScaleKind { SCALE_INT8 = 0, SCALE_E4M3 = 1, SCALE_E8M0 = 2, SCALE_UE4M4 = 3, SCALE_UE5M3 = 4, SCALE_F16 = 5 };

__host__ __device__ constexpr int elem_kind(int fmt)
{
    return fmt == HD_INT8_E4M3 ? ELEM_INT8
         : (fmt == HD_NVINT4 || fmt == HD_INT4_F16) ? ELEM_INT4
         : (fmt == HD_NVFP4 || fmt == HD_MXFP4 || fmt == HD_NVFP4_UE4M4 || fmt == HD_NVFP4_UE5M3 ||
            fmt == HD_FP4_F16)
             ? ELEM_E2M1
             : ELEM_E4M3;
}
__host__ __device__ constexpr int scale_kind(int fmt)
{
    return fmt == HD_INT8_E4M3 ? SCALE_INT8
         : (fmt == HD_NVFP4 || fmt == HD_FP8_E4M3S || fmt == HD_NVINT4) ? SCALE_E4M3
         : fmt == HD_NVFP4_UE4M4 ? SCALE_UE4M4
         : fmt == HD_NVFP4_UE5M3 ? SCALE_UE5M3
         : (fmt == HD_FP4_F16 || fmt == HD_INT4_F16) ? SCALE_F16
                                 : SCALE_E8M0;
}
// Bytes of one stored scale code: binary16 bits for FP16 scales, else a byte.
__host__ __device__ constexpr int scale_bytes(int sk) { return sk == SCALE_F16 ? 2 : 1; }
// Integer element grids (exact arithmetic encode) and 4-bit element codes.
__host__ __device__ constexpr bool elem_int(int ek) { return ek == ELEM_INT8 || ek == ELEM_INT4; }
__host__ __device__ constexpr bool elem_4bit(int ek) { return ek == ELEM_E2M1 || ek == ELEM_INT4; }
// Unsigned every-code-finite scale grids.
__host__ __device__ constexpr bool scale_unsigned(int sk) { return sk == SCALE_UE4M4 || sk == SCALE_UE5M3; }
// First / last search candidate code of a scale grid.
__host__ __device__ constexpr int cand_first(int sk) { return sk == SCALE_E8M0 ? 0 : 1; }
__host__ __device__ constexpr int cand_last(int sk)
{
    return sk == SCALE_E8M0 ? 254 : scale_unsigned(sk) ? 255 : sk == SCALE_F16 ? 0x7BFF : 126;
}
// Scale codes that stand for a number (the rest are NaN / Inf codes, or
// negative binary16 values).
__host__ __device__ constexpr bool scale_code_valid(int sk, int c)
{
    return c >= 0 && c <= cand_last(sk);
}
// Scale codes per binade of the grid (8 for E4M3 / UE5M3 / INT8, 16 for
// UE4M4, 1 for E8M0).
__host__ __device__ constexpr int codes_per_binade(int sk)
{
    return sk == SCALE_E8M0 ? 1 : sk == SCALE_UE4M4 ? 16 : sk == SCALE_F16 ? 1024 : 8;
}
// Largest element magnitude (the C of s = Q_scale(amax / C)).
__host__ __device__ constexpr float elem_max(int ek)
{
    return ek == ELEM_INT8 ? 127.0f : ek == ELEM_INT4 ? 7.0f : ek == ELEM_E2M1 ? 6.0f : 448.0f;
}
// Smallest positive element value.
__host__ __device__ constexpr float elem_min_pos(int ek)
{
    return ek == ELEM_E2M1 ? 0.5f : ek == ELEM_E4M3 ? 0x1p-9f : 1.0f;
}

__host__ __device__ inline float bits_f(uint32_t u)
{
    union { uint32_t u; float f; } v;
    v.u = u;
    return v.f;
}
__host__ __device__ inline uint32_t f_bits(float f)
{
    union { uint32_t u; float f; } v;
    v.f = f;
    return v.u;
}

// Magnitude of the E4M3 code c in 0..126 (exact in fp32): exponent field
// e = c >> 3 and mantissa m = c & 7 give (8 + m) 2^(e - 10), or m 2^-9 when
// e = 0 (subnormal).  Both cases are m' * 2^-9 * 2^(max(e,1) - 1) with
// m' = m + 8 [e > 0], built here from bits.
__host__ __device__ inline float e4m3_value(int c)
{
    const int e = c >> 3, m = c & 7;
    const float mant = (float)(e ? 8 + m : m);           // exact small integer
    const int pw = (e ? e : 1) - 10;                     // power of two of one mantissa step
    return mant * bits_f((uint32_t)(127 + pw) << 23);    // exact product
}

// 2^(c - 127) for c in 0..254; 2^-127 is the fp32 subnormal 0x00400000.
__host__ __device__ inline float e8m0_value(int c)
{
    return c == 0 ? bits_f(0x00400000u) : bits_f((uint32_t)c << 23);
}

// Magnitude of an unsigned UExMy code c (every code finite): exponent field
// e = c >> M, mantissa d = c & (2^M - 1); (2^M + d) 2^(e - bias - M), or
// d 2^(1 - bias - M) when e = 0.
template <int M, int BIAS>
__host__ __device__ inline float ue_value(int c)
{
    const int e = c >> M, d = c & ((1 << M) - 1);
    const float mant = (float)(e ? (1 << M) + d : d);
    const int pw = (e ? e : 1) - BIAS - M;
    return mant * bits_f((uint32_t)(127 + pw) << 23);  // 2^pw is normal for both grids
}

// The fp32 scale of scale code c on grid sk (c = 0 on an E4M3 grid is 0).
// Binary16 is the UExMy formula with M = 10, bias 15 (codes up to 0x7BFF).
__host__ __device__ inline float scale_value(int sk, int c)
{
    if (sk == SCALE_F16) return ue_value<10, 15>(c);
    if (sk == SCALE_E8M0) return e8m0_value(c);
    if (sk == SCALE_UE4M4) return ue_value<4, 7>(c);
    if (sk == SCALE_UE5M3) return ue_value<3, 15>(c);
    const float v = e4m3_value(c);
    return sk == SCALE_INT8 ? v / 127.0f : v;  // IEEE division (INT8 section)
}

// fl32(a / s) for s > 0, given r = fl32(1 / s) (any sign of a: every step is
// an odd function of a).
//  - E8M0 grids: s is a power of two, so a * r is the exactly rounded quotient.
//  - Otherwise: q0 = fl32(a r) is within two ulps of a/s; one correction
//    q1 = fl32(q0 + fl32(a - s q0) r) (Markstein's residual step, both FMAs)
//    lands within one ulp, and a second correction, now with an exact
//    residual, returns the correctly rounded quotient.  bfloat16 inputs need
//    only the first correction: checked exhaustively (every bf16 value against
//    every candidate scale) by the encode parity test, which runs this code.
//  - |a| is clamped to 2^100 first: any quotient that large saturates the
//    element grid for every E4M3-grid scale, and the FMAs stay finite.
//  - FP16 scales take both corrections whatever the input type (the one-step
//    check covered only the scale grids above).
template <int SK, bool ONE_STEP>
__device__ __forceinline__ float quotient(float a, float s, float r)
{
    if (SK == SCALE_E8M0) return a * r;
    a = __builtin_amdgcn_fmed3f(a, -0x1p100f, 0x1p100f);
    float q = a * r;
    float e = __builtin_fmaf(-q, s, a);
    q = __builtin_fmaf(e, r, q);
    if (!ONE_STEP || SK == SCALE_F16) {
        e = __builtin_fmaf(-q, s, a);
        q = __builtin_fmaf(e, r, q);
    }
    return q;
}

// fl32(a / m) for a scale mantissa m in [1, 2) with rm = fl32(1 / m): the
// corrections of quotient() without its clamp (dividing by m >= 1 keeps every
// FMA finite for finite a).  Elements this large saturate the grid either way.
template <bool ONE_STEP>
__device__ __forceinline__ float quotient_m(float a, float m, float rm)
{
    float q = a * rm;
    float e = __builtin_fmaf(-q, m, a);
    q = __builtin_fmaf(e, rm, q);
    if (!ONE_STEP) {
        e = __builtin_fmaf(-q, m, a);
        q = __builtin_fmaf(e, rm, q);
    }
    return q;
}

// Round x >= 0 onto the element grid, saturating; returns the grid VALUE.
// E2M1 / E4M3: add and subtract C = 2^(e + 23 - mbits) where e is the binade
// of x floored at the smallest normal; the add rounds x to a multiple of that
// binade's step with ties to even (the even multiple is the even code).
template <int EK>
__device__ __forceinline__ float round_elem(float x)
{
    if (EK == ELEM_INT8) return __builtin_rintf(fminf(x, 127.0f));
    if (EK == ELEM_INT4) return __builtin_rintf(fminf(x, 7.0f));
    if (EK == ELEM_E2M1) {
        const float xc = fminf(x, 6.0f);
        const float C = bits_f((f_bits(fmaxf(xc, 1.0f)) & 0x7F800000u) + (22u << 23));
        return (xc + C) - C;
    }
    const float xc = fminf(x, 448.0f);
    const float C = bits_f((f_bits(fmaxf(xc, 0x1p-6f)) & 0x7F800000u) + (20u << 23));
    return (xc + C) - C;
}

// Element code (magnitude index, no sign) of a grid value y.
template <int EK>
__device__ __forceinline__ uint32_t elem_index(float y)
{
    if (elem_int(EK)) return (uint32_t)y;
    if (EK == ELEM_E2M1) {
        // the top 10 bits of 1, 1.5, 2, 3, 4, 6 are 0xFE..0x103, i.e. the code
        // plus 0xFC; 0.5 (0xFC) and 0 need the floor of 1 / 0
        const int hi = (int)(f_bits(y) >> 22) - 0xFC;
        return (uint32_t)max(hi, y > 0.0f ? 1 : 0);
    }
    // subnormal codes 0..7 are y * 2^9; normal ones (e + 7) << 3 | mantissa
    const uint32_t u = f_bits(y);
    const uint32_t sub = (uint32_t)(y * 512.0f);
    const uint32_t nrm = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
    return y < 0x1p-6f ? sub : nrm;
}

// Grid value of a magnitude index.
template <int EK>
__device__ __forceinline__ float elem_value(uint32_t idx)
{
    if (elem_int(EK)) return (float)idx;
    if (EK == ELEM_E2M1) {
        // 0 .5 1 1.5 2 3 4 6: (2 + (idx & 1)) * 2^((idx >> 1) - 2), idx 1 is subnormal
        if (idx < 2) return idx ? 0.5f : 0.0f;
        return (float)(2 + (idx & 1)) * bits_f((uint32_t)(127 + (int)(idx >> 1) - 2) << 23);
    }
    return e4m3_value((int)idx);
}

// Full code byte (INT8 two's complement / E2M1 nibble / E4M3 byte) of a signed element.
template <int EK>
__device__ __forceinline__ uint32_t elem_code(uint32_t idx, bool neg)
{
    if (EK == ELEM_INT8) return (uint32_t)(uint8_t)(neg ? -(int)idx : (int)idx);
    if (EK == ELEM_INT4) return (uint32_t)(neg ? -(int)idx : (int)idx) & 15u;  // two's complement nibble
    if (EK == ELEM_E2M1) return idx | (neg ? 8u : 0u);
    return idx | (neg ? 0x80u : 0u);
}

// ---- gfx950 conversion instructions --------------------------------------
// v_cvt_scalef32_pk_fp4_f32 / _fp8_f32 divide two fp32 values by the power of
// two held in the exponent field of `p2` (the field 0 reads as 2^-127) and
// round to nearest-even onto E2M1 / OCP E4M3, keeping the sign; E2M1
// saturates at 6, E4M3 does not (values beyond 464 become NaN), so E4M3 inputs
// are clamped to 448 * p2 first.  The pk_f32 forms return the grid values.
// Checked against the oracle for every bf16 value at every candidate scale by
// the encode parity tests.
typedef float hd_v2f __attribute__((ext_vector_type(2)));
typedef short hd_v2s __attribute__((ext_vector_type(2)));

// two E2M1 codes (element a in bits 0..3, b in 4..7) of a / p2, b / p2
__device__ __forceinline__ uint32_t fp4x2(float a, float b, float p2)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, p2, 0) & 0xFFu;
}
// grid values of the two E2M1 codes in bits 0..7
__device__ __forceinline__ hd_v2f fp4x2_val(uint32_t byte) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0); }
// two E4M3 codes (a in bits 0..7, b in 8..15) of a / p2, b / p2; |a|, |b| <= 448 p2
__device__ __forceinline__ uint32_t fp8x2(float a, float b, float p2)
{
    const hd_v2s old = {0, 0};
    const hd_v2s c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, p2, false);
    return (uint32_t)(uint16_t)c.x | ((uint32_t)(uint16_t)c.y << 16);
}
__device__ __forceinline__ hd_v2f fp8x2_val(uint32_t half) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(half, 1.0f, false); }

// A positive E4M3 or E8M0 scale as m * p2 with m in [1, 2) one of the eight
// E4M3 mantissas (1 for E8M0) and p2 a power of two; rm = fl32(1 / m).
// fl32(a / s) = fl32(a / m) / p2 whenever the result is an fp32 normal, and
// below that every element rounds to code 0 either way, so the conversion
// instructions can take fl32(a / m) and p2.  s == 0 gives m = 1, p2 = 1.
struct ScaleParts {
    float s, m, rm, p2;
};
// TAB: rm comes from rm_tab[j] = fl32(1 / (1 + j / 16)), j = 0 .. 15 (an LDS
// table), in place of a division: for the grids whose mantissas have at most
// four bits (E4M3, UE4M4, UE5M3; not binary16).  Branch-free: s == 0 selects
// m = 1, rm = 1, p2 = 1.
template <int SK, bool TAB = false>
__device__ __forceinline__ ScaleParts scale_parts(float s, const float *rm_tab = nullptr)
{
    ScaleParts r;
    r.s = s;
    if (SK == SCALE_E8M0) {
        r.m = 1.0f;
        r.rm = 1.0f;
        r.p2 = s == 0.0f ? 1.0f : s;
        return r;
    }
    const bool z = s == 0.0f;
    int ex;
    const float f = __builtin_frexpf(s, &ex);  // s = f 2^ex, f in [0.5, 1)
    r.m = z ? 1.0f : 2.0f * f;
    if constexpr (TAB && SK != SCALE_F16)
        r.rm = rm_tab[(f_bits(r.m) >> 19) & 15u];
    else
        r.rm = 1.0f / r.m;
    r.p2 = z ? 1.0f : __builtin_ldexpf(1.0f, ex - 1);
    return r;
}

// Round v >= 0 onto an unsigned UExMy grid (saturating at its largest value)
// and return the code: the add-and-subtract-2^(e + 23 - M) rounding of
// round_elem with the grid's smallest normal exponent, then the code from the
// value's bits (subnormal codes are v / 2^(1 - bias - M)).
template <int M, int BIAS>
__device__ __forceinline__ int ue_round_code(float v)
{
    constexpr int EMIN = 1 - BIAS;  // exponent of the smallest normal
    const float vmax = ue_value<M, BIAS>(255);  // the largest code
    const float xc = fminf(v, vmax);
    const float C = bits_f((f_bits(fmaxf(xc, bits_f((uint32_t)(127 + EMIN) << 23))) & 0x7F800000u) +
                           ((uint32_t)(23 - M) << 23));
    const float y = (xc + C) - C;
    const uint32_t u = f_bits(y);
    const int sub = (int)(y * bits_f((uint32_t)(127 + BIAS - 1 + M) << 23));
    const int nrm = ((int)((u >> 23) & 0xFFu) - 127 + BIAS) << M | (int)((u >> (23 - M)) & ((1u << M) - 1));
    return y < bits_f((uint32_t)(127 + EMIN) << 23) ? sub : nrm;
}

// Binary16 code of v >= 0, rounded to nearest with ties to even and saturated
// at 65504 (0x7BFF).  With e = max(floor(log2 v), -14) one unit in the last
// place is 2^(e - 10), so m = rint(v / 2^(e - 10)) (exact scaling, then the
// hardware's round-to-nearest-even) is the significand as an integer, 1024 ..
// 2048 for normals and 0 .. 1024 below 2^-14, and the code is
// (e + 14) * 1024 + m in both cases (m = 2048 carries into the next binade).
__device__ __forceinline__ int f16_round_code(double v)
{
    if (!(v > 0x1p-25)) return 0;   // half the smallest subnormal ties to the even code 0
    if (v >= 65520.0) return 0x7BFF;  // rounds beyond 65504 (to Inf in IEEE): saturate
    int ex;
    __builtin_frexp(v, &ex);  // v = f 2^ex, f in [0.5, 1): floor(log2 v) = ex - 1
    const int e = max(ex - 1, -14);
    const double m = __builtin_rint(__builtin_ldexp(v, 10 - e));
    return (e + 14) * 1024 + (int)m;
}

// OCP MX rule for power-of-two scales: code of 2^(floor(log2 amax) - emax),
// emax the exponent of the largest element (E2M1 6 = 1.5 2^2, E4M3 448 =
// 1.75 2^8), clamped to E8M0's 2^[-127, 127]; amax = 0 gives code 0.
template <int EK>
__device__ __forceinline__ int ocp_code(float amax)
{
    if (amax == 0.0f) return 0;
    int ex;
    __builtin_frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    int E = ex - 1 - (EK == ELEM_E2M1 ? 2 : 8);
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
    return E + 127;
}

// Naive scale code of a block with max |w| = amax ("Is Finer Better?" §2.1,
// s = Q_scale(amax / C) with round-to-nearest scale quantisation; INT8 stores
// amax itself as E4M3).  E4M3 grids may return code 0 (the zero scale).
// E8M0: nearest power of two in the linear domain, ties upward, clamped to
// 2^[-127, 127].
// fl32(amax / C), C = the element grid's largest value (6, 7 or 448), for
// the non-power-of-two scale grids: two Markstein corrections of amax
// RN(1 / C).  Checked exhaustively against IEEE division for every positive
// float up to 2^100 (the quotient's clamp) and C = 6, 7, 448: they differ only
// where the quotient is an fp32 subnormal (below 2^-126), which every one of
// these grids (E4M3, UE4M4, UE5M3 and binary16, whose smallest values are
// 2^-9 .. 2^-24) snaps to code 0 either way.  INT8 needs no quotient (the
// scale is amax itself), and E8M0 keeps the division: its grid reaches 2^-127.
template <int EK>
__device__ __forceinline__ float div_elem_max(float amax)
{
    constexpr float C = EK == ELEM_E2M1 ? 6.0f : EK == ELEM_INT4 ? 7.0f : 448.0f;
    constexpr float RC = EK == ELEM_E2M1 ? 0x1.555556p-3f : EK == ELEM_INT4 ? 0x1.24924ap-3f : 0x1.24924ap-9f;
    return quotient<SCALE_E4M3, false>(amax, C, RC);
}

template <int EK, int SK>
__device__ __forceinline__ int naive_code(float amax)
{
    if (SK == SCALE_INT8 || SK == SCALE_E4M3) {
        const float v = (SK == SCALE_INT8) ? amax : div_elem_max<EK>(amax);
        const float y = round_elem<ELEM_E4M3>(v);
        return (int)elem_index<ELEM_E4M3>(y);
    }
    if (SK == SCALE_UE4M4) return ue_round_code<4, 7>(div_elem_max<EK>(amax));
    if (SK == SCALE_UE5M3) return ue_round_code<3, 15>(div_elem_max<EK>(amax));
    if (SK == SCALE_F16) return f16_round_code((double)div_elem_max<EK>(amax));  // fp16(fl32(amax / C))
    const float v = amax / elem_max(EK);
    if (v == 0.0f) return 0;
    // v = f 2^E with f in [1, 2); frexp gives the exponent for subnormals too
    int ex;
    const float f = __builtin_frexpf(v, &ex);   // v = f 2^ex, f in [0.5, 1)
    int E = ex - 1;
    if (f >= 0.75f) E += 1;                     // 2f >= 1.5: round up (ties up)
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
    return E + 127;
}

}  // namespace hd
