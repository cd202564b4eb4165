// encode.hpp - per-element encode with a known scale, shared by the Naive /
// encode kernel and the final encode of the search kernel.
#pragma once
#include "common.hpp"
#include "formats.hpp"

namespace hd {

// Encode 8 elements w[0..7] with scale s (s == 0: the zero scale) and
// r = fl32(1/s) (0 for s == 0).  Writes the code of each element (sign
// included) and returns the objective sum_j om_j (w_j - fl32(s q_j))^2 of the
// eight, in float64 and element order (om == NULL: unweighted).  rm_tab: see
// scale_parts (TAB).  Branch-free: the zero scale multiplies the quotients by 0.
template <int EK, int SK, bool ONE_STEP, bool WANT_OBJ = true, bool TAB = false>
__device__ __forceinline__ double encode8(const float *w, float s, float r, const double *om,
                                          uint32_t *code, const float *rm_tab = nullptr)
{
    double obj = 0.0;
    if (elem_int(EK)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float a = fabsf(w[j]);
            // s == 0 (r == 0): fl32(a 0) = 0, fma(-0, 0, a) = a, fma(a, 0, 0) = 0
            const float x = quotient<SK, ONE_STEP>(a, s, r);
            const float y = round_elem<EK>(x);
            code[j] = elem_code<EK>(elem_index<EK>(y), __builtin_signbitf(w[j]) != 0);
            if (WANT_OBJ) {
                const float wq = s * y;  // fl32(s * val(q))
                const double d = (double)a - (double)wq;
                obj += (om ? om[j] : 1.0) * (d * d);
            }
        }
        return obj;
    }
    // E2M1 / E4M3 elements: fl32(w / m) into the conversion instruction with
    // the power of two p2 (s = m p2); the same arithmetic as the search.  The
    // quotient is an odd function of w (its sign is copied back because the
    // correction steps turn -0 into +0) and the conversion keeps the sign,
    // zero included, so its codes already carry the sign bits.
    const ScaleParts sp = scale_parts<SK, TAB>(s, rm_tab);
    const float keep = s == 0.0f ? 0.0f : 1.0f;  // the zero scale: every element to +-0
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // (an FP16 scale's mantissa m is one of 1024: both quotient corrections)
        float v = (SK == SCALE_E8M0 ? w[j]
                                    : __builtin_copysignf(quotient_m<ONE_STEP && SK != SCALE_F16>(w[j], sp.m, sp.rm),
                                                          w[j])) *
                  keep;
        if (EK == ELEM_E4M3) v = fminf(fmaxf(v, -448.0f * sp.p2), 448.0f * sp.p2);
        x[j] = v;
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const uint32_t c2 = EK == ELEM_E2M1 ? fp4x2(x[j], x[j + 1], sp.p2) : fp8x2(x[j], x[j + 1], sp.p2);
        const uint32_t sh = EK == ELEM_E2M1 ? 4u : 8u, mask = EK == ELEM_E2M1 ? 15u : 0xFFu;
        code[j] = c2 & mask;
        code[j + 1] = (c2 >> sh) & mask;
        if (WANT_OBJ) {
            const hd_v2f v = EK == ELEM_E2M1 ? fp4x2_val(c2) : fp8x2_val(c2);
            const double d0 = (double)w[j] - (double)(s * v.x);
            const double d1 = (double)w[j + 1] - (double)(s * v.y);
            obj += (om ? om[j] : 1.0) * (d0 * d0);
            obj += (om ? om[j + 1] : 1.0) * (d1 * d1);
        }
    }
    return obj;
}

// Scale code of block `blk`: a byte, or binary16 bits for FP16 scales.
template <int SK>
__device__ __forceinline__ int load_scale(const uint8_t *scales, int64_t blk)
{
    if (SK == SCALE_F16) return (int)reinterpret_cast<const uint16_t *>(scales)[blk];
    return (int)scales[blk];
}
template <int SK>
__device__ __forceinline__ void store_scale(uint8_t *scales, int64_t blk, int code)
{
    if (SK == SCALE_F16)
        reinterpret_cast<uint16_t *>(scales)[blk] = (uint16_t)code;
    else
        scales[blk] = (uint8_t)code;
}

// Store the 8 codes of elements e0..e0+7 (e0 % 8 == 0).
template <int EK>
__device__ __forceinline__ void store_codes8(uint8_t *codes, int64_t e0, const uint32_t *c)
{
    if (elem_4bit(EK)) {
        const uint32_t v = (c[0] & 15u) | ((c[1] & 15u) << 4) | ((c[2] & 15u) << 8) | ((c[3] & 15u) << 12) |
                           ((c[4] & 15u) << 16) | ((c[5] & 15u) << 20) | ((c[6] & 15u) << 24) |
                           ((c[7] & 15u) << 28);
        *reinterpret_cast<uint32_t *>(codes + e0 / 2) = v;
    } else {
        uint2 v;
        v.x = (c[0] & 255u) | ((c[1] & 255u) << 8) | ((c[2] & 255u) << 16) | ((c[3] & 255u) << 24);
        v.y = (c[4] & 255u) | ((c[5] & 255u) << 8) | ((c[6] & 255u) << 16) | ((c[7] & 255u) << 24);
        *reinterpret_cast<uint2 *>(codes + e0) = v;
    }
}

}  // namespace hd
