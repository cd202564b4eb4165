// quant.hip - Naive scale + encode, encode with given scales, dequantize and
// the weight error: the HBM-bound streaming kernels of the path.
#include "encode.hpp"
#include "kernels.hpp"

namespace hd {


// ---------------------------------------------------------------- encode ---
// Naive ("Is Finer Better?" §2.1: s = Q_scale(amax / C); qwantize "Results",
// INT8: the amax itself stored as E4M3 and divided by 127) when GIVEN is false;
// otherwise the scale code of each block comes from scales_in.
//
// Each wave covers 2048 consecutive weights in four sub-chunks of 512: lane
// l takes weights 512 k + 8 l .. + 7 of sub-chunk k (one 16-byte bf16 or two
// float32 loads, the lanes of a wave on consecutive addresses: loads strided
// across lanes were measured to cut the read rate), so a block of B weights
// is B / 8 adjacent lanes of one sub-chunk (512 % B == 0), combined with
// shuffles.  Codes go out as 4 (4-bit) or 8 bytes per lane and sub-chunk,
// again on consecutive addresses; the first lane of a block writes its scale.
static constexpr int ENC_SUB = 4;

template <int EK, int SK, typename T, int B, bool GIVEN, bool OBJ>
__global__ __launch_bounds__(256) void encode_kernel(const T *__restrict__ W, int64_t total, int64_t K,
                                                     const float *__restrict__ h,
                                                     const uint8_t *__restrict__ scales_in,
                                                     uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                     float *__restrict__ block_obj, int ocp)
{
    constexpr int LPB = B / 8;  // lanes per block
    constexpr bool ONE_STEP = sizeof(T) == 2;
    const int lane = threadIdx.x & 63;
    const int64_t wbase = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * (64 * 8 * ENC_SUB);
    // total % B == 0 and B % 8 == 0: a sub-chunk starting below total is
    // whole, and the lanes of one block are all in or all out
    float w[ENC_SUB][8];
#pragma unroll
    for (int k = 0; k < ENC_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        if (e < total)
            load8_nt<T>(W + e, w[k]);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) w[k][j] = 0.0f;
    }
    const bool weighted = OBJ && h != nullptr;
#pragma unroll
    for (int k = 0; k < ENC_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        const bool in = e < total;
        double om[OBJ ? 8 : 1];
        if (OBJ && weighted && in) {
            const int64_t k0 = e % K;  // rows hold K % 8 == 0 weights: no row end inside
#pragma unroll
            for (int j = 0; j < 8; ++j) om[OBJ ? j : 0] = (double)h[k0 + j];
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(w[k][j]));
        amax = group_max<LPB>(amax);
        const int64_t blk = e / B;
        int code;
        float s;
        if (GIVEN) {
            code = in ? load_scale<SK>(scales_in, blk) : 0;
            s = scale_code_valid(SK, code) ? scale_value(SK, code) : 0.0f;
        } else {
            // ocp (E8M0 grids only): the OCP MX floor rule instead of the snap
            if constexpr (SK == SCALE_E8M0)
                code = ocp ? ocp_code<EK>(amax) : naive_code<EK, SK>(amax);
            else
                code = naive_code<EK, SK>(amax);
            s = scale_value(SK, code);
        }
        const float r = (s != 0.0f) ? 1.0f / s : 0.0f;
        uint32_t c[8];
        double o = encode8<EK, SK, ONE_STEP, OBJ>(w[k], s, r, (weighted && in) ? om : nullptr, c);
        if (OBJ) o = group_sum<LPB>(o);
        if (!in) continue;
        if (elem_4bit(EK)) {
            uint32_t v = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) v |= (c[j] & 15u) << (4 * j);
            __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(codes + e / 2));  // streamed out
        } else {
            uint2 v;
            v.x = (c[0] & 255u) | ((c[1] & 255u) << 8) | ((c[2] & 255u) << 16) | ((c[3] & 255u) << 24);
            v.y = (c[4] & 255u) | ((c[5] & 255u) << 8) | ((c[6] & 255u) << 16) | ((c[7] & 255u) << 24);
            __builtin_nontemporal_store((uint64_t)v.x | ((uint64_t)v.y << 32), reinterpret_cast<uint64_t *>(codes + e));
        }
        if (lane % LPB == 0) {
            if (!GIVEN) store_scale<SK>(scales, blk, code);
            if (OBJ) block_obj[blk] = (float)o;
        }
    }
}

template <int EK, int SK, typename T, bool GIVEN>
static hipError_t encode_b(int B, const void *W, int64_t N, int64_t K, const float *h, const uint8_t *si,
                           uint8_t *codes, uint8_t *scales, float *bo, int ocp, hipStream_t st)
{
    const int64_t total = N * K;
    const int64_t waves = (total + 64 * 8 * ENC_SUB - 1) / (64 * 8 * ENC_SUB);
    const dim3 grid((unsigned)((waves + 3) / 4));
    const T *w = static_cast<const T *>(W);
#define HD_ENC_CASE(BB)                                                                                      \
    case BB:                                                                                                 \
        if (bo)                                                                                              \
            encode_kernel<EK, SK, T, BB, GIVEN, true><<<grid, 256, 0, st>>>(w, total, K, h, si, codes, scales, bo, ocp);  \
        else                                                                                                 \
            encode_kernel<EK, SK, T, BB, GIVEN, false><<<grid, 256, 0, st>>>(w, total, K, h, si, codes, scales, bo, ocp); \
        break;
    switch (B) {
        HD_ENC_CASE(8)
        HD_ENC_CASE(16)
        HD_ENC_CASE(32)
        HD_ENC_CASE(64)
        HD_ENC_CASE(128)
        HD_ENC_CASE(256)
    default: return hipErrorInvalidValue;
    }
#undef HD_ENC_CASE
    return hipGetLastError();
}

template <int EK, int SK>
static hipError_t encode_f(int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                           const uint8_t *si, uint8_t *codes, uint8_t *scales, float *bo, int ocp, hipStream_t st)
{
    if (si) {
        return wdt == 1 ? encode_b<EK, SK, bf16_t, true>(B, W, N, K, h, si, codes, scales, bo, 0, st)
                        : encode_b<EK, SK, float, true>(B, W, N, K, h, si, codes, scales, bo, 0, st);
    }
    return wdt == 1 ? encode_b<EK, SK, bf16_t, false>(B, W, N, K, h, si, codes, scales, bo, ocp, st)
                    : encode_b<EK, SK, float, false>(B, W, N, K, h, si, codes, scales, bo, ocp, st);
}

hipError_t launch_encode(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                         const uint8_t *scales_in, uint8_t *codes, uint8_t *scales, float *block_obj, int ocp,
                         hipStream_t st)
{
#define HD_ENC_FMT(F)                                                                                      \
    case F:                                                                                                \
        return encode_f<elem_kind(F), scale_kind(F)>(B, W, wdt, N, K, h, scales_in, codes, scales, block_obj, ocp, st);
    switch (fmt) {
        HD_ENC_FMT(HD_INT8_E4M3)
        HD_ENC_FMT(HD_NVFP4)
        HD_ENC_FMT(HD_MXFP4)
        HD_ENC_FMT(HD_MXFP8)
        HD_ENC_FMT(HD_FP8_E4M3S)
        HD_ENC_FMT(HD_NVFP4_UE4M4)
        HD_ENC_FMT(HD_NVFP4_UE5M3)
        HD_ENC_FMT(HD_NVINT4)
        HD_ENC_FMT(HD_FP4_F16)
        HD_ENC_FMT(HD_INT4_F16)
    }
#undef HD_ENC_FMT
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------ dequantize ---
// x^ = s q ("Is Finer Better?" §2.1): sign * fl32(s * val(index)).
// With a per-tensor scale t (tscale != NULL): t * fl32(s * val(index)).
// Every store is one 16-byte vector per lane with the lanes of a wave on
// consecutive addresses (VPS = 4 float32 or 8 bfloat16 outputs per lane and
// store): lane l of a wave takes, in each of DQ_G groups, the VPS outputs
// starting at wave_base + g 64 VPS + l VPS, whose codes it loads as one
// 2- to 8-byte word and whose block scale (VPS divides B) it loads once.
static constexpr int DQ_G = 4;

// VPS outputs from VPS codes packed in cw (4 or 8 bits each): the signed grid
// values times s (exact products), times the tensor scale if given.  E2M1 and
// E4M3 codes go through the gfx950 conversions (two values per instruction,
// sign and signed zero kept); the integer grids sign-extend.  Codes outside
// a grid (E4M3 0x7F / 0xFF, INT8 -128, INT4 -8) give a zero of their sign.
template <int EK, int VPS>
__device__ __forceinline__ void dq_group(uint64_t cw, float s, const float *tscale, float *o)
{
    if (EK == ELEM_E2M1) {
        hd_v2f v[4];
        v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)cw, 1.0f, 0);
        v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)cw, 1.0f, 1);
        if constexpr (VPS == 8) {
            v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)cw, 1.0f, 2);
            v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)cw, 1.0f, 3);
        }
#pragma unroll
        for (int p = 0; p < VPS / 2; ++p) {
            o[2 * p] = s * v[p].x;
            o[2 * p + 1] = s * v[p].y;
        }
    } else if (EK == ELEM_E4M3) {
#pragma unroll
        for (int p = 0; p < VPS / 2; ++p) {
            const uint32_t word = (uint32_t)(cw >> (32 * (p / 2))) >> (16 * (p & 1));
            const hd_v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t code = (uint32_t)(cw >> (8 * (2 * p + h))) & 255u;
                const float z = (code & 0x80u) ? -0.0f : 0.0f;
                o[2 * p + h] = (code & 0x7Fu) == 0x7Fu ? z : s * (h ? v.y : v.x);
            }
        }
    } else {
        constexpr int BITS = EK == ELEM_INT8 ? 8 : 4;
#pragma unroll
        for (int j = 0; j < VPS; ++j) {
            const int q = __builtin_amdgcn_sbfe((int)(uint32_t)(cw >> (BITS * j)), 0, BITS);
            o[j] = q == -(1 << (BITS - 1)) ? -0.0f : s * (float)q;
        }
    }
    if (tscale) {
        const float t = tscale[0];
#pragma unroll
        for (int j = 0; j < VPS; ++j) o[j] = t * o[j];
    }
}

template <int EK, int SK, int OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int64_t total,
                                                      int B, void *__restrict__ out,
                                                      const float *__restrict__ tscale)
{
    constexpr int VPS = OUT_BF16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t base = wave * (64 * VPS * DQ_G) + (int64_t)lane * VPS;
    // all loads first (codes and scales of the DQ_G groups), then the stores
    uint64_t cw[DQ_G];
    int sc[DQ_G];
#pragma unroll
    for (int g = 0; g < DQ_G; ++g) {
        const int64_t e = base + (int64_t)g * 64 * VPS;
        cw[g] = 0;
        sc[g] = 0;
        if (e < total) {  // total % 8 == 0: a group starting inside is whole
            if (elem_4bit(EK))
                cw[g] = VPS == 8 ? *reinterpret_cast<const uint32_t *>(codes + e / 2)
                                 : *reinterpret_cast<const uint16_t *>(codes + e / 2);
            else
                cw[g] = VPS == 8 ? *reinterpret_cast<const uint64_t *>(codes + e)
                                 : *reinterpret_cast<const uint32_t *>(codes + e);
            sc[g] = load_scale<SK>(scales, e / B);
        }
    }
#pragma unroll
    for (int g = 0; g < DQ_G; ++g) {
        const int64_t e = base + (int64_t)g * 64 * VPS;
        if (e >= total) break;
        const float s = scale_code_valid(SK, sc[g]) ? scale_value(SK, sc[g]) : 0.0f;
        float o[VPS];
        dq_group<EK, VPS>(cw[g], s, tscale, o);
        if (OUT_BF16) {
            uint4 v;
            v.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
            v.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
            v.z = f32_to_bf16(o[4 % VPS]) | (f32_to_bf16(o[5 % VPS]) << 16);
            v.w = f32_to_bf16(o[6 % VPS]) | (f32_to_bf16(o[7 % VPS]) << 16);
            *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(out) + e) = v;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(out) + e) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
}

template <int EK, int SK>
static hipError_t dequant_f(int B, const uint8_t *codes, const uint8_t *scales, int64_t total, void *out,
                            int out_t, const float *tscale, hipStream_t st)
{
    // one wave per 64 DQ_G VPS outputs (VPS = 8 for bfloat16, 4 for float32)
    const int64_t per_wave = 64 * DQ_G * (out_t == 1 ? 8 : 4);
    const dim3 grid((unsigned)(((total + per_wave - 1) / per_wave + 3) / 4));
    if (out_t == 1)
        dequant_kernel<EK, SK, 1><<<grid, 256, 0, st>>>(codes, scales, total, B, out, tscale);
    else
        dequant_kernel<EK, SK, 0><<<grid, 256, 0, st>>>(codes, scales, total, B, out, tscale);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int B, const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                          void *out, int out_t, const float *tscale, hipStream_t st)
{
    const int64_t total = N * K;
#define HD_DEQ_FMT(F)                                                                                      \
    case F:                                                                                                \
        return dequant_f<elem_kind(F), scale_kind(F)>(B, codes, scales, total, out, out_t, tscale, st);
    switch (fmt) {
        HD_DEQ_FMT(HD_INT8_E4M3)
        HD_DEQ_FMT(HD_NVFP4)
        HD_DEQ_FMT(HD_MXFP4)
        HD_DEQ_FMT(HD_MXFP8)
        HD_DEQ_FMT(HD_FP8_E4M3S)
        HD_DEQ_FMT(HD_NVFP4_UE4M4)
        HD_DEQ_FMT(HD_NVFP4_UE5M3)
        HD_DEQ_FMT(HD_NVINT4)
        HD_DEQ_FMT(HD_FP4_F16)
        HD_DEQ_FMT(HD_INT4_F16)
    }
#undef HD_DEQ_FMT
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------- weight error ---
// ||Wq - W||_F / ||W||_F (qwantize "Results", metric definitions): each
// workgroup sums its grid-stride share in float64, the partials are combined
// in a fixed order by one workgroup.
static constexpr int WE_GRID = 2048;


template <typename TW, typename TQ>
__global__ __launch_bounds__(256) void werr_partial(const TW *__restrict__ W, const TQ *__restrict__ Wq,
                                                    int64_t total, double *__restrict__ part)
{
    __shared__ double sh[4];
    double num = 0.0, den = 0.0;
    // two 8-weight chunks per lane and iteration: four loads in flight
    const int64_t stride = (int64_t)gridDim.x * 256 * 8;
    for (int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; e0 < total; e0 += 2 * stride) {
        const int64_t e1 = e0 + stride;
        const bool two = e1 < total;
        float w[16], q[16];
        load8_nt<TW>(W + e0, w);  // non-temporal: each weight is read once here
        load8_nt<TQ>(Wq + e0, q);
        if (two) {
            load8_nt<TW>(W + e1, w + 8);
            load8_nt<TQ>(Wq + e1, q + 8);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double d = (double)q[j] - (double)w[j];
            num += d * d;
            den += (double)w[j] * (double)w[j];
        }
        if (two) {
#pragma unroll
            for (int j = 8; j < 16; ++j) {
                const double d = (double)q[j] - (double)w[j];
                num += d * d;
                den += (double)w[j] * (double)w[j];
            }
        }
    }
    num = block_sum_256(num, sh);
    den = block_sum_256(den, sh);
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = num;
        part[2 * blockIdx.x + 1] = den;
    }
}

// Sum `n` (num, den) partials in a fixed order; out = sqrt(num) / sqrt(den).
__global__ __launch_bounds__(256) void ratio_final(const double *__restrict__ part, int n,
                                                   double *__restrict__ out, double *__restrict__ sums)
{
    __shared__ double sh[4];
    double a = 0.0, b = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) {
        a += part[2 * i];
        b += part[2 * i + 1];
    }
    a = block_sum_256(a, sh);
    b = block_sum_256(b, sh);
    if (threadIdx.x == 0) {
        *out = sqrt(a) / sqrt(b);
        if (sums) {
            sums[0] = a;
            sums[1] = b;
        }
    }
}

size_t weight_error_ws(int64_t, int64_t) { return sizeof(double) * 2 * WE_GRID; }

hipError_t launch_weight_error(const void *W, int wdt, const void *Wq, int qdt, int64_t N, int64_t K,
                               double *out, double *sums, void *ws, hipStream_t st)
{
    const int64_t total = N * K;
    int64_t g = (total / 8 + 255) / 256;
    const int grid = (int)(g < WE_GRID ? (g > 0 ? g : 1) : WE_GRID);
    double *part = static_cast<double *>(ws);
    if (wdt == 1 && qdt == 1)
        werr_partial<bf16_t, bf16_t><<<grid, 256, 0, st>>>((const bf16_t *)W, (const bf16_t *)Wq, total, part);
    else if (wdt == 1)
        werr_partial<bf16_t, float><<<grid, 256, 0, st>>>((const bf16_t *)W, (const float *)Wq, total, part);
    else if (qdt == 1)
        werr_partial<float, bf16_t><<<grid, 256, 0, st>>>((const float *)W, (const bf16_t *)Wq, total, part);
    else
        werr_partial<float, float><<<grid, 256, 0, st>>>((const float *)W, (const float *)Wq, total, part);
    ratio_final<<<1, 256, 0, st>>>(part, grid, out, sums);
    return hipGetLastError();
}

}  // namespace hd
