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
// shuffles; for B = 4 a lane's eight weights are two whole blocks.  A
// workgroup inside W gathers its codes and scale codes in LDS and writes them
// with 16-byte and 4-byte stores per lane; the last, ragged workgroup (and
// B = 4) writes 4 (4-bit) or 8 bytes per lane and sub-chunk, on consecutive
// addresses, and one scale per block from the block's first lane.
static constexpr int ENC_SUB = 4;

// Scale code of one block with largest magnitude amax: given, or the Naive
// snap (the OCP floor rule on E8M0 grids when ocp is set).
template <int EK, int SK, bool GIVEN>
__device__ __forceinline__ int enc_scale_code(float amax, const uint8_t *scales_in, int64_t blk, bool in, int ocp)
{
    if (GIVEN) return in ? load_scale<SK>(scales_in, blk) : 0;
    if constexpr (SK == SCALE_E8M0) return ocp ? ocp_code<EK>(amax) : naive_code<EK, SK>(amax);
    return naive_code<EK, SK>(amax);
}

// Scale value of a valid code: from the table on the INT8 grid (its values
// are fl32(val / 127), a division each), by bit formula on the others.
template <int SK>
__device__ __forceinline__ float enc_scale_value(int code, const float *stab)
{
    if (SK == SCALE_INT8) return stab[code & 127];
    return scale_value(SK, code);
}

// fl32(1 / s) for the integer element grids (0 for s == 0): from the table
// on the INT8 grid, by division on the others (INT4 elements); E2M1 / E4M3
// elements do not use it (their quotients take scale_parts).
template <int EK, int SK>
__device__ __forceinline__ float enc_recip(float s, int code, const float *rtab)
{
    if (!elem_int(EK)) return 0.0f;
    if (SK == SCALE_INT8) return s != 0.0f ? rtab[code & 127] : 0.0f;
    return s != 0.0f ? 1.0f / s : 0.0f;
}

template <int EK, int SK, typename T, int B, bool GIVEN, bool OBJ>
__global__ __launch_bounds__(256) void encode_kernel(const T *__restrict__ W, int64_t total, int64_t K,
                                                     const float *__restrict__ h,
                                                     const uint8_t *__restrict__ scales_in,
                                                     uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                     float *__restrict__ block_obj, int ocp)
{
    constexpr int LPB = B >= 8 ? B / 8 : 1;  // lanes per block (B = 4: two blocks per lane)
    constexpr bool ONE_STEP = sizeof(T) == 2;
    // reciprocals without a division per block: the INT8 grid's fl32(1 / s)
    // per scale code (0 for code 0), else fl32(1 / (1 + j / 16)) for the
    // mantissas of the E4M3 / UE4M4 / UE5M3 grids (see scale_parts)
    constexpr bool RTAB = SK == SCALE_INT8 || SK == SCALE_E4M3 || SK == SCALE_UE4M4 || SK == SCALE_UE5M3;
    __shared__ float rtab[128], stab[128];  // stab: the INT8 grid's scale values
    if (RTAB) {
        const int t = threadIdx.x;
        if (SK == SCALE_INT8) {
            if (t < 128) {
                const float sv = (t >= 1 && t <= 126) ? scale_value(SCALE_INT8, t) : 0.0f;
                stab[t] = sv;
                rtab[t] = sv != 0.0f ? 1.0f / sv : 0.0f;
            }
        } else if (t < 16) {
            rtab[t] = 1.0f / (1.0f + (float)t * 0.0625f);
        }
        __syncthreads();
    }
    // A workgroup whose weights all lie inside W gathers its codes and scale
    // codes in LDS and writes them out as 16-byte (codes) and 4-byte (scale)
    // stores per lane, instead of one 4- or 8-byte store per lane and one
    // scale per block: fewer, fuller write requests.  The last workgroup of
    // a ragged grid, and B = 4, store directly.
    constexpr int CW = elem_4bit(EK) ? 1 : 2;              // code dwords per lane and sub-chunk
    constexpr int SB = SK == SCALE_F16 ? 2 : 1;            // bytes per scale code
    constexpr int SCB = 512 * ENC_SUB / (B >= 8 ? B : 8) * SB;  // scale bytes per wave (a multiple of 8)
    __shared__ uint32_t lcode[4][64 * ENC_SUB * CW];
    __shared__ uint32_t lscale[4][SCB / 4];
    const bool staged = B >= 8 && (int64_t)(blockIdx.x + 1) * (256 * 8 * ENC_SUB) <= total &&
                        (GIVEN || ((uintptr_t)scales & 3u) == 0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wbase = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * (64 * 8 * ENC_SUB);
    // total % 8 == 0 and total % B == 0: a sub-chunk starting below total is
    // whole, and the lanes of one block are all in or all out.  Every lane
    // loads (sub-chunks past the end read the last 8 weights and are dropped),
    // so the waits can go sub-chunk by sub-chunk.
    float w[ENC_SUB][8];
#pragma unroll
    for (int k = 0; k < ENC_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        load8_nt<T>(W + (e < total ? e : total - 8), w[k]);
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
        if constexpr (B == 4) {
            // two blocks: each half is encoded as eight weights of which the
            // last four are zeros (they encode to 0 and add nothing)
            uint32_t c[8];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                float wh[8], amax = 0.0f;
                double omh[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    wh[j] = j < 4 ? w[k][4 * hb + j] : 0.0f;
                    omh[j] = (OBJ && weighted && in && j < 4) ? om[OBJ ? 4 * hb + j : 0] : 0.0;
                    amax = fmaxf(amax, fabsf(wh[j]));
                }
                const int64_t blk = e / 4 + hb;
                const int code = enc_scale_code<EK, SK, GIVEN>(amax, scales_in, blk, in, ocp);
                const float s = (GIVEN ? scale_code_valid(SK, code) : true) ? enc_scale_value<SK>(code, stab) : 0.0f;
                const float r = enc_recip<EK, SK>(s, code, rtab);
                uint32_t ch[8];
                const double o = encode8<EK, SK, ONE_STEP, OBJ, RTAB>(wh, s, r, (weighted && in) ? omh : nullptr,
                                                                      ch, rtab);
#pragma unroll
                for (int j = 0; j < 4; ++j) c[4 * hb + j] = ch[j];
                if (in) {
                    if (!GIVEN) store_scale<SK>(scales, blk, code);
                    if (OBJ) block_obj[blk] = (float)o;
                }
            }
            if (!in) continue;
            if (elem_4bit(EK)) {
                uint32_t v = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) v |= (c[j] & 15u) << (4 * j);
                __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(codes + e / 2));
            } else {
                const uint32_t lo = (c[0] & 255u) | ((c[1] & 255u) << 8) | ((c[2] & 255u) << 16) | ((c[3] & 255u) << 24);
                const uint32_t hi = (c[4] & 255u) | ((c[5] & 255u) << 8) | ((c[6] & 255u) << 16) | ((c[7] & 255u) << 24);
                __builtin_nontemporal_store((uint64_t)lo | ((uint64_t)hi << 32), reinterpret_cast<uint64_t *>(codes + e));
            }
            continue;
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
            s = scale_code_valid(SK, code) ? enc_scale_value<SK>(code, stab) : 0.0f;
        } else {
            // ocp (E8M0 grids only): the OCP MX floor rule instead of the snap
            if constexpr (SK == SCALE_E8M0)
                code = ocp ? ocp_code<EK>(amax) : naive_code<EK, SK>(amax);
            else
                code = naive_code<EK, SK>(amax);
            s = enc_scale_value<SK>(code, stab);
        }
        const float r = enc_recip<EK, SK>(s, code, rtab);
        uint32_t c[8];
        double o = encode8<EK, SK, ONE_STEP, OBJ, RTAB>(w[k], s, r, (weighted && in) ? om : nullptr, c, rtab);
        if (OBJ) o = group_sum<LPB>(o);
        if (!in) continue;
        uint32_t v[CW];
        if (elem_4bit(EK)) {
            v[0] = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[0] |= (c[j] & 15u) << (4 * j);
        } else {
            v[0] = (c[0] & 255u) | ((c[1] & 255u) << 8) | ((c[2] & 255u) << 16) | ((c[3] & 255u) << 24);
            v[CW - 1] = (c[4] & 255u) | ((c[5] & 255u) << 8) | ((c[6] & 255u) << 16) | ((c[7] & 255u) << 24);
        }
        if (staged) {
            // dword (64 k + lane) CW of the wave's codes
#pragma unroll
            for (int j = 0; j < CW; ++j) lcode[wv][(64 * k + lane) * CW + j] = v[j];
        } else if (elem_4bit(EK)) {
            __builtin_nontemporal_store(v[0], reinterpret_cast<uint32_t *>(codes + e / 2));  // streamed out
        } else {
            __builtin_nontemporal_store((uint64_t)v[0] | ((uint64_t)v[CW - 1] << 32),
                                        reinterpret_cast<uint64_t *>(codes + e));
        }
        if (lane % LPB == 0) {
            if (!GIVEN) {
                if (staged)
                    store_scale<SK>(reinterpret_cast<uint8_t *>(lscale[wv]), (512 * k + 8 * lane) / B, code);
                else
                    store_scale<SK>(scales, blk, code);
            }
            if (OBJ) block_obj[blk] = (float)o;
        }
    }
    if (B >= 8 && staged) {
        __syncthreads();  // staged is uniform over the workgroup
        const hd_u32x4 *src = reinterpret_cast<const hd_u32x4 *>(lcode[wv]);
        hd_u32x4 *dst = reinterpret_cast<hd_u32x4 *>(codes + wbase * CW / 2);
#pragma unroll
        for (int i = lane; i < 16 * ENC_SUB * CW; i += 64) __builtin_nontemporal_store(src[i], dst + i);
        if (!GIVEN) {
            uint32_t *sdst = reinterpret_cast<uint32_t *>(scales + wbase / (B >= 8 ? B : 8) * SB);
            for (int i = lane; i < SCB / 4; i += 64) sdst[i] = lscale[wv][i];
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
        HD_ENC_CASE(4)
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
    // the INT8 grid's scale values fl32(val / 127), one division per code
    // per workgroup instead of one per output group
    __shared__ float stab[128];
    if (SK == SCALE_INT8) {
        if (threadIdx.x < 128)
            stab[threadIdx.x] = scale_code_valid(SK, threadIdx.x) ? scale_value(SK, threadIdx.x) : 0.0f;
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t base = wave * (64 * VPS * DQ_G) + (int64_t)lane * VPS;
    // all loads first (codes and scales of the DQ_G groups), then the stores
    uint64_t cw[DQ_G];
    int sc[DQ_G], sc2[DQ_G];
#pragma unroll
    for (int g = 0; g < DQ_G; ++g) {
        const int64_t e = base + (int64_t)g * 64 * VPS;
        cw[g] = 0;
        sc[g] = 0;
        sc2[g] = 0;
        if (e < total) {  // total % 8 == 0: a group starting inside is whole
            if (elem_4bit(EK))
                cw[g] = VPS == 8 ? *reinterpret_cast<const uint32_t *>(codes + e / 2)
                                 : *reinterpret_cast<const uint16_t *>(codes + e / 2);
            else
                cw[g] = VPS == 8 ? *reinterpret_cast<const uint64_t *>(codes + e)
                                 : *reinterpret_cast<const uint32_t *>(codes + e);
            sc[g] = load_scale<SK>(scales, e / B);
            if (VPS > B) sc2[g] = load_scale<SK>(scales, e / B + 1);  // B = 4, bfloat16: two blocks
        }
    }
#pragma unroll
    for (int g = 0; g < DQ_G; ++g) {
        const int64_t e = base + (int64_t)g * 64 * VPS;
        if (e >= total) break;
        const float s = SK == SCALE_INT8 ? stab[sc[g] & 127] * (sc[g] < 128 ? 1.0f : 0.0f)
                                         : (scale_code_valid(SK, sc[g]) ? scale_value(SK, sc[g]) : 0.0f);
        float o[VPS];
        dq_group<EK, VPS>(cw[g], s, tscale, o);
        if (VPS > B) {  // the second block's four outputs at its own scale
            const float s2 = SK == SCALE_INT8 ? stab[sc2[g] & 127] * (sc2[g] < 128 ? 1.0f : 0.0f)
                                              : (scale_code_valid(SK, sc2[g]) ? scale_value(SK, sc2[g]) : 0.0f);
            float o2[VPS];
            dq_group<EK, VPS>(cw[g], s2, tscale, o2);
#pragma unroll
            for (int j = VPS / 2; j < VPS; ++j) o[j] = o2[j];
        }
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
// Each thread keeps 8 running pairs over its partials i = threadIdx.x + 256 j
// (j mod 8), so 8 loads are in flight per round; indices past n are clamped
// for the load and contribute 0.
__global__ __launch_bounds__(256) void ratio_final(const double *__restrict__ part, int n,
                                                   double *__restrict__ out, double *__restrict__ sums)
{
    __shared__ double sh[4];
    const double2 *pp = reinterpret_cast<const double2 *>(part);
    double av[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0}, bv[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int i0 = threadIdx.x; i0 < n; i0 += 2048) {
        double2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = pp[min(i0 + 256 * u, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = i0 + 256 * u < n;
            av[u] += in ? x[u].x : 0.0;
            bv[u] += in ? x[u].y : 0.0;
        }
    }
    double a = ((av[0] + av[1]) + (av[2] + av[3])) + ((av[4] + av[5]) + (av[6] + av[7]));
    double b = ((bv[0] + bv[1]) + (bv[2] + bv[3])) + ((bv[4] + bv[5]) + (bv[6] + bv[7]));
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

// ------------------------------------------- dequantize + weight error ---
// dequantize() and weight_error() in one pass over the codes and W: each
// 8-weight chunk is decoded exactly as dequant_kernel decodes it, stored in
// the output dtype, and its stored values enter the error sums.  The grid,
// the chunks each thread takes and their order are werr_partial's, so the
// partial sums, and the ratio ratio_final makes of them, are those of
// weight_error(W, Wq) on the Wq written here.
template <int EK, int SK, int OUT_BF16, typename TW>
__device__ __forceinline__ void dqwe_chunk(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                           int B, const float *stab, int64_t e, void *__restrict__ out, const float *w,
                                           double &num, double &den)
{
    uint64_t cw;
    if (elem_4bit(EK))
        cw = *reinterpret_cast<const uint32_t *>(codes + e / 2);
    else
        cw = *reinterpret_cast<const uint64_t *>(codes + e);
    auto sval = [&](int c) {
        return SK == SCALE_INT8 ? stab[c & 127] * (c < 128 ? 1.0f : 0.0f)
                                : (scale_code_valid(SK, c) ? scale_value(SK, c) : 0.0f);
    };
    float o[8];
    dq_group<EK, 8>(cw, sval(load_scale<SK>(scales, e / B)), nullptr, o);
    if (B == 4) {  // the chunk's second block at its own scale
        float o2[8];
        dq_group<EK, 8>(cw, sval(load_scale<SK>(scales, e / B + 1)), nullptr, o2);
#pragma unroll
        for (int j = 4; j < 8; ++j) o[j] = o2[j];
    }
    float q[8];
    if (OUT_BF16) {
        uint32_t u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = f32_to_bf16(o[2 * j]), hi = f32_to_bf16(o[2 * j + 1]);
            u[j] = lo | (hi << 16);
            q[2 * j] = bf16_to_f32(lo);
            q[2 * j + 1] = bf16_to_f32(hi);
        }
        *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(out) + e) = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
        float *op = static_cast<float *>(out) + e;
        *reinterpret_cast<float4 *>(op) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4 *>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = o[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double d = (double)q[j] - (double)w[j];
        num += d * d;
        den += (double)w[j] * (double)w[j];
    }
}

template <int EK, int SK, int OUT_BF16, typename TW>
__global__ __launch_bounds__(256) void dqwe_partial(const uint8_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ scales, int B,
                                                    const TW *__restrict__ W, int64_t total, void *__restrict__ out,
                                                    double *__restrict__ part)
{
    __shared__ double sh[4];
    __shared__ float stab[128];  // the INT8 grid's scale values fl32(val / 127)
    if (SK == SCALE_INT8) {
        if (threadIdx.x < 128)
            stab[threadIdx.x] = scale_code_valid(SK, threadIdx.x) ? scale_value(SK, threadIdx.x) : 0.0f;
        __syncthreads();
    }
    double num = 0.0, den = 0.0;
    const int64_t stride = (int64_t)gridDim.x * 256 * 8;
    for (int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; e0 < total; e0 += 2 * stride) {
        const int64_t e1 = e0 + stride;
        const bool two = e1 < total;
        float w[16];
        load8_nt<TW>(W + e0, w);  // each weight is read once here
        if (two) load8_nt<TW>(W + e1, w + 8);
        dqwe_chunk<EK, SK, OUT_BF16, TW>(codes, scales, B, stab, e0, out, w, num, den);
        if (two) dqwe_chunk<EK, SK, OUT_BF16, TW>(codes, scales, B, stab, e1, out, w + 8, num, den);
    }
    num = block_sum_256(num, sh);
    den = block_sum_256(den, sh);
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = num;
        part[2 * blockIdx.x + 1] = den;
    }
}

template <int EK, int SK>
static void dqwe_f(int B, const uint8_t *codes, const uint8_t *scales, int64_t total, void *out, int out_t,
                   const void *W, int wdt, int grid, double *part, hipStream_t st)
{
    if (wdt == 1) {
        if (out_t == 1)
            dqwe_partial<EK, SK, 1, bf16_t><<<grid, 256, 0, st>>>(codes, scales, B, (const bf16_t *)W, total, out, part);
        else
            dqwe_partial<EK, SK, 0, bf16_t><<<grid, 256, 0, st>>>(codes, scales, B, (const bf16_t *)W, total, out, part);
    } else {
        if (out_t == 1)
            dqwe_partial<EK, SK, 1, float><<<grid, 256, 0, st>>>(codes, scales, B, (const float *)W, total, out, part);
        else
            dqwe_partial<EK, SK, 0, float><<<grid, 256, 0, st>>>(codes, scales, B, (const float *)W, total, out, part);
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

hipError_t launch_dequant_weight_error(int fmt, int B, const uint8_t *codes, const uint8_t *scales, int64_t N,
                                       int64_t K, void *Wq, int out_t, const void *W, int wdt, double *out,
                                       double *sums, void *ws, hipStream_t st)
{
    const int64_t total = N * K;
    int64_t g = (total / 8 + 255) / 256;
    const int grid = (int)(g < WE_GRID ? (g > 0 ? g : 1) : WE_GRID);  // werr_partial's grid
    double *part = static_cast<double *>(ws);
#define HD_DQWE_FMT(F)                                                                                     \
    case F:                                                                                                \
        dqwe_f<elem_kind(F), scale_kind(F)>(B, codes, scales, total, Wq, out_t, W, wdt, grid, part, st);  \
        break;
    switch (fmt) {
        HD_DQWE_FMT(HD_INT8_E4M3)
        HD_DQWE_FMT(HD_NVFP4)
        HD_DQWE_FMT(HD_MXFP4)
        HD_DQWE_FMT(HD_MXFP8)
        HD_DQWE_FMT(HD_FP8_E4M3S)
        HD_DQWE_FMT(HD_NVFP4_UE4M4)
        HD_DQWE_FMT(HD_NVFP4_UE5M3)
        HD_DQWE_FMT(HD_NVINT4)
        HD_DQWE_FMT(HD_FP4_F16)
        HD_DQWE_FMT(HD_INT4_F16)
    default: return hipErrorInvalidValue;
    }
#undef HD_DQWE_FMT
    ratio_final<<<1, 256, 0, st>>>(part, grid, out, sums);
    return hipGetLastError();
}

}  // namespace hd
