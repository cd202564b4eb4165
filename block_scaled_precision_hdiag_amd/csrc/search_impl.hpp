// search_impl.hpp - SSE-Optimal / H-Optimal scale search (qwantize "Results",
// INT8 / NVFP4 / MXFP4 tables; the H weighting is the diagonal-Hessian
// objective of the quantisation algorithms note, §1).
//
// For every block the kernel evaluates
//     obj(c) = sum_j om_j (|w_j| - fl32(s_c Q(fl32(|w_j| / s_c))))^2
// over the candidate scale codes c of the grid, in ascending order, and keeps
// the first strict minimum (the lowest code on ties), then encodes the block
// with it.  om_j = 1 (SSE) or h_j (H).
//
// Mapping (the work is FP32-VALU bound, ~10 instructions per weight and
// candidate):
//   - one lane owns one block segment of SEG = min(B, 32) weights held in
//     registers; a block of B > 32 spans LPB = B / 32 adjacent lanes whose
//     partial objectives are combined with lane shuffles;
//   - all lanes of a workgroup share one block column (so h_j is the same for
//     every lane of a wave and is loaded once), and walk the candidates in
//     lock-step: the candidate (s, 1/s) pair is a broadcast read from LDS and
//     the running argmin needs no cross-lane reduction;
//   - each residual is exact in fp32 and squared / accumulated in float64, so
//     the objective differs from its exact value only by float64 rounding;
//   - candidates at and above the first scale that rounds the block's amax to
//     zero all give sum_j om_j w_j^2 (every element encodes to 0), so the wave
//     stops at the largest such first-zero code over its lanes: the skipped
//     codes could only tie, and ties keep the lower code.
#pragma once
#include "encode.hpp"
#include "kernels.hpp"

namespace hd {

template <int EK, int SK, bool ONE_STEP>
__device__ __forceinline__ float search_resid(float a, float s, float r)
{
    const float x = quotient<SK, ONE_STEP>(a, s, r);
    const float y = round_elem<EK>(x);
    if (EK == ELEM_INT8) {
        const float wq = s * y;  // fl32(s * q): INT8 scales carry a full fp32 mantissa
        return a - wq;
    }
    // E2M1 / E4M3 grid values times an E4M3 or power-of-two scale are exact
    // products, so this single-rounding FMA equals a - fl32(s * y).
    return __builtin_fmaf(-y, s, a);
}

template <int EK, int SK, typename T, int SEG, int LPB, bool WEIGHTED>
__global__ __launch_bounds__(256) void search_kernel(const T *__restrict__ W, int64_t N, int64_t K,
                                                     const float *__restrict__ h, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, float *__restrict__ block_obj)
{
    constexpr int B = SEG * LPB;
    constexpr int ROWS = 256 / LPB;
    constexpr int C0 = cand_first(SK);
    constexpr int NC = cand_last(SK) - C0 + 1;
    constexpr bool ONE_STEP = sizeof(T) == 2;
    __shared__ float2 cand[256];

    const int tid = threadIdx.x;
    if (tid < NC) {
        const float s = scale_value(SK, C0 + tid);
        cand[tid] = make_float2(s, 1.0f / s);
    }
    __syncthreads();

    const int64_t row = (int64_t)blockIdx.x * ROWS + tid / LPB;
    const int seg = tid % LPB;
    const int64_t col0 = (int64_t)blockIdx.y * B + (int64_t)seg * SEG;
    const bool active = row < N;

    float a[SEG];
    uint32_t negmask = 0;
    {
        float w[8];
#pragma unroll
        for (int c8 = 0; c8 < SEG / 8; ++c8) {
            if (active)
                load8<T>(W + row * K + col0 + 8 * c8, w);
            else
                for (int j = 0; j < 8; ++j) w[j] = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                a[8 * c8 + j] = fabsf(w[j]);
                negmask |= (uint32_t)(__builtin_signbitf(w[j]) != 0) << (8 * c8 + j);
            }
        }
    }
    double om[WEIGHTED ? SEG : 1];
    if (WEIGHTED) {
#pragma unroll
        for (int j = 0; j < SEG; ++j) om[j] = (double)h[col0 + j];
    }

    // first candidate index at which the block's amax (hence every element)
    // rounds to zero; NC if none does.  Quotients fall as s grows.
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < SEG; ++j) amax = fmaxf(amax, a[j]);
    amax = group_max<LPB>(amax);
    int lo = 0, hi = NC;  // answer in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const float2 sr = cand[mid];
        if (round_elem<EK>(quotient<SK, ONE_STEP>(amax, sr.x, sr.y)) == 0.0f)
            hi = mid;
        else
            lo = mid + 1;
    }
    const int cend = __builtin_amdgcn_readfirstlane(wave_max_int(lo < NC ? lo : NC - 1));

    double best = __builtin_huge_val();
    int best_c = 0;
    for (int c = 0; c <= cend; ++c) {
        const float2 sr = cand[c];
        double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
        for (int j = 0; j < SEG; j += 2) {
            const double d0 = (double)search_resid<EK, SK, ONE_STEP>(a[j], sr.x, sr.y);
            const double d1 = (double)search_resid<EK, SK, ONE_STEP>(a[j + 1], sr.x, sr.y);
            if (WEIGHTED) {
                acc0 = __builtin_fma(om[j], d0 * d0, acc0);
                acc1 = __builtin_fma(om[j + 1], d1 * d1, acc1);
            } else {
                acc0 = __builtin_fma(d0, d0, acc0);
                acc1 = __builtin_fma(d1, d1, acc1);
            }
        }
        const double acc = group_sum<LPB>(acc0 + acc1);
        if (acc < best) {
            best = acc;
            best_c = c;
        }
    }

    // encode the segment with the chosen scale
    const float s = cand[best_c].x, r = cand[best_c].y;
    if (!active) return;
    const int64_t e0 = row * K + col0;
#pragma unroll
    for (int c8 = 0; c8 < SEG / 8; ++c8) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = ((negmask >> (8 * c8 + j)) & 1u) ? -a[8 * c8 + j] : a[8 * c8 + j];
        uint32_t cd[8];
        encode8<EK, SK, ONE_STEP, false>(w, s, r, nullptr, cd);
        store_codes8<EK>(codes, e0 + 8 * c8, cd);
    }
    if (seg == 0) {
        const int64_t blk = row * (K / B) + blockIdx.y;
        scales[blk] = (uint8_t)(C0 + best_c);
        if (block_obj) block_obj[blk] = (float)best;
    }
}

template <int EK, int SK, typename T, int SEG, int LPB>
static hipError_t search_go(const void *W, int64_t N, int64_t K, const float *h, uint8_t *codes,
                            uint8_t *scales, float *bo, hipStream_t st)
{
    constexpr int ROWS = 256 / LPB;
    const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)(K / (SEG * LPB)));
    const T *w = static_cast<const T *>(W);
    if (h)
        search_kernel<EK, SK, T, SEG, LPB, true><<<grid, 256, 0, st>>>(w, N, K, h, codes, scales, bo);
    else
        search_kernel<EK, SK, T, SEG, LPB, false><<<grid, 256, 0, st>>>(w, N, K, h, codes, scales, bo);
    return hipGetLastError();
}

template <int EK, int SK, typename T>
static hipError_t search_b(int B, const void *W, int64_t N, int64_t K, const float *h, uint8_t *codes,
                           uint8_t *scales, float *bo, hipStream_t st)
{
    switch (B) {
    case 8: return search_go<EK, SK, T, 8, 1>(W, N, K, h, codes, scales, bo, st);
    case 16: return search_go<EK, SK, T, 16, 1>(W, N, K, h, codes, scales, bo, st);
    case 32: return search_go<EK, SK, T, 32, 1>(W, N, K, h, codes, scales, bo, st);
    case 64: return search_go<EK, SK, T, 32, 2>(W, N, K, h, codes, scales, bo, st);
    case 128: return search_go<EK, SK, T, 32, 4>(W, N, K, h, codes, scales, bo, st);
    case 256: return search_go<EK, SK, T, 32, 8>(W, N, K, h, codes, scales, bo, st);
    }
    return hipErrorInvalidValue;
}

template <int EK, int SK>
static hipError_t search_fmt(int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                             uint8_t *codes, uint8_t *scales, float *bo, hipStream_t st)
{
    return wdt == 1 ? search_b<EK, SK, bf16_t>(B, W, N, K, h, codes, scales, bo, st)
                    : search_b<EK, SK, float>(B, W, N, K, h, codes, scales, bo, st);
}

}  // namespace hd
