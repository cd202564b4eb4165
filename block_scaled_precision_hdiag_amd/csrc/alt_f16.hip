// alt_f16.hip - SSE-Optimal / H-Optimal binary16 (FP16 E5M10) block scales by
// alternation (qwantize "Results", "Larger blocks: bs=64 (E4M3 scales) and
// bs=128 (FP16 scales)": the page finds the per-block FP16 scale by
// alternating q -> closed-form continuous s -> FP16 snap instead of a search).
//
// For a fixed element assignment q the objective sum_j om_j (w_j - s q_j)^2 is
// a quadratic in s with its minimum at s* = sum om w q / sum om q^2.  From the
// Naive scale, each round encodes the block at the current scale (which gives
// its objective and the two sums of s*), snaps s* to binary16 and moves there.
// The walk stops at a fixed point, when every om_j q_j^2 is 0, at the zero
// scale, or after ALT_MAX_ROUNDS moves; the block keeps the visited scale with
// the smallest objective, the earliest on ties (so never worse than Naive).
//
// Mapping: as the grid search - one lane per block segment of SEG weights in
// registers, LPB = B / SEG lanes per block combined with shuffles, all lanes
// of a workgroup on one block column so the h_j are shared.  Arithmetic:
//   - fl32(|w| / s) by the corrected reciprocal quotient (both corrections),
//     rounded onto the element grid as in encode;
//   - s |q| is exact in fp32 (11 + 3 significant bits), and the residual
//     |w| - s |q| is formed in float64 from those two fp32 values, so each
//     squared residual is the one the definition gives;
//   - om |w| |q| and om q^2 are exact float64 products (24 + 24 + 3 bits), so
//     the sums of s* carry only float64 addition rounding.
// Lanes whose block has stopped keep running the rounds of the rest of their
// wave (the shuffles need every lane) without changing their result.
#include "encode.hpp"
#include "kernels.hpp"

namespace hd {

static constexpr int ALT_MAX_ROUNDS = 32;

// true on every lane when p holds on every lane of the wave
__device__ __forceinline__ bool alt_wave_all(bool p) { return __ballot(!p) == 0; }

template <int EK, typename T, int SEG, int LPB, bool WEIGHTED>
__global__ __launch_bounds__(256) void alt_f16_kernel(const T *__restrict__ W, int64_t N, int64_t K,
                                                      const float *__restrict__ h, uint8_t *__restrict__ codes,
                                                      uint16_t *__restrict__ scales, float *__restrict__ block_obj)
{
    constexpr int B = SEG * LPB;
    constexpr int ROWS = 256 / LPB;
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * ROWS + tid / LPB;
    const int seg = tid % LPB;
    const int64_t col0 = (int64_t)blockIdx.y * B + (int64_t)seg * SEG;
    const bool active = row < N;  // the same for every lane of a block

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

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < SEG; ++j) amax = fmaxf(amax, a[j]);
    amax = group_max<LPB>(amax);

    int code = naive_code<EK, SCALE_F16>(amax);
    int best_code = code, moves = 0;
    double best = 0.0;
    bool done = !active, first = true;
    for (;;) {
        const float s = scale_value(SCALE_F16, code);
        const float r = s != 0.0f ? 1.0f / s : 0.0f;  // IEEE division
        double obj = 0.0, num = 0.0, den = 0.0;
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            const float x = s != 0.0f ? quotient<SCALE_F16, false>(a[j], s, r) : 0.0f;
            const float y = round_elem<EK>(x);
            const double d = (double)a[j] - (double)(s * y);
            const double o = WEIGHTED ? om[j] : 1.0;
            obj += o * (d * d);
            num += (o * (double)a[j]) * (double)y;
            den += (o * (double)y) * (double)y;
        }
        obj = group_sum<LPB>(obj);
        num = group_sum<LPB>(num);
        den = group_sum<LPB>(den);
        if (!done) {
            if (first || obj < best) {
                best = obj;
                best_code = code;
            }
            if (code == 0 || moves == ALT_MAX_ROUNDS || den == 0.0) {
                done = true;
            } else {
                const int next = f16_round_code(num / den);
                if (next == code) {
                    done = true;
                } else {
                    code = next;
                    ++moves;
                }
            }
        }
        first = false;
        if (alt_wave_all(done)) break;
    }

    if (!active) return;
    const float s = scale_value(SCALE_F16, best_code);
    const float r = s != 0.0f ? 1.0f / s : 0.0f;
    const int64_t e0 = row * K + col0;
#pragma unroll
    for (int c8 = 0; c8 < SEG / 8; ++c8) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = ((negmask >> (8 * c8 + j)) & 1u) ? -a[8 * c8 + j] : a[8 * c8 + j];
        uint32_t cd[8];
        encode8<EK, SCALE_F16, false, false>(w, s, r, nullptr, cd);
        store_codes8<EK>(codes, e0 + 8 * c8, cd);
    }
    if (seg == 0) {
        const int64_t blk = row * (K / B) + blockIdx.y;
        scales[blk] = (uint16_t)best_code;
        if (block_obj) block_obj[blk] = (float)best;
    }
}

template <int EK, typename T, int SEG, int LPB, bool WEIGHTED>
static hipError_t alt_go(const void *W, int64_t N, int64_t K, const float *h, uint8_t *codes, uint8_t *scales,
                         float *bo, hipStream_t st)
{
    constexpr int ROWS = 256 / LPB;
    const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)(K / (SEG * LPB)));
    alt_f16_kernel<EK, T, SEG, LPB, WEIGHTED><<<grid, 256, 0, st>>>(
        static_cast<const T *>(W), N, K, h, codes, reinterpret_cast<uint16_t *>(scales), bo);
    return hipGetLastError();
}

// Lane segments as in the grid search: 32 weights, 16 when the float64 h_j
// also live in registers.
template <int EK, typename T>
static hipError_t alt_b(int B, const void *W, int64_t N, int64_t K, const float *h, uint8_t *codes,
                        uint8_t *scales, float *bo, hipStream_t st)
{
    if (h) {
        switch (B) {
        case 8: return alt_go<EK, T, 8, 1, true>(W, N, K, h, codes, scales, bo, st);
        case 16: return alt_go<EK, T, 16, 1, true>(W, N, K, h, codes, scales, bo, st);
        case 32: return alt_go<EK, T, 16, 2, true>(W, N, K, h, codes, scales, bo, st);
        case 64: return alt_go<EK, T, 16, 4, true>(W, N, K, h, codes, scales, bo, st);
        case 128: return alt_go<EK, T, 16, 8, true>(W, N, K, h, codes, scales, bo, st);
        case 256: return alt_go<EK, T, 16, 16, true>(W, N, K, h, codes, scales, bo, st);
        }
        return hipErrorInvalidValue;
    }
    switch (B) {
    case 8: return alt_go<EK, T, 8, 1, false>(W, N, K, h, codes, scales, bo, st);
    case 16: return alt_go<EK, T, 16, 1, false>(W, N, K, h, codes, scales, bo, st);
    case 32: return alt_go<EK, T, 32, 1, false>(W, N, K, h, codes, scales, bo, st);
    case 64: return alt_go<EK, T, 32, 2, false>(W, N, K, h, codes, scales, bo, st);
    case 128: return alt_go<EK, T, 32, 4, false>(W, N, K, h, codes, scales, bo, st);
    case 256: return alt_go<EK, T, 32, 8, false>(W, N, K, h, codes, scales, bo, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_alt_f16(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                          uint8_t *codes, uint8_t *scales, float *block_obj, hipStream_t st)
{
    if (fmt == HD_FP4_F16)
        return wdt == 1 ? alt_b<ELEM_E2M1, bf16_t>(B, W, N, K, h, codes, scales, block_obj, st)
                        : alt_b<ELEM_E2M1, float>(B, W, N, K, h, codes, scales, block_obj, st);
    if (fmt == HD_INT4_F16)
        return wdt == 1 ? alt_b<ELEM_INT4, bf16_t>(B, W, N, K, h, codes, scales, block_obj, st)
                        : alt_b<ELEM_INT4, float>(B, W, N, K, h, codes, scales, block_obj, st);
    return hipErrorInvalidValue;
}

}  // namespace hd
