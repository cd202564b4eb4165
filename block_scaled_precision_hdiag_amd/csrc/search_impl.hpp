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
// Mapping (the work is VALU bound: about 10 to 13 instructions per weight and
// evaluated candidate):
//   - one lane owns one block segment of SEG weights held in registers (32,
//     or 16 for the weighted search, which also holds h); a block of B > SEG
//     spans LPB = B / SEG adjacent lanes whose partial objectives are combined
//     with lane shuffles;
//   - all lanes of a workgroup share one block column (so h_j is the same for
//     every lane of a wave and is loaded once) and walk the candidates in
//     lock-step, reading each candidate's (s, 1/s) from an LDS table; the
//     running argmin is per lane and needs no cross-lane reduction;
//   - each residual is formed in fp32 and squared / accumulated in float64.
//     It is exact (Sterbenz) for every element that does not saturate, and
//     for elements that encode to zero; for a saturated element
//     (a > 2 fl32(Q s)) the fp32 subtraction rounds once, at most 2^-24
//     relative, so the objective of a candidate that clips is within 2^-23
//     relative of its exact value (the oracle subtracts in float64).  A block
//     whose choice this could move has two candidates within 2^-23 of each
//     other, inside the 1e-6 tie tolerance of the parity bar;
//   - candidates at and above the first scale that rounds the block's amax to
//     zero all give sum_j om_j w_j^2 (every element encodes to 0): they could
//     only tie, and ties keep the lower code, so they are never evaluated;
//   - each lane walks candidate offsets from its own block's Naive code, so
//     the rows of different magnitude that share a wave share offsets, not
//     codes (measured: 1.5-1.9x faster than walking common codes, which also
//     used the gfx950 FP4/FP8 conversions for two weights at a time); the
//     window widens only while some lane cannot prove the candidates outside
//     it strictly worse than its best so far: below it every element above
//     fl32(Q s) saturates (sat_lower_bound), above it every element
//     a <= v1 s stays at code 0 or v1 (small_lower_bound; v1 the smallest
//     positive element).  Both bounds hold for the objective as the kernel
//     computes it, so the chosen code is the one the full scan picks.  For
//     E4M3 elements v1 = 2^-9 makes the upper bound void: their error is
//     nearly scale invariant and the scan runs to the zero tail.
#pragma once
#include "encode.hpp"
#include "kernels.hpp"

namespace hd {

// Lower bound, valid for every candidate scale s' <= s, of the objective the
// kernel computes: an element with a > fl32(Q s) saturates at every s' <= s
// (fl32(a / s') >= Q), its dequantised value is at most fl32(Q s'), and the
// fp32 residual is >= (a - fl32(Q s)) (1 - 2^-24); the other elements add
// >= 0.  The bound is summed in float64 from exact differences, so
// LB (1 - 2^-20) > best proves every such candidate strictly worse.
template <int EK, int SEG, int LPB, bool WEIGHTED>
__device__ __forceinline__ double sat_lower_bound(const float *a, const double *om, float s)
{
    const float qs = elem_max(EK) * s;  // fl32(Q s): what a saturated element dequantises to
    double lb = 0.0;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        double t = (double)a[j] - (double)qs;
        t = t > 0.0 ? t : 0.0;
        lb += (WEIGHTED ? om[j] : 1.0) * (t * t);
    }
    return group_sum<LPB>(lb);
}

// Lower bound, valid for every candidate scale s' >= s, of the objective the
// kernel computes, for element grids whose smallest positive value v1 (INT8,
// INT4: 1; E2M1: 0.5) is at most half the next one: an element with
// a <= v1 s has a / s' <= v1, so it encodes to 0 (residual a) or to v1
// (residual v1 s' - a >= v1 s - a, exact in fp32 by Sterbenz's lemma); it adds
// >= om min(a, v1 s - a)^2, the others >= 0.  (For a < v1 s / 2 this is the
// zero-code term a^2; the other branch also bounds the elements at v1.)
template <int EK, int SEG, int LPB, bool WEIGHTED>
__device__ __forceinline__ double small_lower_bound(const float *a, const double *om, float s)
{
    const double sd = (double)elem_min_pos(EK) * (double)s;
    double lb = 0.0;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        const double aj = (double)a[j];
        const double t = aj <= sd ? fmin(aj, sd - aj) : 0.0;
        lb += (WEIGHTED ? om[j] : 1.0) * (t * t);
    }
    return group_sum<LPB>(lb);
}

// true on every lane when no active lane needs more candidates
__device__ __forceinline__ bool wave_all(bool p) { return __ballot(!p) == 0; }

template <int EK, int SK, bool ONE_STEP>
__device__ __forceinline__ float search_resid(float a, float s, float r)
{
    const float x = quotient<SK, ONE_STEP>(a, s, r);
    const float y = round_elem<EK>(x);
    if (elem_int(EK)) {
        const float wq = s * y;  // fl32(s * q): INT8 scales carry a full fp32 mantissa
        return a - wq;
    }
    // E2M1 / E4M3 grid values times an E4M3 or power-of-two scale are exact
    // products, so this single-rounding FMA equals a - fl32(s * y).
    return __builtin_fmaf(-y, s, a);
}

// evals (optional): the kernel adds the number of (weight, candidate) pairs it
// evaluated, counting the weights of active lanes only (one atomic per wave).
template <int EK, int SK, typename T, int SEG, int LPB, bool WEIGHTED>
__global__ __launch_bounds__(256) void search_kernel(const T *__restrict__ W, int64_t N, int64_t K,
                                                     const float *__restrict__ h, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, float *__restrict__ block_obj,
                                                     unsigned long long *__restrict__ evals)
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
    // every candidate from cendl on gives sum om a^2 (all elements encode to 0)
    const int cendl = lo < NC ? lo : NC - 1;
    // the lane's Naive candidate: each lane walks offsets from its own Naive
    // code, so rows of different magnitude in one wave share the offsets, not
    // the codes
    const int cb = min(max(naive_code<EK, SK>(amax) - C0, 0), cendl);

    double best = __builtin_huge_val();
    int best_c = 0;
    // evaluate offsets o0..o1 from cb; indices are clamped to [0, cendl]:
    // a repeated candidate cannot change the argmin (ties keep the lower code)
    auto eval_range = [&](int o0, int o1) {
        for (int o = o0; o <= o1; ++o) {
            const int c = min(max(cb + o, 0), cendl);
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
            if (acc < best || (acc == best && c < best_c)) {
                best = acc;
                best_c = c;
            }
        }
    };
    // INT8: start one code below Naive to one binade above it (where the
    // optimum lies for nearly every block); the other grids: half a binade
    // below to one binade above.  Widen by SEARCH_STEP codes while some lane
    // cannot prove the candidates beyond its window strictly worse than its
    // best so far (above: small_lower_bound; below: sat_lower_bound)
    constexpr int CPB = codes_per_binade(SK);
    constexpr int SEARCH_STEP = CPB > 8 ? CPB / 2 : 4;
    int olo = EK == ELEM_INT8 ? -1 : -CPB / 2, ohi = CPB;
    eval_range(olo, ohi);
    for (;;) {
        const int c1 = cb + ohi + 1;
        const double lb = small_lower_bound<EK, SEG, LPB, WEIGHTED>(a, om, cand[min(c1, NC - 1)].x);
        const bool need = active && c1 <= cendl && !(lb * (1.0 - 0x1p-20) > best);
        if (wave_all(!need)) break;
        eval_range(ohi + 1, ohi + SEARCH_STEP);
        ohi += SEARCH_STEP;
    }
    for (;;) {
        const int c1 = cb + olo - 1;
        const double lb = sat_lower_bound<EK, SEG, LPB, WEIGHTED>(a, om, cand[max(c1, 0)].x);
        const bool need = active && c1 >= 0 && !(lb * (1.0 - 0x1p-20) > best);
        if (wave_all(!need)) break;
        eval_range(olo - SEARCH_STEP, olo - 1);
        olo -= SEARCH_STEP;
    }

    if (evals != nullptr) {
        // the wave evaluated offsets olo..ohi for each active lane's SEG weights
        const unsigned long long nact = (unsigned long long)__popcll(__ballot(active));
        if ((tid & 63) == 0) atomicAdd(evals, (unsigned long long)(ohi - olo + 1) * nact * SEG);
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
                            uint8_t *scales, float *bo, unsigned long long *ev, hipStream_t st)
{
    constexpr int ROWS = 256 / LPB;
    const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)(K / (SEG * LPB)));
    const T *w = static_cast<const T *>(W);
    // (SEG, LPB) = (32, *) serves only the unweighted search, (16, > 1) only the weighted one
    constexpr bool MAY_W = SEG <= 16, MAY_U = !(SEG == 16 && LPB > 1);
    if constexpr (MAY_W) {
        if (h) {
            search_kernel<EK, SK, T, SEG, LPB, true><<<grid, 256, 0, st>>>(w, N, K, h, codes, scales, bo, ev);
            return hipGetLastError();
        }
    }
    if constexpr (MAY_U)
        search_kernel<EK, SK, T, SEG, LPB, false><<<grid, 256, 0, st>>>(w, N, K, h, codes, scales, bo, ev);
    return hipGetLastError();
}

// Lane segments: 32 weights, or 16 when the float64 weights h_j also live in
// registers (so the H kernels keep two waves per SIMD).
template <int EK, int SK, typename T>
static hipError_t search_b(int B, const void *W, int64_t N, int64_t K, const float *h, uint8_t *codes,
                           uint8_t *scales, float *bo, unsigned long long *ev, hipStream_t st)
{
    if (h) {
        switch (B) {
        case 8: return search_go<EK, SK, T, 8, 1>(W, N, K, h, codes, scales, bo, ev, st);
        case 16: return search_go<EK, SK, T, 16, 1>(W, N, K, h, codes, scales, bo, ev, st);
        case 32: return search_go<EK, SK, T, 16, 2>(W, N, K, h, codes, scales, bo, ev, st);
        case 64: return search_go<EK, SK, T, 16, 4>(W, N, K, h, codes, scales, bo, ev, st);
        case 128: return search_go<EK, SK, T, 16, 8>(W, N, K, h, codes, scales, bo, ev, st);
        case 256: return search_go<EK, SK, T, 16, 16>(W, N, K, h, codes, scales, bo, ev, st);
        }
        return hipErrorInvalidValue;
    }
    switch (B) {
    case 8: return search_go<EK, SK, T, 8, 1>(W, N, K, h, codes, scales, bo, ev, st);
    case 16: return search_go<EK, SK, T, 16, 1>(W, N, K, h, codes, scales, bo, ev, st);
    case 32: return search_go<EK, SK, T, 32, 1>(W, N, K, h, codes, scales, bo, ev, st);
    case 64: return search_go<EK, SK, T, 32, 2>(W, N, K, h, codes, scales, bo, ev, st);
    case 128: return search_go<EK, SK, T, 32, 4>(W, N, K, h, codes, scales, bo, ev, st);
    case 256: return search_go<EK, SK, T, 32, 8>(W, N, K, h, codes, scales, bo, ev, st);
    }
    return hipErrorInvalidValue;
}

template <int EK, int SK>
static hipError_t search_fmt(int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                             uint8_t *codes, uint8_t *scales, float *bo, unsigned long long *ev, hipStream_t st)
{
    return wdt == 1 ? search_b<EK, SK, bf16_t>(B, W, N, K, h, codes, scales, bo, ev, st)
                    : search_b<EK, SK, float>(B, W, N, K, h, codes, scales, bo, ev, st);
}

}  // namespace hd
