// outref.hip - output error of many quantisations of one W against one X
// (qwantize "Results", metric definitions: ||X Wq^T - X W^T||_F / ||X W^T||_F),
// one bf16/fp16 MFMA product per quantisation.
//
// output_reference() runs once per (X, W):
//   - Y = X W^T on the bf16 MFMA units, stored as float32 [M][N], and ||Y||^2;
//   - X' = fp16(x 2^-e_m) with one power-of-two exponent e_m per row of X,
//     chosen so the row's largest magnitude lands in [2^14, 2^15): every bf16
//     value whose scaled magnitude is at least 2^-14 (29 binades under the
//     row maximum) is exact in fp16, so X' carries X exactly in practice.
// output_error_codes() then takes the codes and scales of one quantisation:
//   - the dequantised weights become one exact 16-bit GEMM operand:
//       E2M1 / E4M3 elements: bf16(s val(q)), exact (a 4-bit-significand scale
//         times an element of at most 4 significant bits);
//       INT8: fp16(val(a8) q), the E4M3 scale value times the integer code,
//         exact in fp16 (at most 11 significant bits, |value| < 65504);
//   - D = X Wq^T - Y is formed in the epilogue: acc 2^e_m / 127 - Y for INT8
//     (Wq = fl32(fl32(val/127) q) differs from val q / 127 by two roundings,
//     2^-23 relative, far inside the metric's tolerance), acc - Y otherwise;
//   - the squares are summed in float64 per lane, per workgroup, and once more
//     in a fixed order by a one-workgroup final kernel.
//
// GEMM tiling (gfx950, v_mfma_f32_32x32x16_{bf16,f16}, wave64):
//   - workgroup tile 256 rows of X x 256 rows of the weight operand, 8 waves
//     in a 2 x 4 grid, each owning 128 x 64 outputs as 4 x 2 MFMA tiles (128
//     float accumulators per lane); two waves per SIMD, so one wave's LDS and
//     barrier waits hide behind the other's MFMAs;
//   - K is walked 64 at a time through two 64 KB LDS stages filled by
//     global_load_lds_dwordx4 (global -> LDS without registers), one stage
//     ahead of the MFMAs; the LDS image of every 128-byte row slice is
//     XOR-swizzled so the 16-byte fragment reads of 16 consecutive rows hit all
//     64 banks (no conflicts, checked with SQ_LDS_BANK_CONFLICT); the fragments
//     of the next 16-wide K slice are read while the current one multiplies;
//   - tile order: the workgroups one XCD runs at once cover 8 X tiles for each
//     weight tile, so they share X and weight panels in that XCD's L2;
//   - when the last round of tiles would fill at most half of the CUs, those
//     tiles run as 256 x 128 halves (a second launch), so that round takes
//     about half a tile's time.
#include "common.hpp"
#include "formats.hpp"
#include "kernels.hpp"

namespace hd {

typedef __bf16 ob16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 oh16x8_t __attribute__((ext_vector_type(8)));
typedef float of32x16_t __attribute__((ext_vector_type(16)));

static constexpr int GE_TM = 256;      // X rows per tile
static constexpr int GE_TN = 256;      // weight rows per full tile
static constexpr int GE_GROUP_M = 8;
#ifndef HD_GE_TK
#define HD_GE_TK 64                    // K per LDS stage (32 or 64)
#endif
#ifndef HD_GE_STAGES
#define HD_GE_STAGES 2                 // LDS stages (copies run STAGES - 1 stages ahead)
#endif
#ifndef HD_GE_WN
#define HD_GE_WN 4                     // waves along the weight rows (4: 8 waves of 128 x 64; 2: 4 of 128 x 128)
#endif

// Tile geometry for K step TK, S LDS stages, 2 x WN waves and NJ 32-wide MFMA
// tiles per wave along the weight rows (WN NJ = 8: 256 x 256 tiles; 4: the
// 256 x 128 halves).  Each wave owns 128 X rows x 32 NJ weight rows.
template <int TK, int S, int WN, int NJ>
struct GeCfg {
    static constexpr int NW = 2 * WN;                // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int TN = WN * 32 * NJ;          // weight rows of the tile
    static constexpr int CPR = TK / 8;               // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CPR;             // rows one copy instruction fills
    static constexpr int SWZ = 16 / CPR;             // consecutive rows sharing one XOR value
    static constexpr int STAGE = (GE_TM + TN) * TK;  // 16-bit elements per stage
    static constexpr int DA = GE_TM / RPI / NW;      // copy instructions per wave and stage, X tile
    static constexpr int DB = TN / RPI / NW;         // same, weight tile
    static constexpr size_t LDS = (size_t)S * STAGE * 2;
    static_assert(TK == 32 || TK == 64, "TK");
    static_assert(DA * RPI * NW == GE_TM && DB * RPI * NW == TN, "copy split");
    static_assert(LDS <= 160 * 1024, "LDS");
};

enum { GE_STORE_Y = 0, GE_SUB_Y = 1 };

template <bool F16>
struct Mfma16;
template <>
struct Mfma16<false> {
    typedef ob16x8_t v;
    static __device__ __forceinline__ of32x16_t op(v a, v b, of32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma16<true> {
    typedef oh16x8_t v;
    static __device__ __forceinline__ of32x16_t op(v a, v b, of32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// ------------------------------------------------------------------ GEMM --
// A 16-byte block of zeros in global memory: the source of every staged chunk
// that lies past K (its LDS slot must hold zeros; the copy engine cannot
// select).
__device__ __attribute__((aligned(16))) uint32_t ge_zero16[4] = {0u, 0u, 0u, 0u};

typedef __attribute__((address_space(3))) void ge_lds_void;
typedef __attribute__((address_space(1))) const void ge_gbl_void;

// s_waitcnt vmcnt(n) for a small run-time n (the copies still allowed in flight).
__device__ __forceinline__ void ge_wait_copies(int n)
{
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Tiles: the X x W product is cut into 256 x 256 tiles, numbered in a grouped
// order (GE_GROUP_M X tiles per weight tile).  A launch covers the tile
// numbers lin0 .. lin0 + nlin - 1: one workgroup per tile, with an XCD-aware
// remap of the workgroup index (consecutive workgroups go to different XCDs;
// the remap gives each XCD a contiguous run of tile numbers), or, when
// `split` is set (half-width configuration), two workgroups per tile, each
// taking 128 of its 256 weight rows (the last, partial round of tiles then
// fills twice as many CUs).
// Each workgroup computes acc = A B^T for its tile (A [M][K], B [N][K],
// 16-bit, K % 8 == 0), then
//   MODE GE_STORE_Y: Y[m][n] = acc, partial {0, sum acc^2};
//   MODE GE_SUB_Y:   d = acc f_m - Y[m][n] with f_m = fscale 2^erow[m]
//                    (f_m = 1 when erow is NULL), partial {sum d^2, 0};
// workgroup w writes its partial to part[2 (pbase + w) .. + 1].
template <bool F16, int MODE, int TK, int S, int WN, int NJ>
__global__ __launch_bounds__(128 * WN, 1) void gemm_err_kernel(const uint16_t *__restrict__ A,
                                                                 const uint16_t *__restrict__ Bm, int64_t M,
                                                                 int64_t N, int64_t K, int mt, int nt, int lin0,
                                                                 int nlin, int split, float *__restrict__ Y,
                                                                 const int *__restrict__ erow, double fscale,
                                                                 double *__restrict__ part, int pbase)
{
    typedef GeCfg<TK, S, WN, NJ> C;
    typedef typename Mfma16<F16>::v V;
    extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
    __shared__ double red[2][C::NW];

    const int hw = blockIdx.x;
    int lin, half = 0;
    if (split) {
        lin = lin0 + hw / 2;
        half = hw & 1;
    } else {
        const int per = nlin / 8;
        lin = lin0 + (hw < per * 8 ? (hw % 8) * per + hw / 8 : hw);
    }
    const int group = lin / (GE_GROUP_M * nt);
    const int first_m = group * GE_GROUP_M;
    const int gm = min(mt - first_m, GE_GROUP_M);
    const int within = lin % (GE_GROUP_M * nt);
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    const int64_t m0 = (int64_t)tm * GE_TM, n0 = (int64_t)tn * GE_TN + (int64_t)half * C::TN;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;

    // Staging: global -> LDS by global_load_lds_dwordx4 (no registers).  One
    // instruction of a wave fills 1 KB of LDS, 16 bytes per lane in lane
    // order: RPI rows of TK elements.  Lane l of the wave's i-th instruction
    // fills row r = (4 i + wv) RPI + l / CPR, slot l % CPR, and fetches the
    // 16-byte chunk c = slot ^ ((r / SWZ) % CPR) of that row: the XOR swizzle
    // spreads the 16 rows of one fragment read over all 64 banks.  Chunks past
    // K come from ge_zero16; rows past M / N are clamped to the last row
    // (their outputs are never read).
    const int lrow = lane / C::CPR, slot = lane % C::CPR;
    int64_t aoff[C::DA], boff[C::DB];
    int acs[C::DA], bcs[C::DB];
#pragma unroll
    for (int i = 0; i < C::DA; ++i) {
        const int r = (C::NW * i + wv) * C::RPI + lrow;
        acs[i] = (slot ^ ((r / C::SWZ) % C::CPR)) * 8;
        aoff[i] = min(m0 + r, M - 1) * K + acs[i];
    }
#pragma unroll
    for (int i = 0; i < C::DB; ++i) {
        const int r = (C::NW * i + wv) * C::RPI + lrow;
        bcs[i] = (slot ^ ((r / C::SWZ) % C::CPR)) * 8;
        boff[i] = min(n0 + r, N - 1) * K + bcs[i];
    }
#define GE_ISSUE(k0, buf)                                                                              \
    do {                                                                                               \
        uint16_t *sa_ = glds + (buf) * C::STAGE + wv * C::RPI * TK;                                    \
        uint16_t *sb_ = sa_ + GE_TM * TK;                                                              \
        _Pragma("unroll") for (int i = 0; i < C::DA; ++i)                                              \
        {                                                                                              \
            const void *p_ = (k0) + acs[i] < K ? (const void *)(A + aoff[i] + (k0)) : (const void *)ge_zero16; \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)p_, (ge_lds_void *)(sa_ + C::NW * i * C::RPI * TK), 16, 0, 0); \
        }                                                                                              \
        _Pragma("unroll") for (int i = 0; i < C::DB; ++i)                                              \
        {                                                                                              \
            const void *p_ = (k0) + bcs[i] < K ? (const void *)(Bm + boff[i] + (k0)) : (const void *)ge_zero16; \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)p_, (ge_lds_void *)(sb_ + C::NW * i * C::RPI * TK), 16, 0, 0); \
        }                                                                                              \
    } while (0)

    of32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Fragments of one 16-wide K slice: fa[4] (X rows), fb[NJ] (weight rows),
    // double-buffered so the next slice is read from LDS while the current one
    // multiplies.
    const int fr = lane & 31, fh = lane >> 5;
    V fa[2][4], fb[2][NJ];
#define GE_FRAG(set, bufp, kk)                                                                         \
    do {                                                                                               \
        const int c_ = 2 * (kk) + fh;                                                                  \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
        {                                                                                              \
            const int r_ = wm * 128 + i * 32 + fr;                                                     \
            fa[set][i] = *reinterpret_cast<const V *>((bufp) + r_ * TK + ((c_ ^ ((r_ / C::SWZ) % C::CPR)) * 8)); \
        }                                                                                              \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                                 \
        {                                                                                              \
            const int r_ = wn * 32 * NJ + j * 32 + fr;                                                 \
            fb[set][j] = *reinterpret_cast<const V *>((bufp) + (GE_TM + r_) * TK + ((c_ ^ ((r_ / C::SWZ) % C::CPR)) * 8)); \
        }                                                                                              \
    } while (0)

    // Pipeline: the copies of stage ks + S - 1 are issued right after the
    // barrier that opens stage ks (that barrier also certifies that every wave
    // has finished reading the buffer they overwrite, the one of stage ks - 1).
    // Before the barrier each wave waits for its own copies of stage ks (the
    // copies of later stages may stay in flight) and for its LDS reads.
    const int ksteps = (int)((K + TK - 1) / TK);
    constexpr int D = C::DA + C::DB;
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        if (p < ksteps) GE_ISSUE((int64_t)p * TK, p);
    for (int ks = 0; ks < ksteps; ++ks) {
        ge_wait_copies(min(S - 2, ksteps - 1 - ks) * D);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (ks + S - 1 < ksteps) GE_ISSUE((int64_t)(ks + S - 1) * TK, (ks + S - 1) % S);
        const uint16_t *base = glds + (ks % S) * C::STAGE;
        GE_FRAG(0, base, 0);
#pragma unroll
        for (int kk = 0; kk < TK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < TK / 16) GE_FRAG(cur ^ 1, base, kk + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = Mfma16<F16>::op(fa[cur][i], fb[cur][j], acc[i][j]);
        }
    }
#undef GE_FRAG
#undef GE_ISSUE

    // epilogue: accumulator v of lane l in a 32 x 32 tile is row
    // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
    double sd = 0.0, sy = 0.0;
    const int64_t nb0 = n0 + wn * 32 * NJ + (lane & 31);
    const int64_t mb0 = m0 + wm * 128 + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // row exponents of this lane's 16 rows in tile row i (SUB with erow)
        int ev[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            ev[v] = (MODE == GE_SUB_Y && erow != nullptr) ? erow[min(mb0 + i * 32 + 8 * (v >> 2) + (v & 3), M - 1)] : 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = nb0 + j * 32;
            const bool nin = n < N;
            if (MODE == GE_STORE_Y) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = mb0 + i * 32 + 8 * (v >> 2) + (v & 3);
                    if (m < M && nin) {
                        const float a = acc[i][j][v];
                        Y[m * N + n] = a;
                        sy = __builtin_fma((double)a, (double)a, sy);
                    }
                }
            } else {
                // the 16 reads of Y for this 32 x 32 tile are in flight together
                const int64_t nc = min(n, N - 1);
                float yv[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) yv[v] = Y[min(mb0 + i * 32 + 8 * (v >> 2) + (v & 3), M - 1) * N + nc];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = mb0 + i * 32 + 8 * (v >> 2) + (v & 3);
                    const double f = ldexp(fscale, ev[v]);
                    const double d = (double)acc[i][j][v] * f - (double)yv[v];
                    sd = (m < M && nin) ? __builtin_fma(d, d, sd) : sd;
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        sd += __shfl_xor(sd, o, 64);
        sy += __shfl_xor(sy, o, 64);
    }
    if (lane == 0) {
        red[0][wv] = sd;
        red[1][wv] = sy;
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0, b = 0.0;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) {
            a += red[0][w];
            b += red[1][w];
        }
        part[2 * (int64_t)(pbase + hw)] = a;
        part[2 * (int64_t)(pbase + hw) + 1] = b;
    }
}

// ------------------------------------------------ X -> X' (fp16, row 2^e) --
// One workgroup per row of bf16 X: e_m = floor(log2 max_k |x_mk|) - 14 (0 for
// a zero row), X'[m][k] = fp16(x_mk 2^-e_m), round-to-nearest-even.
__global__ __launch_bounds__(256) void xprep_kernel(const bf16_t *__restrict__ X, int64_t K,
                                                    uint16_t *__restrict__ Xh, int *__restrict__ erow)
{
    __shared__ int shm[4];
    const int64_t m = blockIdx.x;
    const bf16_t *row = X + m * K;
    const int64_t nch = K / 8;
    uint32_t mx = 0;  // largest |x| as bf16 magnitude bits (monotone for finite values)
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = max(mx, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    mx = (uint32_t)wave_max_int((int)mx);
    if ((threadIdx.x & 63) == 0) shm[threadIdx.x >> 6] = (int)mx;
    __syncthreads();
    mx = (uint32_t)max(max(shm[0], shm[1]), max(shm[2], shm[3]));
    int e = 0;
    if (mx != 0) {
        int ex;
        frexpf(bf16_to_f32(mx), &ex);  // max = f 2^ex, f in [0.5, 1)
        e = ex - 1 - 14;
    }
    if (threadIdx.x == 0) erow[m] = e;
    uint16_t *orow = Xh + m * K;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w[j] & 0xFFFFu), -e);
            const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w[j] >> 16), -e);
            o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4 *>(orow + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// --------------------------------------------- codes -> 16-bit GEMM operand --
// INT8: fp16(val(a8) q) (exact); E2M1 / E4M3 elements: bf16(s val(q)) (exact).
// Invalid codes decode to 0, as dequantize() does.
template <int EK, int SK>
__global__ __launch_bounds__(256) void operand_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int64_t total, int B,
                                                      uint16_t *__restrict__ out)
{
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e0 >= total) return;
    const int sc = scales[e0 / B];
    // INT8 carries the E4M3 value of the scale code; 1/127 goes to the epilogue
    const float s = !scale_code_valid(SK, sc) ? 0.0f : (EK == ELEM_INT8 ? e4m3_value(sc) : scale_value(SK, sc));
    uint32_t c[8];
    if (elem_4bit(EK)) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(codes + e0 / 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (v >> (4 * j)) & 15u;
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(codes + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = (v.x >> (8 * j)) & 255u;
            c[4 + j] = (v.y >> (8 * j)) & 255u;
        }
    }
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (EK == ELEM_INT8) {
            const int q = (int)(int8_t)(uint8_t)c[j];
            const float f = q == -128 ? 0.0f : s * (float)q;  // exact: <= 11 significant bits
            o[j] = __builtin_bit_cast(uint16_t, (_Float16)f);
        } else if (EK == ELEM_INT4) {
            const int q = (int)((c[j] ^ 8u) & 15u) - 8;        // two's complement nibble
            o[j] = f32_to_bf16(q == -8 ? 0.0f : s * (float)q);  // exact: <= 7 significant bits
        } else {
            bool neg, ok = true;
            uint32_t idx;
            if (EK == ELEM_E2M1) {
                neg = (c[j] & 8u) != 0;
                idx = c[j] & 7u;
            } else {
                neg = (c[j] & 0x80u) != 0;
                idx = c[j] & 0x7Fu;
                ok = idx != 0x7Fu;
            }
            const float mag = ok ? s * elem_value<EK>(idx) : 0.0f;
            o[j] = f32_to_bf16(neg ? -mag : mag);
        }
    }
    *reinterpret_cast<uint4 *>(out + e0) =
        make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16));
}

// ------------------------------------------------------------ final sums --
// Fixed-order sum of the workgroup partials.  ysq == NULL: store the sum of
// part[.][1] to *ysq_out (the reference's ||Y||^2).  Otherwise
// *out = sqrt(sum part[.][0]) / sqrt(*ysq) and sums = {sum D^2, *ysq}.
__global__ __launch_bounds__(256) void outref_final(const double *__restrict__ part, int64_t n,
                                                    const double *__restrict__ ysq, double *__restrict__ ysq_out,
                                                    double *__restrict__ out, double *__restrict__ sums)
{
    __shared__ double sh[4];
    double a = 0.0, b = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
        a += part[2 * i];
        b += part[2 * i + 1];
    }
    a = block_sum_256(a, sh);
    b = block_sum_256(b, sh);
    if (threadIdx.x == 0) {
        if (ysq == nullptr) {
            *ysq_out = b;
        } else {
            const double y = *ysq;
            *out = sqrt(a) / sqrt(y);
            if (sums) {
                sums[0] = a;
                sums[1] = y;
            }
        }
    }
}

// ---------------------------------------------------------------- layout --
static int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }
static int64_t ge_tiles(int64_t M, int64_t N) { return ((M + GE_TM - 1) / GE_TM) * ((N + GE_TN - 1) / GE_TN); }
static int64_t ge_parts(int64_t M, int64_t N) { return ge_tiles(M, N) + 1024; }  // tiles + split halves

RefLayout output_reference_layout(int64_t M, int64_t N, int64_t K)
{
    RefLayout L;
    L.y = 256;
    L.e = L.y + al256(M * N * 4);
    L.x = L.e + al256(M * 4);
    L.part = L.x + al256(M * K * 2);
    L.bytes = L.part + al256(ge_parts(M, N) * 16);
    return L;
}

size_t output_error_codes_ws(int64_t M, int64_t N, int64_t K)
{
    return (size_t)(al256(N * K * 2) + al256(ge_parts(M, N) * 16));
}

// CUs of the current device (cached per device).
static int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Launch plan: T full tiles on `cus` CUs run in ceil(T / cus) rounds; when
// the last round would fill at most half of the CUs, its tiles run as
// 256 x 128 halves instead (the round then takes half a tile's time).
// Returns the number of workgroup partials written.
template <bool F16, int MODE>
static hipError_t launch_gemm_err(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K,
                                  float *Y, const int *erow, double fscale, double *part, int64_t *nparts,
                                  hipStream_t st)
{
    constexpr int TK = HD_GE_TK, S = HD_GE_STAGES, WN = HD_GE_WN, NJF = 8 / WN, NJH = 4 / WN;
    typedef GeCfg<TK, S, WN, NJF> CF;
    typedef GeCfg<TK, S, WN, NJH> CH;
    static_assert(CF::TN == GE_TN && 2 * CH::TN == GE_TN, "tile widths");
    const int mt = (int)((M + GE_TM - 1) / GE_TM), nt = (int)((N + GE_TN - 1) / GE_TN);
    const int64_t T = (int64_t)mt * nt;
    *nparts = 0;
    if (T == 0) return hipSuccess;
    const int cus = device_cus();
    const int64_t rem = T % cus;
    const bool split = rem > 0 && 2 * rem <= cus;
    const int64_t nfull = split ? T - rem : T;
    hipError_t e;
    if (nfull > 0) {
        e = hipFuncSetAttribute((const void *)gemm_err_kernel<F16, MODE, TK, S, WN, NJF>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)CF::LDS);
        if (e != hipSuccess) return e;
        gemm_err_kernel<F16, MODE, TK, S, WN, NJF><<<(unsigned)nfull, CF::THREADS, CF::LDS, st>>>(
            A, Bm, M, N, K, mt, nt, 0, (int)nfull, 0, Y, erow, fscale, part, 0);
    }
    if (split) {
        e = hipFuncSetAttribute((const void *)gemm_err_kernel<F16, MODE, TK, S, WN, NJH>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)CH::LDS);
        if (e != hipSuccess) return e;
        gemm_err_kernel<F16, MODE, TK, S, WN, NJH><<<(unsigned)(2 * rem), CH::THREADS, CH::LDS, st>>>(
            A, Bm, M, N, K, mt, nt, (int)nfull, (int)rem, 1, Y, erow, fscale, part, (int)nfull);
    }
    *nparts = nfull + (split ? 2 * rem : 0);
    return hipGetLastError();
}

// Y = A B^T in float32 for 16-bit bf16 operands A [M][K], B [N][K] (K % 8 == 0),
// with `part` holding ge_parts(M, N) pairs of doubles of scratch.
int64_t output_gemm_parts_bytes(int64_t M, int64_t N) { return ge_parts(M, N) * 2 * 8; }
hipError_t launch_gemm_store(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K, float *Y,
                             double *part, hipStream_t st)
{
    int64_t np = 0;
    return launch_gemm_err<false, GE_STORE_Y>(A, Bm, M, N, K, Y, nullptr, 1.0, part, &np, st);
}

hipError_t launch_output_reference(const void *X, int64_t M, const void *W, int64_t N, int64_t K, void *ref,
                                   hipStream_t st)
{
    const RefLayout L = output_reference_layout(M, N, K);
    char *r = static_cast<char *>(ref);
    double *ysq = reinterpret_cast<double *>(r);
    float *Y = reinterpret_cast<float *>(r + L.y);
    int *erow = reinterpret_cast<int *>(r + L.e);
    uint16_t *Xh = reinterpret_cast<uint16_t *>(r + L.x);
    double *part = reinterpret_cast<double *>(r + L.part);
    if (M > 0 && K > 0) xprep_kernel<<<(unsigned)M, 256, 0, st>>>((const bf16_t *)X, K, Xh, erow);
    int64_t np = 0;
    hipError_t e = launch_gemm_err<false, GE_STORE_Y>((const uint16_t *)X, (const uint16_t *)W, M, N, K, Y, nullptr,
                                                      1.0, part, &np, st);
    if (e != hipSuccess) return e;
    outref_final<<<1, 256, 0, st>>>(part, np, nullptr, ysq, nullptr, nullptr);
    return hipGetLastError();
}

template <int EK, int SK>
static void launch_operand(const uint8_t *codes, const uint8_t *scales, int64_t total, int B, uint16_t *out,
                           hipStream_t st)
{
    const unsigned g = (unsigned)((total / 8 + 255) / 256);
    operand_kernel<EK, SK><<<g, 256, 0, st>>>(codes, scales, total, B, out);
}

hipError_t launch_output_error_codes(int fmt, int B, const void *X, int64_t M, const uint8_t *codes,
                                     const uint8_t *scales, int64_t N, int64_t K, const void *ref, double *out,
                                     double *sums, void *ws, hipStream_t st)
{
    const RefLayout L = output_reference_layout(M, N, K);
    const char *r = static_cast<const char *>(ref);
    const double *ysq = reinterpret_cast<const double *>(r);
    float *Y = const_cast<float *>(reinterpret_cast<const float *>(r + L.y));
    const int *erow = reinterpret_cast<const int *>(r + L.e);
    const uint16_t *Xh = reinterpret_cast<const uint16_t *>(r + L.x);
    char *w = static_cast<char *>(ws);
    uint16_t *opnd = reinterpret_cast<uint16_t *>(w);
    double *part = reinterpret_cast<double *>(w + al256(N * K * 2));
    const int64_t total = N * K;
    hipError_t e = hipSuccess;
    if (total > 0) {
        switch (fmt) {
        case HD_INT8_E4M3: launch_operand<ELEM_INT8, SCALE_INT8>(codes, scales, total, B, opnd, st); break;
        case HD_NVFP4: launch_operand<ELEM_E2M1, SCALE_E4M3>(codes, scales, total, B, opnd, st); break;
        case HD_MXFP4: launch_operand<ELEM_E2M1, SCALE_E8M0>(codes, scales, total, B, opnd, st); break;
        case HD_MXFP8: launch_operand<ELEM_E4M3, SCALE_E8M0>(codes, scales, total, B, opnd, st); break;
        case HD_FP8_E4M3S: launch_operand<ELEM_E4M3, SCALE_E4M3>(codes, scales, total, B, opnd, st); break;
        case HD_NVFP4_UE4M4: launch_operand<ELEM_E2M1, SCALE_UE4M4>(codes, scales, total, B, opnd, st); break;
        case HD_NVFP4_UE5M3: launch_operand<ELEM_E2M1, SCALE_UE5M3>(codes, scales, total, B, opnd, st); break;
        case HD_NVINT4: launch_operand<ELEM_INT4, SCALE_E4M3>(codes, scales, total, B, opnd, st); break;
        default: return hipErrorInvalidValue;
        }
    }
    int64_t np = 0;
    if (fmt == HD_INT8_E4M3)
        e = launch_gemm_err<true, GE_SUB_Y>(Xh, opnd, M, N, K, Y, erow, 1.0 / 127.0, part, &np, st);
    else
        e = launch_gemm_err<false, GE_SUB_Y>((const uint16_t *)X, opnd, M, N, K, Y, nullptr, 1.0, part, &np, st);
    if (e != hipSuccess) return e;
    outref_final<<<1, 256, 0, st>>>(part, np, ysq, nullptr, out, sums);
    return hipGetLastError();
}

}  // namespace hd
