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
//   - 256 threads = 4 waves in a 2 x 2 grid; workgroup tile 256 rows of X x
//     256 rows of the weight operand; each wave owns 128 x 128 outputs as
//     4 x 4 MFMA tiles (256 float accumulators per lane), so every 16-B LDS
//     fragment read feeds four MFMAs;
//   - K is walked 64 at a time through two LDS stages (144 KB, dynamic): the
//     global loads for step k+1 are in flight while step k multiplies; LDS rows
//     are padded to 144 bytes so the 16-byte fragment reads of 16 consecutive
//     rows hit distinct banks;
//   - tile order: the workgroups one XCD runs at once cover 8 X tiles for each
//     weight tile, so they share X and W panels in that XCD's L2.
#include "common.hpp"
#include "formats.hpp"
#include "kernels.hpp"

namespace hd {

typedef __bf16 ob16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 oh16x8_t __attribute__((ext_vector_type(8)));
typedef float of32x16_t __attribute__((ext_vector_type(16)));

static constexpr int GE_TM = 256;      // X rows per tile
static constexpr int GE_TN = 256;      // weight rows per tile
static constexpr int GE_TK = 64;       // K per LDS stage
static constexpr int GE_THREADS = 256;
static constexpr int GE_GROUP_M = 8;
static constexpr int GE_STAGE = (GE_TM + GE_TN) * GE_TK;  // 16-bit elements per LDS stage
static constexpr size_t GE_LDS = 2 * (size_t)GE_STAGE * 2;

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
// acc = A B^T for one 256 x 256 tile (A [M][K], B [N][K], 16-bit, K % 8 == 0),
// then MODE GE_STORE_Y: Y[m][n] = acc, part = {0, sum acc^2};
//      MODE GE_SUB_Y:   d = acc f_m - Y[m][n] with f_m = 2^erow[m] * fscale
//                       (f_m = 1 when erow is NULL), part = {sum d^2, 0}.
// A 16-byte block of zeros in global memory: the source of every staged chunk
// that lies past K (its LDS slot must hold zeros; the copy engine cannot
// select).
__device__ __attribute__((aligned(16))) uint32_t ge_zero16[4] = {0u, 0u, 0u, 0u};

typedef __attribute__((address_space(3))) void ge_lds_void;
typedef __attribute__((address_space(1))) const void ge_gbl_void;

template <bool F16, int MODE>
__global__ __launch_bounds__(GE_THREADS, 1) void gemm_err_kernel(const uint16_t *__restrict__ A,
                                                                 const uint16_t *__restrict__ Bm, int64_t M,
                                                                 int64_t N, int64_t K, int mt, int nt,
                                                                 float *__restrict__ Y,
                                                                 const int *__restrict__ erow, double fscale,
                                                                 double *__restrict__ part)
{
    typedef typename Mfma16<F16>::v V;
    extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
    __shared__ double red[2][4];

    // tile index: XCD-aware remap, then GE_GROUP_M X tiles per weight tile
    const int nblk = mt * nt;
    const int hw = blockIdx.x;
    const int per = nblk / 8;
    const int lin = hw < per * 8 ? (hw % 8) * per + hw / 8 : hw;
    const int group = lin / (GE_GROUP_M * nt);
    const int first_m = group * GE_GROUP_M;
    const int gm = min(mt - first_m, GE_GROUP_M);
    const int within = lin % (GE_GROUP_M * nt);
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    const int64_t m0 = (int64_t)tm * GE_TM, n0 = (int64_t)tn * GE_TN;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;

    // Staging: global -> LDS by the copy path of global_load_lds_dwordx4 (no
    // registers).  One instruction of a wave fills 1 KB of LDS, 16 bytes per
    // lane in lane order: 8 rows of 128 bytes (64 K-elements).  Lane l of the
    // wave's i-th instruction fills LDS row r = 32 i + 8 wv + l / 8, slot
    // l % 8, and fetches the 16-byte chunk c = slot ^ ((r >> 1) & 7) of that
    // row: the XOR swizzle spreads the 16 rows of one fragment read over all
    // 64 banks.  Chunks past K come from ge_zero16; rows past M / N are
    // clamped to the last row (their outputs are never read).
    const int lr = 8 * wv + (lane >> 3), slot = lane & 7;
    int64_t aoff[8], boff[8];
    int csw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 32 * i + lr;
        csw[i] = (slot ^ ((r >> 1) & 7)) * 8;
        aoff[i] = min(m0 + r, M - 1) * K + csw[i];
        boff[i] = min(n0 + r, N - 1) * K + csw[i];
    }
#define GE_ISSUE(k0, buf)                                                                              \
    do {                                                                                               \
        uint16_t *sa_ = glds + (buf) * GE_STAGE + (8 * wv) * GE_TK;                                    \
        uint16_t *sb_ = sa_ + GE_TM * GE_TK;                                                           \
        _Pragma("unroll") for (int i = 0; i < 8; ++i)                                                  \
        {                                                                                              \
            const bool in_ = (k0) + csw[i] < K;                                                        \
            const void *pa_ = in_ ? (const void *)(A + aoff[i] + (k0)) : (const void *)ge_zero16;      \
            const void *pb_ = in_ ? (const void *)(Bm + boff[i] + (k0)) : (const void *)ge_zero16;     \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)pa_, (ge_lds_void *)(sa_ + 32 * i * GE_TK), 16, 0, 0); \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)pb_, (ge_lds_void *)(sb_ + 32 * i * GE_TK), 16, 0, 0); \
        }                                                                                              \
    } while (0)

    of32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Fragments of one 16-wide K slice: a[4] (X rows) and b[4] (weight rows),
    // double-buffered so the slice after the current one is read from LDS
    // while the current one multiplies.  The last slice of a stage is read
    // before the barrier, so the first slice of the next stage can be read
    // right after it, behind the last 16 MFMAs of this stage.
    const int fr = lane & 31, fh = lane >> 5;
    V fa[2][4], fb[2][4];
#define GE_FRAG(set, bufp, kk)                                                                         \
    do {                                                                                               \
        const int c_ = 2 * (kk) + fh;                                                                  \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
        {                                                                                              \
            const int r_ = wm * 128 + i * 32 + fr;                                                     \
            fa[set][i] = *reinterpret_cast<const V *>((bufp) + r_ * GE_TK + ((c_ ^ ((r_ >> 1) & 7)) * 8)); \
        }                                                                                              \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                  \
        {                                                                                              \
            const int r_ = GE_TM + wn * 128 + j * 32 + fr;                                             \
            fb[set][j] = *reinterpret_cast<const V *>((bufp) + r_ * GE_TK + ((c_ ^ ((r_ >> 1) & 7)) * 8)); \
        }                                                                                              \
    } while (0)

    const int ksteps = (int)((K + GE_TK - 1) / GE_TK);
    GE_ISSUE((int64_t)0, 0);
    __syncthreads();  // waits for the copies (vmcnt) and publishes them
    GE_FRAG(0, glds, 0);
    for (int ks = 0; ks < ksteps; ++ks) {
        const int buf = ks & 1;
        const bool more = ks + 1 < ksteps;
        if (more) GE_ISSUE((int64_t)(ks + 1) * GE_TK, buf ^ 1);
        const uint16_t *base = glds + buf * GE_STAGE;
#pragma unroll
        for (int kk = 0; kk < GE_TK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < GE_TK / 16) {
                GE_FRAG(cur ^ 1, base, kk + 1);
            } else {
                // every read of this stage is issued: wait for the next
                // stage's copies, then start reading it
                __syncthreads();
                if (more) GE_FRAG(cur ^ 1, glds + (buf ^ 1) * GE_STAGE, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Mfma16<F16>::op(fa[cur][i], fb[cur][j], acc[i][j]);
        }
    }
#undef GE_FRAG
#undef GE_ISSUE

    // epilogue: accumulator v of lane l in a 32 x 32 tile is row
    // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
    double sd = 0.0, sy = 0.0;
    const int64_t nb0 = n0 + wn * 128 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t mrow[16];
        double f[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            mrow[v] = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            f[v] = 1.0;
            if (MODE == GE_SUB_Y && erow != nullptr) f[v] = ldexp(fscale, erow[min(mrow[v], M - 1)]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = nb0 + j * 32;
            const int64_t nc = min(n, N - 1);
            if (MODE == GE_STORE_Y) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (mrow[v] < M && n < N) {
                        const float a = acc[i][j][v];
                        Y[mrow[v] * N + n] = a;
                        sy = __builtin_fma((double)a, (double)a, sy);
                    }
                }
            } else {
                // all 16 reads of Y in flight before the first use
                float yv[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) yv[v] = Y[min(mrow[v], M - 1) * N + nc];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const double d = (double)acc[i][j][v] * f[v] - (double)yv[v];
                    sd = (mrow[v] < M && n < N) ? __builtin_fma(d, d, sd) : sd;
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
        part[2 * (int64_t)blockIdx.x] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        part[2 * (int64_t)blockIdx.x + 1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
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
    const bool sval = SK == SCALE_E8M0 ? sc <= 254 : sc <= 126;
    // INT8 carries the E4M3 value of the scale code; 1/127 goes to the epilogue
    const float s = !sval ? 0.0f : (EK == ELEM_INT8 ? e4m3_value(sc) : scale_value(SK, sc));
    uint32_t c[8];
    if (EK == ELEM_E2M1) {
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
static int64_t at_least1(int64_t x) { return x > 0 ? x : 1; }

RefLayout output_reference_layout(int64_t M, int64_t N, int64_t K)
{
    RefLayout L;
    L.y = 256;
    L.e = L.y + al256(M * N * 4);
    L.x = L.e + al256(M * 4);
    L.part = L.x + al256(M * K * 2);
    L.bytes = L.part + al256(at_least1(ge_tiles(M, N)) * 16);
    return L;
}

size_t output_error_codes_ws(int64_t M, int64_t N, int64_t K)
{
    return (size_t)(al256(N * K * 2) + al256(at_least1(ge_tiles(M, N)) * 16));
}

template <bool F16, int MODE>
static hipError_t launch_gemm_err(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K,
                                  float *Y, const int *erow, double fscale, double *part, hipStream_t st)
{
    const int mt = (int)((M + GE_TM - 1) / GE_TM), nt = (int)((N + GE_TN - 1) / GE_TN);
    const int64_t nb = (int64_t)mt * nt;
    if (nb == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)gemm_err_kernel<F16, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GE_LDS);
    if (e != hipSuccess) return e;
    gemm_err_kernel<F16, MODE><<<(unsigned)nb, GE_THREADS, GE_LDS, st>>>(A, Bm, M, N, K, mt, nt, Y, erow, fscale,
                                                                         part);
    return hipGetLastError();
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
    hipError_t e = launch_gemm_err<false, GE_STORE_Y>((const uint16_t *)X, (const uint16_t *)W, M, N, K, Y, nullptr,
                                                      1.0, part, st);
    if (e != hipSuccess) return e;
    outref_final<<<1, 256, 0, st>>>(part, ge_tiles(M, N), nullptr, ysq, nullptr, nullptr);
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
        default: return hipErrorInvalidValue;
        }
    }
    if (fmt == HD_INT8_E4M3)
        e = launch_gemm_err<true, GE_SUB_Y>(Xh, opnd, M, N, K, Y, erow, 1.0 / 127.0, part, st);
    else
        e = launch_gemm_err<false, GE_SUB_Y>((const uint16_t *)X, opnd, M, N, K, Y, nullptr, 1.0, part, st);
    if (e != hipSuccess) return e;
    outref_final<<<1, 256, 0, st>>>(part, ge_tiles(M, N), ysq, nullptr, out, sums);
    return hipGetLastError();
}

}  // namespace hd
