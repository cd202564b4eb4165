// outerr.hip - relative output error ||X Wq^T - X W^T||_F / ||X W^T||_F
// (qwantize "Results", metric definitions): the one dense contraction of the
// path, on the bf16 MFMA units.
//
//   Y = X W^T and D = X dW^T with dW = fl32(Wq - W) carried as two bf16
//   terms hi + lo (rounding the difference, not Wq, keeps INT8 codes that bf16
//   cannot hold from moving the metric; the lo term keeps dW to ~2^-17);
//   the kernel never writes Y or D: each output tile is squared and summed in
//   float64 in registers, and one (sum D^2, sum Y^2) pair per workgroup is
//   reduced in a fixed order by a final one-workgroup kernel.
//
// GEMM tiling (gfx950, v_mfma_f32_32x32x16_bf16, wave64):
//   - workgroup = 8 waves, macro tile 256 rows of X x 128 rows of W, and the
//     same 128 rows of dW-hi and dW-lo: the X tile is loaded once and feeds
//     all three products (640 staged rows per 256 x 128 x 3 products);
//   - wave (wm, wn): 64 rows of X x 64 rows of W, as 2 x 2 MFMA tiles of
//     32 x 32 for Y and 2 x 2 for D (hi and lo accumulate into the same D
//     tiles) -> 128 fp32 accumulators per lane, 12 MFMAs per 16 of K;
//   - K is walked 32 at a time through two LDS stages (100 KB, dynamic; global
//     loads for step k+1 are in flight while step k multiplies); LDS rows are
//     padded to 80 bytes so the 16-byte fragment reads of 8 consecutive lanes
//     hit distinct bank groups;
//   - the tile index is remapped so the workgroups that one XCD runs at a time
//     share X and W panels in that XCD's L2 (8 consecutive X tiles per W tile).
// Inputs that are not (bf16 X, bf16 W, K % 32 == 0) take a float32 vector path.
#include "common.hpp"
#include "kernels.hpp"

namespace hd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

static constexpr int OE_TM = 256;     // X rows per tile
static constexpr int OE_TN = 128;     // W rows per tile (and as many dW rows)
static constexpr int OE_TK = 32;      // K per stage
static constexpr int OE_PITCH = 40;   // bf16 per LDS row (32 + 8 padding)
static constexpr int OE_GROUP_M = 8;  // X tiles walked per W tile

// -------------------------------------------------- dW = Wq - W as hi + lo --
// dW = fl32(Wq - W) split into two bfloat16 terms, hi = bf16(dW) and
// lo = bf16(dW - hi): X hi^T + X lo^T carries dW to ~2^-17 relative, where
// bf16(dW) alone (2^-9) would move the metric by ~1e-4 when a few outlier
// input channels dominate ||D||.
template <typename TQ>
__global__ __launch_bounds__(256) void delta_kernel(const bf16_t *__restrict__ W, const TQ *__restrict__ Wq,
                                                    int64_t total, bf16_t *__restrict__ hi, bf16_t *__restrict__ lo)
{
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e0 >= total) return;
    float w[8], q[8];
    load8<bf16_t>(W + e0, w);
    load8<TQ>(Wq + e0, q);
    uint32_t oh[8], ol[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = q[j] - w[j];
        oh[j] = f32_to_bf16(d);
        ol[j] = f32_to_bf16(d - bf16_to_f32(oh[j]));
    }
    uint4 v;
    v.x = oh[0] | (oh[1] << 16);
    v.y = oh[2] | (oh[3] << 16);
    v.z = oh[4] | (oh[5] << 16);
    v.w = oh[6] | (oh[7] << 16);
    *reinterpret_cast<uint4 *>(hi + e0) = v;
    v.x = ol[0] | (ol[1] << 16);
    v.y = ol[2] | (ol[3] << 16);
    v.z = ol[4] | (ol[5] << 16);
    v.w = ol[6] | (ol[7] << 16);
    *reinterpret_cast<uint4 *>(lo + e0) = v;
}

// --------------------------------------------------------------- MFMA GEMM --
static constexpr int OE_THREADS = 512;  // 8 waves: 4 (X rows) x 2 (W rows)
// LDS stage: the X tile and NP panels of 128 B rows (W, hi, lo; or hi, lo
// when ||X W^T||^2 is given and Y is not needed)
__host__ __device__ constexpr int oe_stage(int np) { return (OE_TM + np * OE_TN) * OE_PITCH; }
constexpr size_t oe_lds_bytes(int np) { return 2 * (size_t)oe_stage(np) * sizeof(bf16_t); }

template <bool WITH_Y>
__global__ __launch_bounds__(OE_THREADS, 1) void outerr_mfma(const bf16_t *__restrict__ X, const bf16_t *__restrict__ W,
                                                   const bf16_t *__restrict__ dhi, const bf16_t *__restrict__ dlo,
                                                   int64_t M, int64_t N, int64_t K, int mt, int nt,
                                                   double *__restrict__ part)
{
    extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
    __shared__ double red[2][8];

    // tile index: XCD-aware remap, then 8 X tiles per W tile
    const int nblk = mt * nt;
    const int hw = blockIdx.x;
    const int per = nblk / 8;
    const int lin = hw < per * 8 ? (hw % 8) * per + hw / 8 : hw;
    const int group = lin / (OE_GROUP_M * nt);
    const int first_m = group * OE_GROUP_M;
    const int gm = min(mt - first_m, OE_GROUP_M);
    const int within = lin % (OE_GROUP_M * nt);
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    const int64_t m0 = (int64_t)tm * OE_TM, n0 = (int64_t)tn * OE_TN;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 3, wn = wv >> 2;  // 64 rows of X x 64 rows of W / dW

    // global -> register staging, 16-byte chunks: X tile 256 x 32 (2 per
    // thread), the NP 128 x 32 B panels (one chunk per thread and panel: row
    // tid / 4 of panel i)
    constexpr int NP = WITH_Y ? 3 : 2;
    constexpr int OE_STAGE = oe_stage(NP);
    constexpr int PH = WITH_Y ? 1 : 0;  // LDS panel index of dW-hi
    const int sr = tid >> 2, sk = (tid & 3) * 8;
    const bf16_t *const panel[3] = {WITH_Y ? W : dhi, WITH_Y ? dhi : dlo, dlo};
    uint4 ra[2], rb[NP];
#define OE_GLOAD(k0)                                                                                       \
    do {                                                                                                   \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                      \
        {                                                                                                  \
            const int64_t m = m0 + 128 * i + sr;                                                           \
            ra[i] = m < M ? *reinterpret_cast<const uint4 *>(X + m * K + (k0) + sk) : make_uint4(0, 0, 0, 0); \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < NP; ++i)                                                     \
        {                                                                                                  \
            const int64_t n = n0 + sr;                                                                     \
            rb[i] = n < N ? *reinterpret_cast<const uint4 *>(panel[i] + n * K + (k0) + sk)                 \
                          : make_uint4(0, 0, 0, 0);                                                        \
        }                                                                                                  \
    } while (0)
#define OE_SWRITE(buf)                                                                                     \
    do {                                                                                                   \
        bf16_t *base_ = lds + (buf) * OE_STAGE;                                                            \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                      \
            *reinterpret_cast<uint4 *>(base_ + (128 * i + sr) * OE_PITCH + sk) = ra[i];                    \
        _Pragma("unroll") for (int i = 0; i < NP; ++i)                                                     \
            *reinterpret_cast<uint4 *>(base_ + (OE_TM + 128 * i + sr) * OE_PITCH + sk) = rb[i];            \
    } while (0)

    f32x16_t accy[2][2], accd[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                accy[i][j][v] = 0.0f;
                accd[i][j][v] = 0.0f;
            }

    const int ksteps = (int)(K / OE_TK);
    OE_GLOAD(0);
    OE_SWRITE(0);
    __syncthreads();
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    for (int ks = 0; ks < ksteps; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < ksteps) OE_GLOAD((int64_t)(ks + 1) * OE_TK);
        const bf16_t *base = lds + buf * OE_STAGE;
#pragma unroll
        for (int kk = 0; kk < OE_TK; kk += 16) {
            bf16x8_t af[2], bw[2], bh[2], bl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t *>(base + (wm * 64 + i * 32 + fr) * OE_PITCH + kk + fk);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int br = OE_TM + wn * 64 + j * 32 + fr;
                if (WITH_Y) bw[j] = *reinterpret_cast<const bf16x8_t *>(base + br * OE_PITCH + kk + fk);
                bh[j] = *reinterpret_cast<const bf16x8_t *>(base + (br + PH * OE_TN) * OE_PITCH + kk + fk);
                bl[j] = *reinterpret_cast<const bf16x8_t *>(base + (br + (PH + 1) * OE_TN) * OE_PITCH + kk + fk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (WITH_Y)
                        accy[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], accy[i][j], 0, 0, 0);
                    accd[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bh[j], accd[i][j], 0, 0, 0);
                    accd[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bl[j], accd[i][j], 0, 0, 0);
                }
        }
        if (ks + 1 < ksteps) OE_SWRITE(buf ^ 1);
        __syncthreads();
    }

    double sy = 0.0, sd = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const double y = (double)accy[i][j][v], d = (double)accd[i][j][v];
                if (WITH_Y) sy = __builtin_fma(y, y, sy);
                sd = __builtin_fma(d, d, sd);
            }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        sy += __shfl_xor(sy, o, 64);
        sd += __shfl_xor(sd, o, 64);
    }
    if (lane == 0) {
        red[0][wv] = sd;
        red[1][wv] = sy;
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0, b = 0.0;
        for (int w = 0; w < 8; ++w) {
            a += red[0][w];
            b += red[1][w];
        }
        part[2 * (int64_t)blockIdx.x] = a;
        part[2 * (int64_t)blockIdx.x + 1] = b;
    }
#undef OE_GLOAD
#undef OE_SWRITE
}

// ------------------------------------------------------ float32 VALU path --
// One lane per (row of X, row of W): both dot products in fp32 FMAs.
template <typename TX, typename TW, typename TQ>
__global__ __launch_bounds__(256) void outerr_valu(const TX *__restrict__ X, const TW *__restrict__ W,
                                                   const TQ *__restrict__ Wq, int64_t M, int64_t N, int64_t K,
                                                   double *__restrict__ part)
{
    __shared__ double sh[4];
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    double dd = 0.0, yy = 0.0;
    if (idx < M * N) {
        const int64_t m = idx / N, n = idx % N;
        float y = 0.0f, d = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float x = sizeof(TX) == 2 ? bf16_to_f32(((const bf16_t *)X)[m * K + k]) : ((const float *)X)[m * K + k];
            const float w = sizeof(TW) == 2 ? bf16_to_f32(((const bf16_t *)W)[n * K + k]) : ((const float *)W)[n * K + k];
            const float q = sizeof(TQ) == 2 ? bf16_to_f32(((const bf16_t *)Wq)[n * K + k]) : ((const float *)Wq)[n * K + k];
            y = __builtin_fmaf(x, w, y);
            d = __builtin_fmaf(x, q - w, d);
        }
        yy = (double)y * (double)y;
        dd = (double)d * (double)d;
    }
    dd = block_sum_256(dd, sh);
    yy = block_sum_256(yy, sh);
    if (threadIdx.x == 0) {
        part[2 * (int64_t)blockIdx.x] = dd;
        part[2 * (int64_t)blockIdx.x + 1] = yy;
    }
}

__global__ __launch_bounds__(256) void outerr_final(const double *__restrict__ part, int64_t n,
                                                    const double *__restrict__ ysq, double *__restrict__ out,
                                                    double *__restrict__ sums)
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
        if (ysq) b = *ysq;
        *out = sqrt(a) / sqrt(b);
        if (sums) {
            sums[0] = a;
            sums[1] = b;
        }
    }
}

bool output_error_uses_mfma(int xdt, int wdt, int64_t K) { return xdt == 1 && wdt == 1 && K % OE_TK == 0; }

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static int64_t oe_blocks(int64_t M, int64_t N, int64_t K, bool mfma)
{
    if (mfma) return ((M + OE_TM - 1) / OE_TM) * ((N + OE_TN - 1) / OE_TN);
    return (M * N + 255) / 256;
}

size_t output_error_ws(int64_t M, int64_t N, int64_t K, bool mfma)
{
    const int64_t nb = oe_blocks(M, N, K, mfma);
    const int64_t dw = mfma ? 2 * align256(N * K * 2) : 0;
    return (size_t)(dw + align256((nb > 0 ? nb : 1) * 16));
}

hipError_t launch_output_error(const void *X, int xdt, int64_t M, const void *W, int wdt, const void *Wq,
                               int qdt, int64_t N, int64_t K, const double *ysq, double *out, double *sums,
                               void *ws, hipStream_t st)
{
    const bool mfma = output_error_uses_mfma(xdt, wdt, K);
    int64_t nb = oe_blocks(M, N, K, mfma);
    char *wsb = static_cast<char *>(ws);
    if (mfma) {
        bf16_t *dhi = reinterpret_cast<bf16_t *>(wsb);
        bf16_t *dlo = reinterpret_cast<bf16_t *>(wsb + align256(N * K * 2));
        double *part = reinterpret_cast<double *>(wsb + 2 * align256(N * K * 2));
        const int64_t total = N * K;
        const unsigned g = (unsigned)((total / 8 + 255) / 256);
        if (total > 0) {
            if (qdt == 1)
                delta_kernel<bf16_t><<<g, 256, 0, st>>>((const bf16_t *)W, (const bf16_t *)Wq, total, dhi, dlo);
            else
                delta_kernel<float><<<g, 256, 0, st>>>((const bf16_t *)W, (const float *)Wq, total, dhi, dlo);
        }
        const int mt = (int)((M + OE_TM - 1) / OE_TM), nt = (int)((N + OE_TN - 1) / OE_TN);
        if (nb > 0) {
            if (ysq) {
                const size_t lds = oe_lds_bytes(2);
                hipError_t e = hipFuncSetAttribute((const void *)outerr_mfma<false>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
                outerr_mfma<false><<<(unsigned)nb, OE_THREADS, lds, st>>>((const bf16_t *)X, (const bf16_t *)W, dhi,
                                                                          dlo, M, N, K, mt, nt, part);
            } else {
                const size_t lds = oe_lds_bytes(3);
                hipError_t e = hipFuncSetAttribute((const void *)outerr_mfma<true>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
                outerr_mfma<true><<<(unsigned)nb, OE_THREADS, lds, st>>>((const bf16_t *)X, (const bf16_t *)W, dhi,
                                                                         dlo, M, N, K, mt, nt, part);
            }
        }
        outerr_final<<<1, 256, 0, st>>>(part, nb, ysq, out, sums);
        return hipGetLastError();
    }
    double *part = reinterpret_cast<double *>(wsb);
#define HD_OE_VALU(TX, TW, TQ)                                                                         \
    outerr_valu<TX, TW, TQ><<<(unsigned)nb, 256, 0, st>>>((const TX *)X, (const TW *)W, (const TQ *)Wq, M, N, \
                                                          K, part)
    if (nb > 0) {
        if (xdt == 1) {
            if (wdt == 1) { if (qdt == 1) HD_OE_VALU(bf16_t, bf16_t, bf16_t); else HD_OE_VALU(bf16_t, bf16_t, float); }
            else { if (qdt == 1) HD_OE_VALU(bf16_t, float, bf16_t); else HD_OE_VALU(bf16_t, float, float); }
        } else {
            if (wdt == 1) { if (qdt == 1) HD_OE_VALU(float, bf16_t, bf16_t); else HD_OE_VALU(float, bf16_t, float); }
            else { if (qdt == 1) HD_OE_VALU(float, float, bf16_t); else HD_OE_VALU(float, float, float); }
        }
    }
#undef HD_OE_VALU
    outerr_final<<<1, 256, 0, st>>>(part, nb, ysq, out, sums);
    return hipGetLastError();
}

}  // namespace hd
