// hdiag.hip - h_j = sum_t X[t][j]^2, the diagonal of X^T X that weights the
// H-Optimal objective (quantisation algorithms note, §1).  HBM-bound column
// reduction over a row-major X [M, K].
//
// Pass 1: the rows are cut into R chunks (1024 or 2048 workgroups in all, at
// least 128 rows each); a 256-thread workgroup owns a 512-column strip of one
// chunk.  Each lane streams 16-byte row segments (8 columns) down the chunk,
// one row in four per wave, four rows in flight, with non-temporal loads
// (X is read once), and keeps 8 float64
// sums of float64 squares (exact for every bf16 and fp32 value: a float64
// product of two 24-bit significands needs 48 bits, and its exponent range
// covers squares of the smallest subnormal and the largest finite fp32), so
// the only rounding is float64 addition.  The four waves' sums are added through LDS
// in a fixed order and stored as a float64 partial [R][K] in the workspace.
// Pass 2: h[j] = fl32(sum over the R partials, in a fixed order).
// A one-column-per-lane variant covers K % 8 != 0.
#include <mutex>

#include "common.hpp"
#include "hdiag.h"
#include "kernels.hpp"

namespace hd {

static constexpr int HD_COLS = 512;  // columns per workgroup (64 lanes x 8)
static constexpr int HD_RIF = 4;     // rows in flight per lane
// non-temporal loads: X is streamed once (measured: 5.99 vs 5.2 TB/s at
// 244449 x 9728 bf16 with the workgroup counts below)
template <typename T>
__device__ __forceinline__ void hd_load8(const T *p, float *v)
{
    load8_nt<T>(p, v);
}

static void hdiag_shape(int64_t M, int64_t K, int64_t *col_tiles, int64_t *chunks)
{
    const int64_t cols = (K % 8 == 0) ? HD_COLS : 256;
    int64_t ct = (K + cols - 1) / cols;
    if (ct < 1) ct = 1;
    // about 2048 workgroups for large X (more loads in flight), 1024 for
    // small X (fewer partials to write and re-read); at least 128 rows each
    const int64_t wgs = M * K >= ((int64_t)1 << 29) ? 2048 : 1024;
    int64_t r = (M + 127) / 128;
    const int64_t want = (wgs + ct - 1) / ct;
    if (r > want) r = want;
    if (r < 1) r = 1;
    *col_tiles = ct;
    *chunks = r;
}

size_t hdiag_ws(int64_t M, int64_t K)
{
    int64_t ct, r;
    hdiag_shape(M, K, &ct, &r);
    return (size_t)r * (size_t)K * sizeof(double);
}

// x^2 in float64, exact for every finite float32 (hence bf16) value; a float32
// square would flush or round below 2^-126 and overflow above 2^64.
template <typename T>
__device__ __forceinline__ double sq(float x)
{
    return (double)x * (double)x;
}

template <typename T>
__global__ __launch_bounds__(256) void hdiag_vec(const T *__restrict__ X, int64_t M, int64_t K,
                                                 int64_t rows_per_chunk, double *__restrict__ part)
{
    __shared__ double red[3][64][8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * HD_COLS + lane * 8;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_chunk;
    int64_t t1 = t0 + rows_per_chunk;
    if (t1 > M) t1 = M;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < K) {
        const T *p = X + col;
        int64_t t = t0 + wv;
        // HD_RIF rows in flight per lane (non-temporal: X is read once)
        for (; t + 4 * (HD_RIF - 1) < t1; t += 4 * HD_RIF) {
            float v[HD_RIF][8];
#pragma unroll
            for (int u = 0; u < HD_RIF; ++u) hd_load8<T>(p + (t + 4 * u) * K, v[u]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                double s4 = 0.0;
#pragma unroll
                for (int u = 0; u < HD_RIF; u += 4)
                    s4 += (sq<T>(v[u][j]) + sq<T>(v[u + 1][j])) + (sq<T>(v[u + 2][j]) + sq<T>(v[u + 3][j]));
                acc[j] += s4;
            }
        }
        for (; t < t1; t += 4) {
            float v0[8];
            hd_load8<T>(p + t * K, v0);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += sq<T>(v0[j]);
        }
    }
    if (wv > 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wv - 1][lane][j] = acc[j];
    }
    __syncthreads();
    if (wv == 0 && col < K) {
        double *o = part + (int64_t)blockIdx.y * K + col;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = ((acc[j] + red[0][lane][j]) + red[1][lane][j]) + red[2][lane][j];
    }
}

template <typename T>
__global__ __launch_bounds__(256) void hdiag_col(const T *__restrict__ X, int64_t M, int64_t K,
                                                 int64_t rows_per_chunk, double *__restrict__ part)
{
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= K) return;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_chunk;
    int64_t t1 = t0 + rows_per_chunk;
    if (t1 > M) t1 = M;
    double acc = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        const float x = sizeof(T) == 2 ? bf16_to_f32(((const bf16_t *)X)[t * K + col]) : ((const float *)X)[t * K + col];
        acc += sq<T>(x);
    }
    part[(int64_t)blockIdx.y * K + col] = acc;
}

// h[col] = sum of the R row-chunk partials of col, in float64: 64 columns per
// workgroup; wave g sums the chunks r = g + 4 i as four running sums over
// i mod 4 (four loads in flight per lane and round; chunks past R are clamped
// for the load and contribute 0), and the 16 sums are combined in a fixed
// order.
__global__ __launch_bounds__(256) void hdiag_final(const double *__restrict__ part, int64_t R, int64_t K,
                                                   float *__restrict__ h)
{
    __shared__ double sh[4][64];
    const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 64 + c;
    double sv[4] = {0.0, 0.0, 0.0, 0.0};
    if (col < K)
        for (int64_t r0 = g; r0 < R; r0 += 16) {
            double x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = part[min<int64_t>(r0 + 4 * u, R - 1) * K + col];
#pragma unroll
            for (int u = 0; u < 4; ++u) sv[u] += r0 + 4 * u < R ? x[u] : 0.0;
        }
    sh[g][c] = (sv[0] + sv[1]) + (sv[2] + sv[3]);
    __syncthreads();
    if (g == 0 && col < K) h[col] = (float)((sh[0][c] + sh[1][c]) + (sh[2][c] + sh[3][c]));
}

hipError_t launch_hdiag(const void *X, int xdt, int64_t M, int64_t K, float *h, void *ws, hipStream_t st)
{
    int64_t ct, R;
    hdiag_shape(M, K, &ct, &R);
    const int64_t rpc = (M + R - 1) / R;
    double *part = static_cast<double *>(ws);
    const dim3 grid((unsigned)ct, (unsigned)R);
    if (K % 8 == 0) {
        if (xdt == 1)
            hdiag_vec<bf16_t><<<grid, 256, 0, st>>>((const bf16_t *)X, M, K, rpc, part);
        else
            hdiag_vec<float><<<grid, 256, 0, st>>>((const float *)X, M, K, rpc, part);
    } else {
        if (xdt == 1)
            hdiag_col<bf16_t><<<grid, 256, 0, st>>>((const bf16_t *)X, M, K, rpc, part);
        else
            hdiag_col<float><<<grid, 256, 0, st>>>((const float *)X, M, K, rpc, part);
    }
    hdiag_final<<<(unsigned)((K + 63) / 64), 256, 0, st>>>(part, R, K, h);
    return hipGetLastError();
}

// ------------------------------------------------------ hdiag_noalloc ---
// The row-chunk partials of hdiag_noalloc() live in this file-scope array, one
// copy per GPU for the life of the process, instead of a caller workspace.
// Host code never passes the symbol itself to a kernel (on the host it names a
// stand-in, not device memory): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is used.  Every partial is written by pass 1 before pass 2
// reads it, so nothing has to be cleared between calls.
static __device__ __align__(256) double scratch[HD_NOALLOC_SCRATCH_BYTES / sizeof(double)];

static constexpr int HD_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[HD_MAX_DEVICES];

size_t hdiag_noalloc_limit() { return sizeof(scratch); }

hipError_t hdiag_scratch_address(hipStream_t st, void **ptr)
{
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (st != nullptr) {
        hipDevice_t d = 0;
        e = hipStreamGetDevice(st, &d);
        if (e != hipSuccess) return e;
        dev = (int)d;
    }
    if (dev < 0 || dev >= HD_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace hd
