// gptq.hip - GPTQ on top of a scale choice (qwantize "Results", "GPTQ
// Quantization": GPTQ of Frantar et al. with the GPTQ block equal to the
// quantisation block, columns in natural order (GPTQ-Seq) or block columns by
// descending Hessian-weighted loss (GPTQ-Ord); quantisation-algorithms note,
// §1: H = X^T X + lambda I, columns quantised in sequence, each residual
// propagated through H^-1).
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   1. H = X^T X (gptq_hessian): for K % 8 == 0 the bf16 MFMA product of
//      output_gram read straight from row-major X, its lower tile triangle
//      computed and each element stored with its mirror; otherwise X is
//      transposed into the workspace and the full product computed; float32
//      (bf16 products are exact; the sums carry float32 accumulation).
//   2. h = diag(H), lambda = damp * mean(h) (1 if the mean is 0).
//   3. GPTQ-Ord only: the method's own scales on W, the h-weighted loss of
//      every block column in float64 (fixed summation order), and the
//      processing order by descending loss (ties: lower block first).
//   4. P = J (Hp + lambda I) J, Hp = H with rows and columns in processing
//      order and J the reversal, in float64; a recursive Cholesky gives
//      L^-1 for P = L L^T directly (leaves of 64 x 64 factored and inverted
//      in LDS; above them L21 = P21 L11^-T, S22 = P22 - L21 L21^T,
//      (L^-1)21 = -(L22^-1) L21 (L11^-1), all float64 GEMMs, on the matrix
//      cores from 256 rows and columns up).  Then
//      (Hp + lambda I)^-1 = U^T U with U = J L^-1 J (upper triangular), and the
//      loop uses V[c][k] = U[c][k] / U[c][c] in float64.
//   5. The column loop over panels of BL = 128 (256 for B = 256) columns:
//      gptq_panel_kernel walks a panel with one wave per row (each lane
//      holding BL / 64 working values in registers): at each
//      quantisation block it picks every row's scale with the method from the
//      current values rounded to float32 (the quantiser's input; the
//      full-grid argmin with the lanes splitting the candidates, or the FP16
//      alternation), then encodes the block's columns one by one,
//      broadcasting each error e = w - q to the row's lanes, which apply
//      w_k -= e V[c][k] inside the panel; then W[:, pe:] -= E V[panel, pe:]
//      applies the panel's errors to every later column (the float64
//      matrix-core GEMM of the factorisation).  Working weights, V and the
//      errors are float64: GPTQ's decisions cascade along a row (a flipped
//      element changes every later compensation), and with float32 working
//      weights about 0.3% of INT8 elements moved against a float64 loop,
//      while float64 rounding in another order moved none.
// Codes and scales are written at the original column / block positions.
#include <algorithm>
#include <cstdlib>

#include "encode.hpp"
#include "hdiag.h"
#include "kernels.hpp"

namespace hd {

// --------------------------------------------------------------- helpers ---

// Xt[k][m] = X[m][k] for m < M, 0 for M <= m < M8 (bf16 bits): the staging of
// the Hessian's product when K % 8 != 0 (rows of X then are not whole 16-byte
// chunks, which the in-place product reads).
__global__ __launch_bounds__(256) void gptq_transpose_kernel(const uint16_t *__restrict__ X, int64_t M, int64_t K,
                                                             int64_t M8, uint16_t *__restrict__ Xt)
{
    __shared__ uint16_t t[64][66];
    const int64_t m0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    for (int r = ty; r < 64; r += 4) {
        const int64_t m = m0 + r, k = k0 + tx;
        t[r][tx] = (m < M && k < K) ? X[m * K + k] : (uint16_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t k = k0 + r, m = m0 + tx;
        if (k < K && m < M8) Xt[k * M8 + m] = t[tx][r];
    }
}

// h[k] = H[k][k]; stat[0] = lambda (damp * mean(h), or 1 when it is 0).
__global__ __launch_bounds__(256) void gptq_diag_kernel(const float *__restrict__ H, int64_t K, double damp,
                                                        float *__restrict__ h, double *__restrict__ stat)
{
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const float v = H[k * K + k];
        h[k] = v;
        s += (double)v;
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double mean = red[0] / (double)K;
        stat[0] = mean > 0.0 ? damp * mean : 1.0;
    }
}

// Hessian-weighted loss of block column b: sum over rows of
// sum_j h_j (|w| - fl32(s q))^2 at the given scales, in float64; each block's
// sum runs j in order and the rows are reduced in a fixed tree, so the result
// does not depend on scheduling.
template <int EK, int SK, typename T>
__global__ __launch_bounds__(256) void gptq_block_loss_kernel(const T *__restrict__ W, int64_t N, int64_t K, int B,
                                                              const float *__restrict__ h,
                                                              const uint8_t *__restrict__ scales,
                                                              double *__restrict__ loss)
{
    __shared__ double red[256];
    const int64_t b = blockIdx.x, nb = K / B;
    double acc = 0.0;
    for (int64_t n = threadIdx.x; n < N; n += 256) {
        const int code = load_scale<SK>(scales, n * nb + b);
        const float s = scale_code_valid(SK, code) ? scale_value(SK, code) : 0.0f;
        const float r = s != 0.0f ? 1.0f / s : 0.0f;
        double o = 0.0;
        for (int j = 0; j < B; ++j) {
            const int64_t e = n * K + b * B + j;
            const float a = fabsf(sizeof(T) == 2 ? __uint_as_float((uint32_t)((const uint16_t *)W)[e] << 16)
                                                 : ((const float *)W)[e]);
            const float x = s != 0.0f ? quotient<SK, false>(a, s, r) : 0.0f;
            const float wq = s * round_elem<EK>(x);
            const double d = (double)a - (double)wq;
            o += (double)h[b * B + j] * (d * d);
        }
        acc += o;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[b] = red[0];
}

// Processing order: slot of block b = number of blocks that go before it
// (larger loss, or equal loss and lower index); perm[slot] = b (also into
// order_out when given).  Also clears the factorisation's info word.
__global__ __launch_bounds__(256) void gptq_rank_kernel(const double *__restrict__ loss, int64_t nb, int ordered,
                                                        int *__restrict__ perm, int32_t *__restrict__ order_out,
                                                        int *__restrict__ info)
{
    if (threadIdx.x == 0) info[0] = 0;
    for (int64_t b = threadIdx.x; b < nb; b += 256) {
        int64_t slot = b;
        if (ordered) {
            slot = 0;
            const double lb = loss[b];
            for (int64_t o = 0; o < nb; ++o) slot += (loss[o] > lb || (loss[o] == lb && o < b)) ? 1 : 0;
        }
        perm[slot] = (int)b;
        if (order_out) order_out[slot] = (int32_t)b;
    }
}

// Processing-order maps: col[i] = original column of processed column i,
// hp[i] = h[col[i]]; Wp[n][i] = W[n][col[i]] as float64.
template <typename T>
__global__ __launch_bounds__(256) void gptq_gather_kernel(const T *__restrict__ W, int64_t N, int64_t K, int B,
                                                          const int *__restrict__ perm, const float *__restrict__ h,
                                                          int *__restrict__ col, float *__restrict__ hp,
                                                          double *__restrict__ Wp)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= K) return;
    const int64_t c = (int64_t)perm[i / B] * B + i % B;
    if (blockIdx.y == 0) {
        col[i] = (int)c;
        hp[i] = h[c];
    }
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
        const int64_t e = n * K + c;
        Wp[n * K + i] = (double)(sizeof(T) == 2 ? __uint_as_float((uint32_t)((const uint16_t *)W)[e] << 16)
                                                : ((const float *)W)[e]);
    }
}

// P[i][j] = Hp[K-1-i][K-1-j] + lambda [i == j] (float64): the reversed,
// permuted, damped Hessian.
__global__ __launch_bounds__(256) void gptq_build_p_kernel(const float *__restrict__ H, int64_t K,
                                                           const int *__restrict__ col,
                                                           const double *__restrict__ stat, double *__restrict__ P)
{
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x, i = blockIdx.y;
    if (j >= K) return;
    const int64_t ci = col[K - 1 - i], cj = col[K - 1 - j];
    double v = (double)H[ci * K + cj];
    if (i == j) v += stat[0];
    P[i * K + j] = v;
}

// V[c][k] = U[c][k] / U[c][c] for k > c, U[c][k] = Li[K-1-c][K-1-k] (float64).
__global__ __launch_bounds__(256) void gptq_build_v_kernel(const double *__restrict__ Li, int64_t K,
                                                           double *__restrict__ V)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x, c = blockIdx.y;
    if (k >= K) return;
    const int64_t rc = K - 1 - c;
    V[c * K + k] = k > c ? Li[rc * K + (K - 1 - k)] / Li[rc * K + rc] : 0.0;
}

// ---------------------------------------------- float64 factorisation ---

// Lane l's value of v, for a compile-time lane index (two 32-bit readlanes).
__device__ __forceinline__ double gq_lane(double v, int l)
{
    const long long b = __double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(b & 0xffffffff), l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Leaf: L = chol(P block), n <= 64, then Li = L^-1 (lower); only Li is kept.
// The block sits in LDS (rows / columns >= n padded with the identity) and is
// factored in four panels of 16 columns:
//   (a) one wave factors the panel's 16 x 16 diagonal block in registers,
//       lane i holding row i (right-looking; pivots and column entries are
//       passed between lanes by readlane, so the 16 steps need no barrier);
//   (b) one thread per row below solves that row of the panel by forward
//       substitution against the diagonal factor;
//   (c) all threads subtract the panel's outer product from the trailing
//       lower triangle.
// Then each wave inverts one diagonal 16 x 16 factor the same way (lane i
// holding row i of the inverse), and block forward substitution fills the
// off-diagonal blocks: X_pq = -X_pp sum_{q <= m < p} L_pm X_mq.  Eighteen
// barriers in all, against two per column for a column-at-a-time scheme.
// info[0] gets the first non-positive pivot's global index + 1 (the pivot is
// then replaced by 1 so the factorisation still finishes).
__global__ __launch_bounds__(256) void gptq_chol_leaf_kernel(const double *__restrict__ P, int64_t ld, int64_t off,
                                                             int n, double *__restrict__ Li, int *__restrict__ info)
{
    __shared__ double A[64][65];       // the block, then L (lower)
    __shared__ double X[64][65];       // L^-1 (lower)
    __shared__ double St[16][3 * 16 + 1];  // sums of the substitution
    __shared__ double rdg[64];         // 1 / L_kk
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15;
    for (int e = tid; e < 64 * 64; e += 256) {
        const int i = e >> 6, k = e & 63;
        A[i][k] = (i < n && k <= i) ? P[(off + i) * ld + off + k] : (i == k ? 1.0 : 0.0);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c0 = 16 * p, T = 48 - 16 * p;
        // (a) diagonal block: lanes 0..15 of wave 0 (the others repeat them)
        if (wv == 0) {
            double d[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) d[k] = k <= li ? A[c0 + li][c0 + k] : 0.0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                double piv = gq_lane(d[j], j);
                if (!(piv > 0.0)) {
                    if (lane == j && info && c0 + j < n) atomicCAS(info, 0, (int)(off + c0 + j + 1));
                    piv = 1.0;
                }
                const double pv = sqrt(piv), r = 1.0 / pv;
                d[j] = li > j ? d[j] * r : (li == j ? pv : 0.0);
#pragma unroll
                for (int k = j + 1; k < 16; ++k) d[k] = __builtin_fma(-d[j], gq_lane(d[j], k), d[k]);
            }
            if (lane < 16) {
#pragma unroll
                for (int k = 0; k < 16; ++k) A[c0 + li][c0 + k] = k <= li ? d[k] : 0.0;
                rdg[c0 + li] = 1.0 / d[li];
            }
        }
        __syncthreads();
        if (T == 0) break;
        // (b) rows below: L[r][c0 + q] = (A[r][c0 + q] - sum_{m < q} L[r][c0 + m] L[c0 + q][c0 + m]) / L_qq
        if (tid < T) {
            const int r = c0 + 16 + tid;
            double x[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                double sq = A[r][c0 + q];
#pragma unroll
                for (int m = 0; m < q; ++m) sq = __builtin_fma(-x[m], A[c0 + q][c0 + m], sq);
                x[q] = sq * rdg[c0 + q];
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) A[r][c0 + q] = x[q];
        }
        __syncthreads();
        // (c) trailing lower triangle
        for (int e = tid; e < T * T; e += 256) {
            const int r = c0 + 16 + e / T, q = c0 + 16 + e % T;
            if (q > r) continue;
            double acc = 0.0;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc = __builtin_fma(A[r][c0 + m], A[q][c0 + m], acc);
            A[r][q] -= acc;
        }
        __syncthreads();
    }
    // inverses of the diagonal factors: wave p, lanes 0..15 (lane i: row i)
    {
        const int c0 = 16 * wv;
        double x[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) x[m] = m == li ? 1.0 : 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const double rk = rdg[c0 + k];
            if (li == k) {
#pragma unroll
                for (int m = 0; m <= k; ++m) x[m] *= rk;
            }
            const double lik = li > k ? A[c0 + li][c0 + k] : 0.0;
#pragma unroll
            for (int m = 0; m <= k; ++m) x[m] = __builtin_fma(-lik, gq_lane(x[m], k), x[m]);
        }
        if (lane < 16) {
#pragma unroll
            for (int m = 0; m < 16; ++m) X[c0 + li][c0 + m] = m <= li ? x[m] : 0.0;
        }
    }
    __syncthreads();
    // block forward substitution, block rows 1..3
#pragma unroll
    for (int p = 1; p < 4; ++p) {
        // St[a][16 q + b] = sum_{m = q}^{p-1} sum_t L[16p + a][16m + t] X[16m + t][16q + b]
        for (int e = tid; e < 256 * p; e += 256) {
            const int q = e >> 8, a = (e >> 4) & 15, b = e & 15;
            double acc = 0.0;
            for (int m = q; m < p; ++m)
#pragma unroll
                for (int t = 0; t < 16; ++t) acc = __builtin_fma(A[16 * p + a][16 * m + t], X[16 * m + t][16 * q + b], acc);
            St[a][16 * q + b] = acc;
        }
        __syncthreads();
        // X_pq[a][b] = -sum_{t <= a} X_pp[a][t] St[t][16 q + b]
        for (int e = tid; e < 256 * p; e += 256) {
            const int q = e >> 8, a = (e >> 4) & 15, b = e & 15;
            double acc = 0.0;
#pragma unroll
            for (int t = 0; t <= a; ++t) acc = __builtin_fma(X[16 * p + a][16 * p + t], St[t][16 * q + b], acc);
            X[16 * p + a][16 * q + b] = -acc;
        }
        __syncthreads();
    }
    for (int e = tid; e < 64 * 64; e += 256) {
        const int i = e >> 6, k = e & 63;
        if (i < n && k < n) Li[(off + i) * ld + off + k] = k <= i ? X[i][k] : 0.0;
    }
}

// Structure flags of the float64 GEMM: operands known to be zero outside a
// triangle let a tile skip those k, and a symmetric result needs only the
// tiles that touch its lower triangle.
enum {
    TRI_B_KGE_N = 1,  // Bop[k][n] = 0 unless k >= n
    TRI_B_KLE_N = 2,  // Bop[k][n] = 0 unless k <= n
    TRI_A_KLE_M = 4,  // A[m][k] = 0 unless k <= m
    TRI_C_LOWER = 8   // only entries with n <= m are needed
};

// One float64 product C[m][n] = alpha sum_k A[m][k] Bop[k][n] + beta C[m][n]
// (row-major, leading dimensions lda / ldb / ldc; Bop = B or, with TB, B^T);
// `tri` (TRI_* flags) limits the k range and the tiles; gx = output tiles
// along N at the kernel's tile width.
struct GqGemm {
    int64_t M, N, K;
    double alpha;
    const double *A;
    int64_t lda;
    const double *B;
    int64_t ldb;
    double beta;
    double *C;
    int64_t ldc;
    int tri, gx;
};

// 64 x 64 output tile (bx, by) on the VALU: 4 x 4 per thread of 256, k in
// steps of 32 through LDS with the next step's operands loaded into
// registers during the current one.
template <bool TB>
__device__ __forceinline__ void gq_fma_tile(const GqGemm &g, int bx, int by, double (*As)[65], double (*Bs)[65])
{
    const int64_t M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const double *__restrict__ A = g.A;
    const double *__restrict__ Bm = g.B;
    const int tri = g.tri;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int64_t m0 = (int64_t)by * 64, n0 = (int64_t)bx * 64;
    if ((tri & TRI_C_LOWER) && n0 > m0 + 63) return;
    int64_t kb = 0, ke = K;
    if (tri & TRI_B_KGE_N) kb = n0;
    if (tri & TRI_B_KLE_N) ke = min(ke, n0 + 64);
    if (tri & TRI_A_KLE_M) ke = min(ke, m0 + 64);
    double acc[4][4] = {};
    double ra[8], rb[8];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = tid + 256 * q;
            const int64_t m = m0 + e / 32, k = k0 + e % 32;
            ra[q] = (m < M && k < ke) ? A[m * lda + k] : 0.0;
            int64_t n, kq;
            if (TB) { n = n0 + e / 32; kq = k0 + e % 32; } else { kq = k0 + e / 64; n = n0 + e % 64; }
            rb[q] = (n < N && kq < ke) ? (TB ? Bm[n * ldb + kq] : Bm[kq * ldb + n]) : 0.0;
        }
    };
    if (kb < ke) fetch(kb);
    for (int64_t k0 = kb; k0 < ke; k0 += 32) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = tid + 256 * q;
            As[e % 32][e / 32] = ra[q];
            if (TB) Bs[e % 32][e / 32] = rb[q]; else Bs[e / 64][e % 64] = rb[q];
        }
        __syncthreads();
        if (k0 + 32 < ke) fetch(k0 + 32);
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) {
            double av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(av[i], bv[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx + 16 * j;
            if (n >= N) continue;
            double *c = g.C + m * g.ldc + n;
            *c = g.beta == 0.0 ? g.alpha * acc[i][j] : g.beta * *c + g.alpha * acc[i][j];
        }
    }
}

template <bool TB>
__global__ __launch_bounds__(256) void gptq_dgemm_kernel(GqGemm g)
{
    __shared__ double As[32][65];
    __shared__ double Bs[32][65];
    gq_fma_tile<TB>(g, blockIdx.x, blockIdx.y, As, Bs);
}

// Two independent products in one launch (the first with Bop = B^T, the
// second with Bop = B): workgroups 0 .. nb1 - 1 take the first's tiles.
__global__ __launch_bounds__(256) void gptq_dgemm_pair_kernel(GqGemm g1, GqGemm g2, int nb1)
{
    __shared__ double As[32][65];
    __shared__ double Bs[32][65];
    const int b = blockIdx.x;
    if (b < nb1)
        gq_fma_tile<true>(g1, b % g1.gx, b / g1.gx, As, Bs);
    else
        gq_fma_tile<false>(g2, (b - nb1) % g2.gx, (b - nb1) / g2.gx, As, Bs);
}

// The same product on the float64 matrix cores (v_mfma_f64_16x16x4f64: lane l
// supplies A[l % 16][l / 16] and Bop[l / 16][l % 16] of a 16 x 4 by 4 x 16
// step and holds C[l / 16 + 4 v][l % 16], v = 0..3).  TILE x TILE output tile
// per workgroup of four waves (TILE = 128, or 64 for products too small to
// fill the chip with 128-tiles), TILE/2 x TILE/2 per wave as NB x NB MFMA
// blocks; k in steps of 16 through LDS (k-major rows, pitch TILE + 16
// doubles: the four k rows of one fragment read fall on alternate halves of
// the banks), the next step's operands loaded into registers while the
// current one is multiplied.  Operands are read in aligned 16-byte pairs:
// K, lda, ldb (and N when Bop = B) multiples of 8 and 2 doubles, base
// pointers 16-byte aligned.
typedef double gq_d4 __attribute__((ext_vector_type(4)));

template <bool TB, int TILE>
__device__ __forceinline__ void gq_mfma_tile(const GqGemm &g, int bx, int by, double *As, double *Bs)
{
    constexpr int PITCH = TILE + 16, NB = TILE / 32, CH = TILE / 16, CPR = 16 / CH, NP = CH / 2;
    const int64_t M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const double *__restrict__ A = g.A;
    const double *__restrict__ Bm = g.B;
    const int tri = g.tri;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
    const int64_t m0 = (int64_t)by * TILE, n0 = (int64_t)bx * TILE;
    if ((tri & TRI_C_LOWER) && n0 > m0 + TILE - 1) return;
    int64_t kb = 0, ke = K;
    if (tri & TRI_B_KGE_N) kb = n0;
    if (tri & TRI_B_KLE_N) ke = min(ke, n0 + TILE);
    if (tri & TRI_A_KLE_M) ke = min(ke, m0 + TILE);

    // staging: thread t loads CH consecutive doubles (NP 16-byte pairs) of
    // A row t / CPR, k chunk t % CPR; of Bop likewise with TB (B row = n),
    // else of B row k = t / 16, n chunk t % 16.  Every k bound above is a
    // multiple of 8, so a chunk is wholly inside or wholly outside [kb, ke).
    const int sr = tid / CPR, sc = (tid % CPR) * CH, br = tid >> 4, bc = (tid & 15) * CH;
    double2 ra[NP], rb[NP];
    auto fetch = [&](int64_t k0) {
        {
            const int64_t m = m0 + sr, k = k0 + sc;
            const bool ok = m < M && k < ke;
            const double2 *p = reinterpret_cast<const double2 *>(A + (ok ? m * lda + k : 0));
#pragma unroll
            for (int q = 0; q < NP; ++q) ra[q] = ok ? p[q] : make_double2(0.0, 0.0);
        }
        if (TB) {
            const int64_t n = n0 + sr, k = k0 + sc;
            const bool ok = n < N && k < ke;
            const double2 *p = reinterpret_cast<const double2 *>(Bm + (ok ? n * ldb + k : 0));
#pragma unroll
            for (int q = 0; q < NP; ++q) rb[q] = ok ? p[q] : make_double2(0.0, 0.0);
        } else {
            const int64_t k = k0 + br, n = n0 + bc;
            const bool ok = k < ke && n < N;
            const double2 *p = reinterpret_cast<const double2 *>(Bm + (ok ? k * ldb + n : 0));
#pragma unroll
            for (int q = 0; q < NP; ++q) rb[q] = ok ? p[q] : make_double2(0.0, 0.0);
        }
    };

    gq_d4 acc[NB][NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = gq_d4{0.0, 0.0, 0.0, 0.0};

    if (kb < ke) fetch(kb);
    const int fr = lane & 15, fk = lane >> 4;
    for (int64_t k0 = kb; k0 < ke; k0 += 16) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            As[(sc + 2 * q) * PITCH + sr] = ra[q].x;
            As[(sc + 2 * q + 1) * PITCH + sr] = ra[q].y;
            if (TB) {
                Bs[(sc + 2 * q) * PITCH + sr] = rb[q].x;
                Bs[(sc + 2 * q + 1) * PITCH + sr] = rb[q].y;
            } else {
                *reinterpret_cast<double2 *>(&Bs[br * PITCH + bc + 2 * q]) = rb[q];
            }
        }
        __syncthreads();
        if (k0 + 16 < ke) fetch(k0 + 16);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const int kr = (4 * k4 + fk) * PITCH;
            double av[NB], bv[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) av[i] = As[kr + wm * (TILE / 2) + i * 16 + fr];
#pragma unroll
            for (int j = 0; j < NB; ++j) bv[j] = Bs[kr + wn * (TILE / 2) + j * 16 + fr];
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * (TILE / 2) + i * 16 + fk + 4 * v;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int64_t n = n0 + wn * (TILE / 2) + j * 16 + fr;
                if (n >= N) continue;
                double *c = g.C + m * g.ldc + n;
                *c = g.beta == 0.0 ? g.alpha * acc[i][j][v] : g.beta * *c + g.alpha * acc[i][j][v];
            }
        }
}

template <bool TB, int TILE>
__global__ __launch_bounds__(256, 2) void gptq_dgemm_mfma_kernel(GqGemm g)
{
    __shared__ __attribute__((aligned(16))) double As[16 * (TILE + 16)];
    __shared__ __attribute__((aligned(16))) double Bs[16 * (TILE + 16)];
    gq_mfma_tile<TB, TILE>(g, blockIdx.x, blockIdx.y, As, Bs);
}

template <int TILE>
__global__ __launch_bounds__(256, 2) void gptq_dgemm_mfma_pair_kernel(GqGemm g1, GqGemm g2, int nb1)
{
    __shared__ __attribute__((aligned(16))) double As[16 * (TILE + 16)];
    __shared__ __attribute__((aligned(16))) double Bs[16 * (TILE + 16)];
    const int b = blockIdx.x;
    if (b < nb1)
        gq_mfma_tile<true, TILE>(g1, b % g1.gx, b / g1.gx, As, Bs);
    else
        gq_mfma_tile<false, TILE>(g2, (b - nb1) % g2.gx, (b - nb1) / g2.gx, As, Bs);
}

static GqGemm gq_gemm(int64_t M, int64_t N, int64_t K, double alpha, const double *A, int64_t lda, const double *Bm,
                      int64_t ldb, double beta, double *C, int64_t ldc, int tri)
{
    GqGemm g;
    g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.A = A; g.lda = lda; g.B = Bm; g.ldb = ldb;
    g.beta = beta; g.C = C; g.ldc = ldc; g.tri = tri; g.gx = 0;
    return g;
}

// Which kernel a product takes: 0 the VALU 64-tiles, else the matrix-core
// tile width.  Products of 256 rows and columns and up (with aligned
// operands) go to the matrix cores, with 128-tiles when they give at least
// two rounds of workgroups, unless the schedule setting HD_SCHED_GPTQ_TILE
// (64 or 128) names the width.
template <bool TB>
static int gq_tile(const GqGemm &g)
{
    const bool aligned = g.K % 8 == 0 && g.lda % 2 == 0 && g.ldb % 2 == 0 && (TB || g.N % 8 == 0) &&
                         reinterpret_cast<uintptr_t>(g.A) % 16 == 0 && reinterpret_cast<uintptr_t>(g.B) % 16 == 0;
    if (!(g.M >= 256 && g.N >= 256 && aligned)) return 0;
    const int forced = schedule_setting(HD_SCHED_GPTQ_TILE);
    const int64_t t128 = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    return (forced == 128 || (forced != 64 && t128 >= 2 * 256)) ? 128 : 64;
}

static int64_t gq_tiles(GqGemm &g, int tile)
{
    const int t = tile ? tile : 64;
    g.gx = (int)((g.N + t - 1) / t);
    return (int64_t)g.gx * ((g.M + t - 1) / t);
}

template <bool TB>
static void dgemm(int64_t M, int64_t N, int64_t K, double alpha, const double *A, int64_t lda, const double *Bm,
                  int64_t ldb, double beta, double *C, int64_t ldc, int tri, hipStream_t st)
{
    if (M <= 0 || N <= 0) return;
    GqGemm g = gq_gemm(M, N, K, alpha, A, lda, Bm, ldb, beta, C, ldc, tri);
    const int tile = gq_tile<TB>(g);
    gq_tiles(g, tile);
    const int t = tile ? tile : 64;
    const dim3 grid((unsigned)g.gx, (unsigned)((M + t - 1) / t));
    if (tile == 128)
        gptq_dgemm_mfma_kernel<TB, 128><<<grid, 256, 0, st>>>(g);
    else if (tile == 64)
        gptq_dgemm_mfma_kernel<TB, 64><<<grid, 256, 0, st>>>(g);
    else
        gptq_dgemm_kernel<TB><<<grid, 256, 0, st>>>(g);
}

// Two independent products (g1 with Bop = B^T, g2 with Bop = B) in one launch
// when both take the same kernel family and tile width, else one after the
// other.
static void dgemm_pair(GqGemm g1, GqGemm g2, hipStream_t st)
{
    const int t1 = gq_tile<true>(g1), t2 = gq_tile<false>(g2);
    if (t1 != t2 || g1.M <= 0 || g1.N <= 0 || g2.M <= 0 || g2.N <= 0) {
        dgemm<true>(g1.M, g1.N, g1.K, g1.alpha, g1.A, g1.lda, g1.B, g1.ldb, g1.beta, g1.C, g1.ldc, g1.tri, st);
        dgemm<false>(g2.M, g2.N, g2.K, g2.alpha, g2.A, g2.lda, g2.B, g2.ldb, g2.beta, g2.C, g2.ldc, g2.tri, st);
        return;
    }
    const int64_t nb1 = gq_tiles(g1, t1), nb2 = gq_tiles(g2, t2);
    const unsigned grid = (unsigned)(nb1 + nb2);
    if (t1 == 128)
        gptq_dgemm_mfma_pair_kernel<128><<<grid, 256, 0, st>>>(g1, g2, (int)nb1);
    else if (t1 == 64)
        gptq_dgemm_mfma_pair_kernel<64><<<grid, 256, 0, st>>>(g1, g2, (int)nb1);
    else
        gptq_dgemm_pair_kernel<<<grid, 256, 0, st>>>(g1, g2, (int)nb1);
}

// Recursive Cholesky-with-inverse of the n x n diagonal block of P at `off`
// (row-major, leading dimension ld): writes L^-1 of that block into Li
// (same position).  P's trailing block is overwritten by its Schur
// complement.  T (>= (n/2)^2 doubles, free on entry) holds L21; T2 is a stack
// of temporaries that must survive the recursive calls.
static void cholinv(double *P, double *Li, int64_t ld, int64_t off, int64_t n, double *T, double *T2, int *info,
                    hipStream_t st)
{
    if (n <= 64) {
        gptq_chol_leaf_kernel<<<1, 256, 0, st>>>(P, ld, off, (int)n, Li, info);
        return;
    }
    const int64_t n1 = ((n / 2 + 63) / 64) * 64, n2 = n - n1;
    double *P11 = P + off * ld + off, *P21 = P11 + n1 * ld, *P22 = P21 + n1;
    double *Li11 = Li + off * ld + off, *Li21 = Li11 + n1 * ld, *Li22 = Li21 + n1;
    cholinv(P, Li, ld, off, n1, T, T2, info, st);
    // L21 = P21 L11^-T  (T: n2 x n1; L11^-T is upper triangular)
    dgemm<true>(n2, n1, n1, 1.0, P21, ld, Li11, ld, 0.0, T, n1, TRI_B_KLE_N, st);
    // S22 = P22 - L21 L21^T (symmetric: the recursion reads its lower triangle)
    // and L21 L11^-1 (T2: n2 x n1, kept across the recursion on S22): both
    // read only T and L11^-1, so they share one launch
    double *Tm = T2;
    dgemm_pair(gq_gemm(n2, n2, n1, -1.0, T, n1, T, n1, 1.0, P22, ld, TRI_C_LOWER),
               gq_gemm(n2, n1, n1, 1.0, T, n1, Li11, ld, 0.0, Tm, n1, TRI_B_KGE_N), st);
    cholinv(P, Li, ld, off + n1, n2, T, T2 + n2 * n1, info, st);
    // (L^-1)21 = -L22^-1 (L21 L11^-1), L22^-1 lower triangular
    dgemm<false>(n2, n1, n2, -1.0, Li22, ld, Tm, n1, 0.0, Li21, ld, TRI_A_KLE_M, st);
}

// ------------------------------------------------------- column loop ---

enum { GQ_NAIVE = 0, GQ_GRID = 1, GQ_ALT = 2 };

// Objective of one block (values v[0..B-1] in LDS, fp32) at scale s:
// sum_j om_j (|v_j| - fl32(s q_j))^2 in float64, j in order - the oracle's
// block objective, operation for operation.
template <int EK, int SK, bool WEIGHTED>
__device__ __forceinline__ double gq_objective(const float *v, const float *om, int B, float s, float r)
{
    double o = 0.0;
    for (int j = 0; j < B; ++j) {
        const float a = fabsf(v[j]);
        const float x = s != 0.0f ? quotient<SK, false>(a, s, r) : 0.0f;
        const float wq = s * round_elem<EK>(x);
        const double d = (double)a - (double)wq;
        o += (WEIGHTED ? (double)om[j] : 1.0) * (d * d);
    }
    return o;
}

// The FP16 alternation of alt_f16.hip for one block held in LDS, run by one
// lane with every sum in element order.
template <int EK, bool WEIGHTED>
__device__ int gq_alternation(const float *v, const float *om, int B)
{
    float amax = 0.0f;
    for (int j = 0; j < B; ++j) amax = fmaxf(amax, fabsf(v[j]));
    int code = naive_code<EK, SCALE_F16>(amax), best_code = code;
    float s = scale_value(SCALE_F16, code);
    double best = gq_objective<EK, SCALE_F16, WEIGHTED>(v, om, B, s, s != 0.0f ? 1.0f / s : 0.0f);
    for (int round = 0; round < 32 && code != 0; ++round) {
        const float r = 1.0f / s;
        double num = 0.0, den = 0.0;
        for (int j = 0; j < B; ++j) {
            const float a = fabsf(v[j]);
            const float y = round_elem<EK>(quotient<SCALE_F16, false>(a, s, r));
            const double o = WEIGHTED ? (double)om[j] : 1.0;
            num += (o * (double)a) * (double)y;
            den += (o * (double)y) * (double)y;
        }
        if (den == 0.0) break;
        const int next = f16_round_code(num / den);
        if (next == code) break;
        code = next;
        s = scale_value(SCALE_F16, code);
        const double obj = gq_objective<EK, SCALE_F16, WEIGHTED>(v, om, B, s, s != 0.0f ? 1.0f / s : 0.0f);
        if (obj < best) {
            best = obj;
            best_code = code;
        }
    }
    return best_code;
}

// One panel [p0, p0 + 64 SEGP) of the column loop: one wave per row, four
// rows per workgroup, each lane holding SEGP consecutive float64 working
// values.  A column is encoded from its working value rounded to float32 (as
// the scale choice sees it); its error e = w - q is taken in float64.
template <int EK, int SK, int KIND, bool WEIGHTED, int SEGP>
__global__ __launch_bounds__(256) void gptq_panel_kernel(double *__restrict__ Wp, const double *__restrict__ V,
                                                         const float *__restrict__ hp, const int *__restrict__ col,
                                                         int64_t N, int64_t K, int B, int64_t p0, int ocp,
                                                         uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                         double *__restrict__ E)
{
    constexpr int BL = 64 * SEGP;
    __shared__ float blk[4][256 + 4];
    __shared__ float oms[256];
    const int tid = threadIdx.x, r = tid / 64, l = tid % 64;
    const int64_t n = (int64_t)blockIdx.x * 4 + r;
    const bool active = n < N;
    const int64_t pe = min(p0 + BL, K);
    const int64_t nb = K / B;

    double w[SEGP];
#pragma unroll
    for (int i = 0; i < SEGP; ++i) {
        const int64_t c = p0 + l * SEGP + i;
        w[i] = (active && c < pe) ? Wp[n * K + c] : 0.0;
    }
    // vp[u][i]: V[c][p0 + l SEGP + i] for the next column c = u (mod 4)
    double vp[4][SEGP];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < SEGP; ++i) {
            const int64_t c = p0 + u, k = p0 + l * SEGP + i;
            vp[u][i] = (c < pe && k > c && k < pe) ? V[c * K + k] : 0.0;
        }
    for (int64_t cs = p0; cs < pe; cs += B) {
        // the block's current values, and its h
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SEGP; ++i) {
            const int64_t c = p0 + l * SEGP + i;
            if (c >= cs && c < cs + B) blk[r][c - cs] = (float)w[i];
        }
        if (WEIGHTED)
            for (int j = tid; j < B; j += 256) oms[j] = hp[cs + j];
        __syncthreads();
        const float *v = blk[r];
        int code;
        if (KIND == GQ_NAIVE) {
            float amax = 0.0f;
            for (int j = l; j < B; j += 64) amax = fmaxf(amax, fabsf(v[j]));
            amax = group_max<64>(amax);
            if constexpr (SK == SCALE_E8M0)
                code = ocp ? ocp_code<EK>(amax) : naive_code<EK, SK>(amax);
            else
                code = naive_code<EK, SK>(amax);
        } else if (KIND == GQ_ALT) {
            code = l == 0 ? gq_alternation<EK, WEIGHTED>(v, oms, B) : 0;
            code = __shfl(code, 0, 64);
        } else {
            // full-grid argmin: lane l takes candidates c0 + l, c0 + l + 64, ...
            constexpr int C0 = cand_first(SK), C1 = cand_last(SK);
            double best = __builtin_huge_val();
            int bc = C1 + 1;
            for (int c = C0 + l; c <= C1; c += 64) {
                const float s = scale_value(SK, c);
                const double o = gq_objective<EK, SK, WEIGHTED>(v, oms, B, s, 1.0f / s);
                if (o < best) {
                    best = o;
                    bc = c;
                }
            }
            // lexicographic (objective, code) minimum over the wave
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const double ob = __shfl_xor(best, m, 64);
                const int oc = __shfl_xor(bc, m, 64);
                if (ob < best || (ob == best && oc < bc)) {
                    best = ob;
                    bc = oc;
                }
            }
            code = bc;
        }
        const float s = scale_value(SK, code);
        const float rs = s != 0.0f ? 1.0f / s : 0.0f;
        if (active && l == 0) store_scale<SK>(scales, n * nb + col[cs] / B, code);
        // encode the block's columns in order; each error goes to the later
        // columns of the panel held by the row's lanes.  The row of V each
        // column needs is loaded four columns ahead (B is a multiple of 4).
        uint32_t lo = 0;
        for (int64_t c4 = cs; c4 < cs + B; c4 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t c = c4 + u;
                const int own = (int)((c - p0) / SEGP), slot = (int)((c - p0) % SEGP);
                double e = 0.0;
                if (l == own) {
                    double wd = 0.0;
#pragma unroll
                    for (int i = 0; i < SEGP; ++i)
                        if (i == slot) wd = w[i];
                    const float wv = (float)wd;
                    const float a = fabsf(wv);
                    const float x = s != 0.0f ? quotient<SK, false>(a, s, rs) : 0.0f;
                    const float y = round_elem<EK>(x);
                    const float wq = s * y;
                    e = wd - (double)(__builtin_signbitf(wv) ? -wq : wq);
                    const uint32_t cd = elem_code<EK>(elem_index<EK>(y), __builtin_signbitf(wv) != 0);
                    if (active) {
                        E[n * BL + (c - p0)] = e;
                        const int64_t oc = col[c];
                        if (elem_4bit(EK)) {
                            if ((c & 1) == 0)
                                lo = cd & 15u;
                            else
                                codes[n * (K / 2) + oc / 2] = (uint8_t)(lo | ((cd & 15u) << 4));
                        } else {
                            codes[n * K + oc] = (uint8_t)cd;
                        }
                    }
                }
                e = __shfl(e, own, 64);
#pragma unroll
                for (int i = 0; i < SEGP; ++i) {
                    const int64_t k = p0 + l * SEGP + i;
                    if (k > c && k < pe) w[i] = __builtin_fma(-e, vp[u][i], w[i]);
                }
                // the V row of column c + 4
                const int64_t cn = c + 4;
#pragma unroll
                for (int i = 0; i < SEGP; ++i) {
                    const int64_t k = p0 + l * SEGP + i;
                    vp[u][i] = (cn < pe && k > cn && k < pe) ? V[cn * K + k] : 0.0;
                }
            }
        }
    }
}

// ------------------------------------------------------------ launchers ---

static int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t gptq_hessian_ws(int64_t M, int64_t K)
{
    if (K % 8 == 0) return 256;  // nothing is staged: X is read in place
    const int64_t M8 = (M + 7) / 8 * 8;
    return al256(K * M8 * 2) + al256(output_gemm_parts_bytes(K, K));
}

// col[k] = k (the sequential order); info[0] = 0.
__global__ __launch_bounds__(256) void gptq_iota_kernel(int *__restrict__ col, int64_t K, int *__restrict__ info)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k < K) col[k] = (int)k;
    if (k == 0) info[0] = 0;
}

__global__ void gptq_copy_int_kernel(const int *__restrict__ src, int *__restrict__ dst)
{
    if (threadIdx.x == 0) dst[0] = src[0];
}

__global__ __launch_bounds__(256) void gptq_zero_kernel(float *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

hipError_t launch_gptq_hessian(const void *X, int64_t M, int64_t K, float *H, void *ws, hipStream_t st)
{
    if (M == 0) {  // no rows: H = 0
        gptq_zero_kernel<<<1024, 256, 0, st>>>(H, K * K);
        return hipGetLastError();
    }
    // K % 8 == 0: the lower tile triangle of X^T X, read from row-major X,
    // each element stored with its mirror; otherwise X^T is staged and the
    // full product computed
    if (K % 8 == 0) return launch_gram_store(X, M, K, H, st);
    const int64_t M8 = (M + 7) / 8 * 8;
    uint16_t *Xt = static_cast<uint16_t *>(ws);
    double *part = reinterpret_cast<double *>(static_cast<char *>(ws) + al256(K * M8 * 2));
    const dim3 tg((unsigned)((K + 63) / 64), (unsigned)((M8 + 63) / 64));
    gptq_transpose_kernel<<<tg, 256, 0, st>>>(static_cast<const uint16_t *>(X), M, K, M8, Xt);
    return launch_gemm_store(Xt, Xt, K, K, M8, H, part, st);
}

// Workspace of launch_gptq (bytes), carved in this order.
struct GqLayout {
    int64_t P, Li, T, T2, V, Wp, E, h, hp, col, perm, loss, stat, info, sc, bytes;
};
static GqLayout gq_layout(int B, int64_t N, int64_t K)
{
    GqLayout L;
    const int64_t nb = K / B, BL = B > 128 ? 256 : 128, h1 = (K / 2 + 63) / 64 * 64;
    int64_t o = 0;
    L.P = o; o += al256(K * K * 8);
    L.Li = o; o += al256(K * K * 8);
    L.T = o; o += al256(h1 * h1 * 8);
    L.T2 = o; o += al256(K * K * 8 / 2);
    L.V = o; o += al256(K * K * 8);
    L.Wp = o; o += al256(N * K * 8);
    L.E = o; o += al256(N * BL * 8);
    L.h = o; o += al256(K * 4);
    L.hp = o; o += al256(K * 4);
    L.col = o; o += al256(K * 4);
    L.perm = o; o += al256(nb * 4);
    L.loss = o; o += al256(nb * 8);
    L.stat = o; o += 256;
    L.info = o; o += 256;
    L.sc = o; o += al256(N * nb * 2);
    L.bytes = o;
    return L;
}
int64_t gptq_ws(int B, int64_t N, int64_t K) { return gq_layout(B, N, K).bytes; }

template <int EK, int SK, int KIND, bool WEIGHTED>
static void gq_panel(double *Wp, const double *V, const float *hp, const int *col, int64_t N, int64_t K, int B,
                     int64_t p0, int ocp, uint8_t *codes, uint8_t *scales, double *E, hipStream_t st)
{
    const unsigned g = (unsigned)((N + 3) / 4);
    if (B > 128)
        gptq_panel_kernel<EK, SK, KIND, WEIGHTED, 4><<<g, 256, 0, st>>>(Wp, V, hp, col, N, K, B, p0, ocp, codes,
                                                                         scales, E);
    else
        gptq_panel_kernel<EK, SK, KIND, WEIGHTED, 2><<<g, 256, 0, st>>>(Wp, V, hp, col, N, K, B, p0, ocp, codes,
                                                                         scales, E);
}

template <int EK, int SK>
static void gq_panel_m(int method, double *Wp, const double *V, const float *hp, const int *col, int64_t N,
                       int64_t K, int B, int64_t p0, uint8_t *codes, uint8_t *scales, double *E, hipStream_t st)
{
    if (method == HD_NAIVE || method == HD_NAIVE_OCP) {
        gq_panel<EK, SK, GQ_NAIVE, false>(Wp, V, hp, col, N, K, B, p0, method == HD_NAIVE_OCP, codes, scales, E,
                                          st);
        return;
    }
    constexpr int KIND = SK == SCALE_F16 ? GQ_ALT : GQ_GRID;
    if (method == HD_H_OPT)
        gq_panel<EK, SK, KIND, true>(Wp, V, hp, col, N, K, B, p0, 0, codes, scales, E, st);
    else
        gq_panel<EK, SK, KIND, false>(Wp, V, hp, col, N, K, B, p0, 0, codes, scales, E, st);
}

template <int EK, int SK>
static void gq_loss(const void *W, int wdt, int64_t N, int64_t K, int B, const float *h, const uint8_t *sc,
                    double *loss, hipStream_t st)
{
    const unsigned nb = (unsigned)(K / B);
    if (wdt == HD_BF16)
        gptq_block_loss_kernel<EK, SK, uint16_t><<<nb, 256, 0, st>>>(static_cast<const uint16_t *>(W), N, K, B, h,
                                                                     sc, loss);
    else
        gptq_block_loss_kernel<EK, SK, float><<<nb, 256, 0, st>>>(static_cast<const float *>(W), N, K, B, h, sc,
                                                                  loss);
}

template <int EK, int SK>
static hipError_t gq_run(int method, int B, const void *W, int wdt, int64_t N, int64_t K, const float *H, double damp,
                         int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int *info_out, void *ws,
                         int fmt, const double *Vg, const int *info_g, hipStream_t st)
{
    const GqLayout L = gq_layout(B, N, K);
    char *base = static_cast<char *>(ws);
    double *P = reinterpret_cast<double *>(base + L.P), *Li = reinterpret_cast<double *>(base + L.Li);
    double *T = reinterpret_cast<double *>(base + L.T), *T2 = reinterpret_cast<double *>(base + L.T2);
    double *V = reinterpret_cast<double *>(base + L.V), *Wp = reinterpret_cast<double *>(base + L.Wp);
    double *E = reinterpret_cast<double *>(base + L.E);
    float *h = reinterpret_cast<float *>(base + L.h);
    float *hp = reinterpret_cast<float *>(base + L.hp);
    int *col = reinterpret_cast<int *>(base + L.col), *perm = reinterpret_cast<int *>(base + L.perm);
    double *loss = reinterpret_cast<double *>(base + L.loss), *stat = reinterpret_cast<double *>(base + L.stat);
    int *info = info_out ? info_out : reinterpret_cast<int *>(base + L.info);
    uint8_t *sc = reinterpret_cast<uint8_t *>(base + L.sc);
    const int64_t nb = K / B;

    gptq_diag_kernel<<<1, 256, 0, st>>>(H, K, damp, h, stat);
    hipError_t e = hipSuccess;
    if (ordered) {
        // the method's own scales on W, then the h-weighted loss per block column
        const float *hh = method == HD_H_OPT ? h : nullptr;
        if (method == HD_NAIVE || method == HD_NAIVE_OCP)
            e = launch_encode(fmt, B, W, wdt, N, K, nullptr, nullptr, codes, sc, nullptr, method == HD_NAIVE_OCP,
                              st);
        else if (SK == SCALE_F16)
            e = launch_alt_f16(fmt, B, W, wdt, N, K, hh, codes, sc, nullptr, st);
        else
            e = launch_search(fmt, B, W, wdt, N, K, hh, codes, sc, nullptr, nullptr, st);
        if (e != hipSuccess) return e;
        gq_loss<EK, SK>(W, wdt, N, K, B, h, sc, loss, st);
    }
    gptq_rank_kernel<<<1, 256, 0, st>>>(loss, nb, ordered, perm, block_order, info);
    {
        const dim3 g((unsigned)((K + 255) / 256), (unsigned)std::min<int64_t>(N > 0 ? N : 1, 4096));
        if (wdt == HD_BF16)
            gptq_gather_kernel<uint16_t><<<g, 256, 0, st>>>(static_cast<const uint16_t *>(W), N, K, B, perm, h, col,
                                                            hp, Wp);
        else
            gptq_gather_kernel<float><<<g, 256, 0, st>>>(static_cast<const float *>(W), N, K, B, perm, h, col, hp,
                                                         Wp);
    }
    if (Vg != nullptr) {
        // a factor of the sequential order made by gptq_factor: its status, its V
        gptq_copy_int_kernel<<<1, 64, 0, st>>>(info_g, info);
        V = const_cast<double *>(Vg);
    } else {
        gptq_build_p_kernel<<<dim3((unsigned)((K + 255) / 256), (unsigned)K), 256, 0, st>>>(H, K, col, stat, P);
        // the recursion multiplies by whole diagonal blocks of L^-1, whose upper
        // off-diagonal parts it never writes: they must read as zero
        gptq_zero_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<float *>(Li), 2 * K * K);
        cholinv(P, Li, K, 0, K, T, T2, info, st);
        gptq_build_v_kernel<<<dim3((unsigned)((K + 255) / 256), (unsigned)K), 256, 0, st>>>(Li, K, V);
    }
    const int BL = B > 128 ? 256 : 128;
    for (int64_t p0 = 0; p0 < K; p0 += BL) {
        const int64_t pe = std::min<int64_t>(p0 + BL, K);
        gq_panel_m<EK, SK>(method, Wp, V, hp, col, N, K, B, p0, codes, scales, E, st);
        // the panel's errors into every later column: Wp[:, pe:] -= E V[p0:pe, pe:]
        // (beta = 1, alpha = -1: one float64 rounding per entry)
        if (pe < K)
            dgemm<false>(N, K - pe, pe - p0, -1.0, E, pe - p0, V + p0 * K + pe, K, 1.0, Wp + pe, K, 0, st);
    }
    return hipGetLastError();
}

// The float64 factor V of the sequential order, made once for every GPTQ
// call that shares H and the damping: V (what the column loop reads) at byte
// GQ_FACTOR_V of the factor buffer, the factorisation's status (0, or 1 + the
// first non-positive pivot) at byte 0.
static constexpr int64_t GQ_FACTOR_V = 256;
int64_t gptq_factor_bytes(int64_t K) { return GQ_FACTOR_V + al256(K * K * 8); }
int64_t gptq_factor_ws(int64_t K) { return gptq_ws(32, 0, K); }

hipError_t launch_gptq_factor(const float *H, int64_t K, double damp, void *factor, int *info_out, void *ws,
                              hipStream_t st)
{
    const GqLayout L = gq_layout(32, 0, K);
    char *base = static_cast<char *>(ws);
    double *P = reinterpret_cast<double *>(base + L.P), *Li = reinterpret_cast<double *>(base + L.Li);
    double *T = reinterpret_cast<double *>(base + L.T), *T2 = reinterpret_cast<double *>(base + L.T2);
    float *h = reinterpret_cast<float *>(base + L.h);
    int *col = reinterpret_cast<int *>(base + L.col);
    double *stat = reinterpret_cast<double *>(base + L.stat);
    int *info = static_cast<int *>(factor);
    double *V = reinterpret_cast<double *>(static_cast<char *>(factor) + GQ_FACTOR_V);
    gptq_diag_kernel<<<1, 256, 0, st>>>(H, K, damp, h, stat);
    gptq_iota_kernel<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(col, K, info);
    gptq_build_p_kernel<<<dim3((unsigned)((K + 255) / 256), (unsigned)K), 256, 0, st>>>(H, K, col, stat, P);
    gptq_zero_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<float *>(Li), 2 * K * K);
    cholinv(P, Li, K, 0, K, T, T2, info, st);
    gptq_build_v_kernel<<<dim3((unsigned)((K + 255) / 256), (unsigned)K), 256, 0, st>>>(Li, K, V);
    if (info_out) gptq_copy_int_kernel<<<1, 64, 0, st>>>(info, info_out);
    return hipGetLastError();
}

static hipError_t gq_dispatch(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                              const float *H, double damp, int ordered, uint8_t *codes, uint8_t *scales,
                              int32_t *block_order, int *info, void *ws, const double *Vg, const int *info_g,
                              hipStream_t st);

hipError_t launch_gptq(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *H,
                       double damp, int ordered, uint8_t *codes, uint8_t *scales, int32_t *block_order, int *info,
                       void *ws, hipStream_t st)
{
    return gq_dispatch(method, fmt, B, W, wdt, N, K, H, damp, ordered, codes, scales, block_order, info, ws, nullptr,
                       nullptr, st);
}

hipError_t launch_gptq_factored(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                                const float *H, const void *factor, uint8_t *codes, uint8_t *scales,
                                int32_t *block_order, int *info, void *ws, hipStream_t st)
{
    const int *info_g = static_cast<const int *>(factor);
    const double *Vg = reinterpret_cast<const double *>(static_cast<const char *>(factor) + GQ_FACTOR_V);
    return gq_dispatch(method, fmt, B, W, wdt, N, K, H, 0.0, 0, codes, scales, block_order, info, ws, Vg, info_g,
                       st);
}

static hipError_t gq_dispatch(int method, int fmt, int B, const void *W, int wdt, int64_t N, int64_t K,
                              const float *H, double damp, int ordered, uint8_t *codes, uint8_t *scales,
                              int32_t *block_order, int *info, void *ws, const double *Vg, const int *info_g,
                              hipStream_t st)
{
#define HD_GQ_FMT(F)                                                                                          \
    case F:                                                                                                   \
        return gq_run<elem_kind(F), scale_kind(F)>(method, B, W, wdt, N, K, H, damp, ordered, codes, scales, \
                                                   block_order, info, ws, F, Vg, info_g, st);
    switch (fmt) {
        HD_GQ_FMT(HD_INT8_E4M3)
        HD_GQ_FMT(HD_NVFP4)
        HD_GQ_FMT(HD_MXFP4)
        HD_GQ_FMT(HD_MXFP8)
        HD_GQ_FMT(HD_FP8_E4M3S)
        HD_GQ_FMT(HD_NVFP4_UE4M4)
        HD_GQ_FMT(HD_NVFP4_UE5M3)
        HD_GQ_FMT(HD_NVINT4)
        HD_GQ_FMT(HD_FP4_F16)
        HD_GQ_FMT(HD_INT4_F16)
    }
#undef HD_GQ_FMT
    return hipErrorInvalidValue;
}

}  // namespace hd
