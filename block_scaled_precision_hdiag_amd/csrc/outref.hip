// outref.hip - output error of many quantisations of one W against one X
// (qwantize "Results", metric definitions: ||X Wq^T - X W^T||_F / ||X W^T||_F),
// one bf16/fp16 MFMA product per quantisation, directly (X Wq^T - Y) or
// through G = X^T X (output_gram and the C E^T walk below).
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
//   - the X^T X products (output_gram()'s scaled float16 triangle, and the
//     GPTQ Hessian's mirrored float32 matrix) stage rows of X itself (the
//     reduction index) and read the MFMA fragments with the LDS transpose
//     read ds_read_b64_tr_b16 (two per fragment), so X needs no transposed
//     copy;
//   - tile order: the workgroups one XCD runs at once cover 8 X tiles for each
//     weight tile, so they share X and weight panels in that XCD's L2;
//   - when the last round of tiles would fill at most half of the CUs, those
//     tiles run as 256 x 128 halves (a second launch), so that round takes
//     about half a tile's time.
#include <algorithm>
#include <cstdlib>

#include "common.hpp"
#include "formats.hpp"
#include "hdiag.h"
#include "kernels.hpp"

namespace hd {

typedef __bf16 ob16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 oh16x8_t __attribute__((ext_vector_type(8)));
typedef float of32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 ob16x4_t __attribute__((ext_vector_type(4)));

// Permutation of the 32-byte pairs of a staged X row by its residue mod 4
// (XOR with 0, 3, 5, 6): the 4 rows one 16-lane group reads at one pair
// position land on 4 different pairs mod 4, and the 8 rows x 2 pairs of one
// wave read on 8 different pairs mod 8.
__device__ __forceinline__ constexpr int tr_sig(int r) { return (0x6530 >> (4 * r)) & 15; }

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

enum { GE_STORE_Y = 0, GE_SUB_Y = 1, GE_GRAM = 2, GE_QUAD = 3, GE_SYRK = 4 };
// GRAM and SYRK read X^T from row-major X through the LDS transpose reads
template <int MODE>
static constexpr bool ge_tr = MODE == GE_GRAM || MODE == GE_SYRK;

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

// Arguments of gemm_err_kernel.  acc = A B^T over the K range of a work item,
// for 16-bit A [M][K] and B [N][K] (row pitch K, K % 8 == 0).
struct GeArgs {
    const uint16_t *A, *B;
    int64_t M, N, K;
    int mt, nt;        // 256-row tiles of A and of B
    int lin0, nlin;    // work items of this launch: lin0 .. lin0 + nlin - 1
    int split;         // STORE_Y / SUB_Y: two half-width workgroups per tile
    float *Y;          // STORE_Y (written) / SUB_Y (read): float [M][N]
    const int *erow;   // SUB_Y: exponent per row of A (may be NULL); QUAD: per row of B (E)
    double fscale;     // SUB_Y
    const float *r;    // GRAM: 1 / sqrt(h) per row of A (A = B)
    uint16_t *C;       // GRAM: float16 [N][N] output
    double *part;      // per-workgroup partials, pairs of doubles (not GRAM)
    int qa, qe;        // QUAD: bands per panel, E tiles per E group
    int qg, qper;      // QUAD: gangs, workgroup slots per gang
    int64_t qcpg;      // QUAD: panel columns per E group
    int64_t qcols;     // QUAD: panel columns in all (E groups x qcpg)
    int pbase;
};

// Work items and their epilogues, by MODE.
//   STORE_Y, SUB_Y: the A x B product is cut into 256 x 256 tiles, numbered in
//     a grouped order (GE_GROUP_M A tiles per B tile); one workgroup per tile,
//     or, when `split` is set (half-width configuration), two workgroups per
//     tile, each taking 128 of its 256 B rows (the last, partial round of
//     tiles then fills twice as many CUs).  Epilogue:
//       STORE_Y: Y[m][n] = acc, partial {0, sum acc^2};
//       SUB_Y:   d = acc f_m - Y[m][n] with f_m = fscale 2^erow[m] (f_m = 1
//                when erow is NULL), partial {sum d^2, 0}.
//   GRAM, SYRK (A = B = X^T read from row-major X [K][M], K the reduction
//     length and pitch M, so acc = X^T X): the tiles (tm, tn) with tn <= tm of
//     the lower triangle, in groups of GE_GROUP_M tile rows (column-major
//     inside a group).  Epilogue: GRAM: C[n][m] = fp16(f acc[m][n] r[m]
//     r[n]) (the transposed position, so C holds the upper block triangle),
//     f = 2 off the diagonal tiles, 1 on them, and C[m][m] = 0; SYRK:
//     Y[m][n] = Y[n][m] = acc[m][n] (float32) from the elements with m >= n.
//   QUAD (A = the C of GRAM, M = K; B = E [N][K], the rows of one or more
//     quantisations): persistent workgroups in qg gangs of qper slots; slot
//     sl of a gang is band offset qb = sl / qe and E tile offset qu = sl % qe
//     (slots past qa qe idle).  The work is cut into E groups of qe E tiles
//     and, within each, panels of qa bands of C; panel i has the columns
//     (K blocks) J = qa i .. mt - 1.  Gang x walks the x-th of qg equal runs
//     of all (E group, panel, column) in order, each member doing band
//     qa i + qb of E tile g qe + qu at the columns where J >= band, so the
//     members read the same qa C blocks and qe E blocks of a column at the
//     same time (a gang is one XCD's worth of workgroups).  acc[m][e] =
//     (E C)[e][m] for the C rows m of the band; when the tile (band, E tile)
//     changes or the run ends, sum acc[m][e] E[e][m] 4^erow[e] over the tile
//     goes to part[(E tile mt + band) qg + gang] (zeroed beforehand) and acc
//     restarts at zero.  Summed over an E row range, the slots give that
//     range's E C E^T trace with C's upper block triangle standing for both
//     halves.  Returns without the partial pair below.
// Consecutive workgroup indices go to different XCDs; the index is remapped
// so that each XCD runs a contiguous run of item numbers.  Workgroup w writes
// its partial to part[2 (pbase + w) .. + 1].
template <bool F16, int MODE, int TK, int S, int WN, int NJ>
__global__ __launch_bounds__(128 * WN, 1) void gemm_err_kernel(const GeArgs ga)
{
    typedef GeCfg<TK, S, WN, NJ> C;
    typedef typename Mfma16<F16>::v V;
    extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
    __shared__ double red[2][C::NW];
    const uint16_t *__restrict__ A = ga.A;
    const uint16_t *__restrict__ Bm = ga.B;
    const int64_t M = ga.M, N = ga.N, K = ga.K;

    const int hw = blockIdx.x;
    int lin, half = 0;
    if (ga.split) {
        lin = ga.lin0 + hw / 2;
        half = hw & 1;
    } else {
        const int per = ga.nlin / 8;
        lin = ga.lin0 + (hw < per * 8 ? (hw % 8) * per + hw / 8 : hw);
    }
    int64_t m0, n0, kb = 0, ke = K;
    float fold = 1.0f;
    int64_t qc0 = 0, qc1 = 0;  // QUAD: this workgroup's panel columns
    int qb = 0, qu = 0, qx = 0;  // QUAD: band offset, E tile offset, gang
    if (MODE == GE_GRAM || MODE == GE_SYRK) {
        int g0 = 0, base = 0, gm = 0;
        for (;;) {
            gm = min(GE_GROUP_M, ga.mt - g0);
            const int cnt = g0 * gm + gm * (gm + 1) / 2;
            if (lin < base + cnt) break;
            base += cnt;
            g0 += GE_GROUP_M;
        }
        int w = lin - base, tm, tn;
        if (w < g0 * gm) {
            tn = w / gm;
            tm = g0 + w % gm;
        } else {
            w -= g0 * gm;
            int c = 0;
            while (w >= gm - c) {
                w -= gm - c;
                ++c;
            }
            tn = g0 + c;
            tm = tn + w;
        }
        m0 = (int64_t)tm * GE_TM;
        n0 = (int64_t)tn * GE_TN;
        fold = tm != tn ? 2.0f : 1.0f;
    } else if (MODE == GE_QUAD) {
        // gang qx = lin / qper, slot sl: band offset qb = sl / qe, E tile
        // offset qu = sl % qe (slots past qa qe idle); the gang's run of
        // panel columns is [qc0, qc1)
        const int sl = lin % ga.qper;
        qx = lin / ga.qper;
        qb = sl / ga.qe;
        qu = sl % ga.qe;
        qc0 = ga.qcols * qx / ga.qg;
        qc1 = sl < ga.qa * ga.qe ? ga.qcols * (qx + 1) / ga.qg : qc0;
        m0 = 0;
        n0 = 0;
    } else {
        const int group = lin / (GE_GROUP_M * ga.nt);
        const int first_m = group * GE_GROUP_M;
        const int gm = min(ga.mt - first_m, GE_GROUP_M);
        const int within = lin % (GE_GROUP_M * ga.nt);
        const int tm = first_m + within % gm;
        const int tn = within / gm;
        m0 = (int64_t)tm * GE_TM;
        n0 = (int64_t)tn * GE_TN + (int64_t)half * C::TN;
    }

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
    //
    // GRAM stages rows of X itself (A = B = X^T, read without a transposed
    // copy): stage row r is X row k0 + r (the reduction index), 256 columns
    // (m0 .. m0 + 255 for A, n0 .. n0 + 255 for B), 512 bytes.  Lane l of
    // the wave's i-th instruction fills row r = 2 (NW i + wv) + l / 32,
    // 16-byte slot l % 32, with chunk c = 2 ((slot / 2) ^ tr_sig(r % 4)) +
    // slot % 2 of those columns: the 32-byte pairs of a row are permuted by
    // the row's residue mod 4 so that the transposed fragment reads (GE_FRAG
    // below: 4 rows x 32 bytes per 16 lanes, 8 rows x 64 bytes per wave)
    // spread over the banks.  Rows past K (the reduction length) and columns
    // past M / N are read as zeros.
    const int lrow = lane / C::CPR, slot = lane % C::CPR;
    int64_t aoff[C::DA], boff[C::DB];
    int acs[C::DA], bcs[C::DB];
    // GRAM: the i-th instruction's row is tr_r0 + 2 NW i, a multiple of 4
    // past tr_r0, so its chunk permutation, and hence its column, is the
    // instruction-0 one: one column offset per operand (tr_ok*: not past M / N).
    const int tr_r0 = 2 * wv + (lane >> 5);
    int64_t tr_a = 0, tr_b = 0;
    bool tr_oka = false, tr_okb = false;
    const uintptr_t tr_zero = (uintptr_t)ge_zero16;
    if (ge_tr<MODE>) {
        static_assert(!ge_tr<MODE> || (C::TN == GE_TN && C::DA * 2 * C::NW == TK && C::DB * 2 * C::NW == TK &&
                                          (2 * C::NW) % 4 == 0),
                      "GRAM staging: full 256 x 256 tiles, 2 rows per instruction");
        const int ts = lane & 31;
        const int c = (((ts >> 1) ^ tr_sig(tr_r0 & 3)) << 1) | (ts & 1);
        tr_oka = m0 + 8 * c < M;
        tr_okb = n0 + 8 * c < N;
        tr_a = tr_oka ? (int64_t)tr_r0 * M + m0 + 8 * c : 0;
        tr_b = tr_okb ? (int64_t)tr_r0 * N + n0 + 8 * c : 0;
    } else {
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
    // GRAM: X rows k0 + acs[i] (zeros past K, the reduction length, and for
    // columns past M); the same LDS placement as GE_ISSUE (1 KB per
    // instruction, 2 rows of 512 bytes)
#define GE_ISSUE_T(k0, buf)                                                                            \
    do {                                                                                               \
        uint16_t *sa_ = glds + (buf) * C::STAGE + wv * C::RPI * TK;                                    \
        uint16_t *sb_ = sa_ + GE_TM * TK;                                                              \
        const int64_t kr_ = (int64_t)(k0) + tr_r0;                                                     \
        const uint16_t *pa_ = A + tr_a + (int64_t)(k0) * M;                                            \
        const uint16_t *pb_ = Bm + tr_b + (int64_t)(k0) * N;                                           \
        _Pragma("unroll") for (int i = 0; i < C::DA; ++i)                                              \
        {                                                                                              \
            const bool ok_ = tr_oka & (kr_ + 2 * C::NW * i < K);                                       \
            const uintptr_t p_ = ok_ ? (uintptr_t)(pa_ + (int64_t)(2 * C::NW * i) * M) : tr_zero;     \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)p_, (ge_lds_void *)(sa_ + C::NW * i * C::RPI * TK), 16, 0, 0); \
        }                                                                                              \
        _Pragma("unroll") for (int i = 0; i < C::DB; ++i)                                              \
        {                                                                                              \
            const bool ok_ = tr_okb & (kr_ + 2 * C::NW * i < K);                                       \
            const uintptr_t p_ = ok_ ? (uintptr_t)(pb_ + (int64_t)(2 * C::NW * i) * N) : tr_zero;     \
            __builtin_amdgcn_global_load_lds((ge_gbl_void *)p_, (ge_lds_void *)(sb_ + C::NW * i * C::RPI * TK), 16, 0, 0); \
        }                                                                                              \
    } while (0)
#define GE_STAGE_IN(k0, buf)                                                                           \
    do {                                                                                               \
        if constexpr (ge_tr<MODE>)                                                                     \
            GE_ISSUE_T(k0, buf);                                                                       \
        else                                                                                           \
            GE_ISSUE(k0, buf);                                                                         \
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
    // GRAM (stage rows = reduction index): one fragment is two LDS
    // transpose reads (ds_read_b64_tr_b16).  In each 16-lane group g of the
    // wave, source lane s reads 4 consecutive columns 4 (s % 4) of stage row
    // 16 kk + 8 (g / 2) + 4 h + s / 4; the read hands output lane i the i-th
    // column of the group's 16 from those 4 rows, i.e. the 4 reduction
    // indices 8 (g / 2) + 4 h + 0..3 of MFMA row 16 (g % 2) + i: the A / B
    // operand layout of v_mfma_f32_32x32x16 (lane l: row l % 32, reduction
    // indices 8 (l / 32) .. + 7), h = 0 and 1 giving its two halves.
    const int tg = lane >> 4, trow = 8 * (tg >> 1) + ((lane & 15) >> 2), tq = lane & 3;
    const int tsig = tr_sig(((lane & 15) >> 2));
#define GE_TRV(bufp, row, sl)                                                                          \
    ({                                                                                                 \
        const auto lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                                    \
            (__attribute__((address_space(3))) ob16x4_t *)((bufp) + (row) * 256 + (((sl) ^ tsig) * 16) + 4 * tq)); \
        const auto hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                                    \
            (__attribute__((address_space(3))) ob16x4_t *)((bufp) + ((row) + 4) * 256 + (((sl) ^ tsig) * 16) + 4 * tq)); \
        __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7);                                   \
    })
#define GE_FRAG(set, bufp, kk)                                                                         \
    do {                                                                                               \
        if constexpr (ge_tr<MODE>) {                                                                   \
            const int row_ = 16 * (kk) + trow;                                                         \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                              \
                fa[set][i] = GE_TRV(bufp, row_, (wm * 128 + i * 32) / 16 + (tg & 1));                   \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                             \
                fb[set][j] = GE_TRV((bufp) + GE_TM * TK, row_, (wn * 32 * NJ + j * 32) / 16 + (tg & 1)); \
            break;                                                                                     \
        }                                                                                              \
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
    constexpr int D = C::DA + C::DB;
#define GE_COMPUTE(stage)                                                                              \
    do {                                                                                               \
        const uint16_t *base = glds + (stage) * C::STAGE;                                              \
        GE_FRAG(0, base, 0);                                                                           \
        _Pragma("unroll") for (int kk = 0; kk < TK / 16; ++kk)                                         \
        {                                                                                              \
            const int cur = kk & 1;                                                                    \
            if (kk + 1 < TK / 16) GE_FRAG(cur ^ 1, base, kk + 1);                                      \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                              \
                _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i][j] =                             \
                    Mfma16<F16>::op(fa[cur][i], fb[cur][j], acc[i][j]);                                \
        }                                                                                              \
    } while (0)
    double sd = 0.0, sy = 0.0;
    if (MODE == GE_QUAD) {
        // Persistent walk over this member's columns of [qc0, qc1): the
        // copies run S - 1 k-steps ahead across column, panel and E group
        // boundaries; when the tile (band, E tile) changes or the run ends,
        // the accumulators go through the epilogue, the workgroup's sum goes
        // to part[(E tile * mt + band) * qg + gang], and acc restarts at zero.
        // K block J has `full` k-steps, the last one (J = mt - 1) `last`.
        const int full = GE_TN / TK;
        const int last = (int)((K - (int64_t)(ga.mt - 1) * GE_TN + TK - 1) / TK);
        const int mt = ga.mt, qa = ga.qa, qe = ga.qe, nte = ga.nt;
        // cursor (c, E group g, panel i, K block J) on this member's valid
        // columns: band qa i + qb exists, J >= band, E tile g qe + qu exists
#define GE_QBAND(i) (qa * (i) + qb)
#define GE_QTILE(g) ((g) * qe + qu)
#define GE_QVALID(g, i, J) (GE_QBAND(i) < mt && (J) >= GE_QBAND(i) && GE_QTILE(g) < nte)
#define GE_QNEXT(c, g, i, J)                                                                           \
    do {                                                                                               \
        ++(c);                                                                                         \
        if (++(J) == mt) {                                                                             \
            ++(i);                                                                                     \
            (J) = qa * (i);                                                                            \
            if ((J) >= mt) {                                                                           \
                (i) = 0;                                                                               \
                (J) = 0;                                                                               \
                ++(g);                                                                                 \
            }                                                                                          \
        }                                                                                              \
    } while ((c) < qc1 && !GE_QVALID(g, i, J))
        int64_t cc = qc0;
        int cg = (int)(qc0 / ga.qcpg), ci = 0, cJ = 0;
        {
            int64_t r = qc0 % ga.qcpg;
            while (ci * qa < mt && r >= mt - qa * ci) {
                r -= mt - qa * ci;
                ++ci;
            }
            cJ = qa * ci + (int)r;
            if (cc < qc1 && !GE_QVALID(cg, ci, cJ)) GE_QNEXT(cc, cg, ci, cJ);
        }
        int64_t ic = cc;
        int ig = cg, ii = ci, iJ = cJ, ikk = 0, ckk = 0, atk = -1, btl = -1;
#define GE_QISSUE(buf)                                                                                 \
    do {                                                                                               \
        const int itk_ = GE_QBAND(ii), itl_ = GE_QTILE(ig);                                            \
        if (itk_ != atk) {                                                                             \
            atk = itk_;                                                                                \
            _Pragma("unroll") for (int i = 0; i < C::DA; ++i)                                          \
            {                                                                                          \
                const int r_ = (C::NW * i + wv) * C::RPI + lrow;                                       \
                aoff[i] = min((int64_t)itk_ * GE_TM + r_, M - 1) * K + acs[i];                         \
            }                                                                                          \
        }                                                                                              \
        if (itl_ != btl) {                                                                             \
            btl = itl_;                                                                                \
            _Pragma("unroll") for (int i = 0; i < C::DB; ++i)                                          \
            {                                                                                          \
                const int r_ = (C::NW * i + wv) * C::RPI + lrow;                                       \
                boff[i] = min((int64_t)itl_ * GE_TN + r_, N - 1) * K + bcs[i];                         \
            }                                                                                          \
        }                                                                                              \
        GE_ISSUE((int64_t)iJ * GE_TN + (int64_t)ikk * TK, buf);                                        \
        if (++ikk == (iJ < mt - 1 ? full : last)) {                                                    \
            ikk = 0;                                                                                   \
            GE_QNEXT(ic, ig, ii, iJ);                                                                  \
        }                                                                                              \
    } while (0)
        int inflight = 0, st = 0;
#pragma unroll
        for (int b = 0; b < S - 1; ++b)
            if (ic < qc1) {
                GE_QISSUE(b);
                ++inflight;
            }
        while (cc < qc1) {
            ge_wait_copies((inflight - 1) * D);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (ic < qc1) {
                GE_QISSUE((st + S - 1) % S);
                ++inflight;
            }
            GE_COMPUTE(st % S);
            --inflight;
            ++st;
            if (++ckk == (cJ < mt - 1 ? full : last)) {
                ckk = 0;
                const int ctk = GE_QBAND(ci), ctl = GE_QTILE(cg);
                GE_QNEXT(cc, cg, ci, cJ);
                if (cc >= qc1 || GE_QBAND(ci) != ctk || GE_QTILE(cg) != ctl) {
                    // epilogue of tile (ctk, ctl): acc[i][j][4 g + u] = (E C)[e][m + u]
                    // for the C rows m = mb0 + 32 i + 8 g and the E row
                    // e = nb0 + 32 j; times E[e][m .. m + 3] (one 8-byte load;
                    // the 16 loads of a row are in flight together), scaled by
                    // 4^erow[e]
                    const int64_t mb0 = (int64_t)ctk * GE_TM + wm * 128 + 4 * (lane >> 5);
                    const int64_t nb0 = (int64_t)ctl * GE_TN + wn * 32 * NJ + (lane & 31);
                    double sdl = 0.0;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int64_t e = nb0 + j * 32;
                        const int64_t ec = min(e, N - 1);
                        const uint16_t *er = Bm + ec * K;
                        uint2 ld[4][4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int g = 0; g < 4; ++g)
                                ld[i][g] = *reinterpret_cast<const uint2 *>(er + min(mb0 + i * 32 + 8 * g, M - 4));
                        double t = 0.0;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const uint32_t w2[2] = {ld[i][g].x, ld[i][g].y};
                                double q = 0.0;
#pragma unroll
                                for (int u = 0; u < 4; ++u) {
                                    const _Float16 ev =
                                        __builtin_bit_cast(_Float16, (uint16_t)(w2[u >> 1] >> (16 * (u & 1))));
                                    q += (double)acc[i][j][4 * g + u] * (double)(float)ev;
                                }
                                t = mb0 + i * 32 + 8 * g < M ? t + q : t;
                            }
                        if (e < N) sdl += ldexp(t, 2 * ga.erow[ec]);
                    }
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) sdl += __shfl_xor(sdl, o, 64);
                    if (lane == 0) red[0][wv] = sdl;
                    __syncthreads();
                    if (tid == 0) {
                        double a = 0.0;
#pragma unroll
                        for (int w = 0; w < C::NW; ++w) a += red[0][w];
                        ga.part[((int64_t)ctl * mt + ctk) * ga.qg + qx] = a;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
#pragma unroll
                            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
                }
            }
        }
#undef GE_QISSUE
#undef GE_QNEXT
#undef GE_QVALID
#undef GE_QTILE
#undef GE_QBAND
        return;
    } else {
        // Pipeline: the copies of stage ks + S - 1 are issued right after the
        // barrier that opens stage ks (that barrier also certifies that every
        // wave has finished reading the buffer they overwrite, the one of
        // stage ks - 1).  Before the barrier each wave waits for its own copies
        // of stage ks (the copies of later stages may stay in flight) and for
        // its LDS reads.
        const int ksteps = (int)((ke - kb + TK - 1) / TK);
#pragma unroll
        for (int p = 0; p < S - 1; ++p)
            if (p < ksteps) GE_STAGE_IN(kb + (int64_t)p * TK, p);
        for (int ks = 0; ks < ksteps; ++ks) {
            ge_wait_copies(min(S - 2, ksteps - 1 - ks) * D);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (ks + S - 1 < ksteps) GE_STAGE_IN(kb + (int64_t)(ks + S - 1) * TK, (ks + S - 1) % S);
            GE_COMPUTE(ks % S);
        }
    }
#undef GE_COMPUTE
#undef GE_FRAG
#undef GE_TRV
#undef GE_STAGE_IN
#undef GE_ISSUE_T
#undef GE_ISSUE

    // epilogue: accumulator v of lane l in a 32 x 32 tile is row
    // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
    const int64_t nb0 = n0 + wn * 32 * NJ + (lane & 31);
    const int64_t mb0 = m0 + wm * 128 + 4 * (lane >> 5);
    if (MODE == GE_GRAM) {
        // acc[i][j][4 g + u] = G[m + u][n] for m = mb0 + 32 i + 8 g (a multiple
        // of 4; M % 8 == 0, so m < M covers m + 3) and n = nb0 + 32 j: one
        // 8-byte store of C[n][m .. m + 3], the transposed position.
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = nb0 + j * 32;
            if (n >= N) continue;
            const float rn = ga.r[n] * fold;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t m = mb0 + i * 32 + 8 * g;
                    if (m >= M) continue;
                    const float4 rm = *reinterpret_cast<const float4 *>(ga.r + m);
                    const float rr[4] = {rm.x, rm.y, rm.z, rm.w};
                    uint32_t hv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float c = m + u == n ? 0.0f : acc[i][j][4 * g + u] * rr[u] * rn;
                        hv[u] = __builtin_bit_cast(uint16_t, (_Float16)c);
                    }
                    *reinterpret_cast<uint2 *>(ga.C + n * M + m) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
                }
        }
        return;
    }
    if (MODE == GE_SYRK) {
        // acc[i][j][4 g + u] = H[m + u][n] (m, n as for GRAM): the element and
        // its mirror H[n][m + u] are written from the lower triangle only
        // (m + u >= n; on the diagonal tiles the upper elements come from their
        // mirrors), so H is exactly symmetric.  Y: float [N][N].
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = nb0 + j * 32;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t m = mb0 + i * 32 + 8 * g;
                    if (m >= M || m + 3 < n) continue;
                    const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                        acc[i][j][4 * g + 3]};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (m + u >= n) ga.Y[(m + u) * N + n] = v[u];
                    if (m > n) {
                        *reinterpret_cast<float4 *>(ga.Y + n * N + m) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (m + u > n) ga.Y[n * N + m + u] = v[u];
                    }
                }
        }
        return;
    }
    if (MODE != GE_QUAD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // row exponents of this lane's 16 rows in tile row i (SUB with erow)
        int ev[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            ev[v] = (MODE == GE_SUB_Y && ga.erow != nullptr) ? ga.erow[min(mb0 + i * 32 + 8 * (v >> 2) + (v & 3), M - 1)] : 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = nb0 + j * 32;
            const bool nin = n < N;
            if (MODE == GE_STORE_Y) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = mb0 + i * 32 + 8 * (v >> 2) + (v & 3);
                    if (m < M && nin) {
                        const float y = acc[i][j][v];
                        ga.Y[m * N + n] = y;
                        sy = __builtin_fma((double)y, (double)y, sy);
                    }
                }
            } else {
                // the 16 reads of Y for this 32 x 32 tile are in flight together
                const int64_t nc = min(n, N - 1);
                float yv[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) yv[v] = ga.Y[min(mb0 + i * 32 + 8 * (v >> 2) + (v & 3), M - 1) * N + nc];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = mb0 + i * 32 + 8 * (v >> 2) + (v & 3);
                    const double f = ldexp(ga.fscale, ev[v]);
                    const double d = (double)acc[i][j][v] * f - (double)yv[v];
                    sd = (m < M && nin) ? __builtin_fma(d, d, sd) : sd;
                }
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
        ga.part[2 * (int64_t)(ga.pbase + hw)] = a;
        ga.part[2 * (int64_t)(ga.pbase + hw) + 1] = b;
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
template <bool F16, int MODE, int NJ, int TK = HD_GE_TK, int S = HD_GE_STAGES, int WN = HD_GE_WN>
static hipError_t ge_launch(const GeArgs &ga, int64_t grid, hipStream_t st)
{
    typedef GeCfg<TK, S, WN, NJ> C;
    if (grid <= 0) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void *)gemm_err_kernel<F16, MODE, TK, S, WN, NJ>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    if (e != hipSuccess) return e;
    gemm_err_kernel<F16, MODE, TK, S, WN, NJ><<<(unsigned)grid, C::THREADS, C::LDS, st>>>(ga);
    return hipGetLastError();
}

static GeArgs ge_args(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K)
{
    GeArgs ga = {};
    ga.A = A;
    ga.B = Bm;
    ga.M = M;
    ga.N = N;
    ga.K = K;
    ga.mt = (int)((M + GE_TM - 1) / GE_TM);
    ga.nt = (int)((N + GE_TN - 1) / GE_TN);
    ga.fscale = 1.0;
    return ga;
}

template <bool F16, int MODE>
static hipError_t launch_gemm_err(const uint16_t *A, const uint16_t *Bm, int64_t M, int64_t N, int64_t K,
                                  float *Y, const int *erow, double fscale, double *part, int64_t *nparts,
                                  hipStream_t st)
{
    constexpr int WN = HD_GE_WN, NJF = 8 / WN, NJH = 4 / WN;
    static_assert(GeCfg<HD_GE_TK, HD_GE_STAGES, WN, NJF>::TN == GE_TN &&
                      2 * GeCfg<HD_GE_TK, HD_GE_STAGES, WN, NJH>::TN == GE_TN,
                  "tile widths");
    GeArgs ga = ge_args(A, Bm, M, N, K);
    ga.Y = Y;
    ga.erow = erow;
    ga.fscale = fscale;
    ga.part = part;
    const int64_t T = (int64_t)ga.mt * ga.nt;
    *nparts = 0;
    if (T == 0) return hipSuccess;
    const int cus = device_cus();
    const int64_t rem = T % cus;
    const bool split = rem > 0 && 2 * rem <= cus;
    const int64_t nfull = split ? T - rem : T;
    ga.lin0 = 0;
    ga.nlin = (int)nfull;
    hipError_t e = ge_launch<F16, MODE, NJF>(ga, nfull, st);
    if (e != hipSuccess) return e;
    if (split) {
        ga.lin0 = (int)nfull;
        ga.nlin = (int)rem;
        ga.split = 1;
        ga.pbase = (int)nfull;
        e = ge_launch<F16, MODE, NJH>(ga, 2 * rem, st);
        if (e != hipSuccess) return e;
    }
    *nparts = nfull + (split ? 2 * rem : 0);
    return hipSuccess;
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

// ===================================================== output error by Gram ==
// ||X D^T||_F^2 = sum_n d_n^T G d_n with G = X^T X (D = Wq - W, or W itself
// for ||X W^T||^2): once G is known, each quantisation costs an N x K x K
// product instead of an M x N x K one (M = rows of X), and G's symmetry halves
// that.  With h = diag(G) and the scaled rows e_n = d_n sqrt(h):
//   d^T G d = sum_j d_j^2 h_j + e^T C e,   C = G / sqrt(h h^T) off the diagonal,
// where |C_jk| <= 1 (Cauchy-Schwarz).  The diagonal sum is taken exactly (in
// float64 from the float32 d and h); only the off-diagonal part goes through
// the float16 MFMA product, with C in float16 and e in float16 under one
// power-of-two scale per row.
//
// output_gram():   h (hdiag), sqrt(h), 1/sqrt(h) (0 for h = 0); X^T in the
//                  workspace; C's upper block triangle (256 x 256 blocks,
//                  diagonal blocks whole) from one bf16 MFMA product over
//                  half of the tiles, off-diagonal blocks stored as 2 C so
//                  that the upper triangle stands for both halves;
// output_error_gram(): e and the diagonal sums per row (one workgroup per
//                  row), then C E^T over each item's K range with the
//                  epilogue sum of acc * e, then a fixed-order final sum.

// h (copied unless it already is the buffer's), sqrt(h) and 1/sqrt(h) (0 for h = 0).
__global__ __launch_bounds__(256) void gram_prep_kernel(const float *__restrict__ hin, int64_t K, float *__restrict__ h,
                                                        float *__restrict__ sq, float *__restrict__ r)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    const float v = hin[k];
    if (hin != h) h[k] = v;
    const float q = sqrtf(v);
    sq[k] = q;
    r[k] = v > 0.0f ? 1.0f / q : 0.0f;
}

__global__ __launch_bounds__(256) void gram_zero_kernel(uint16_t *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// The raw memory of one 8-weight chunk at flat index e0 (a multiple of 8):
// the weights (16 bytes of bf16 in w0, or 32 bytes of float32 in w0, w1),
// the codes (8-bit: c.x, c.y; 4-bit: c.x) and the block's scale code (B is a
// power of two: block index by shift).  REF: the weights only.  Loading every
// chunk of a row before decoding any lets the row's loads overlap.
struct GramRaw {
    uint4 w0, w1;
    uint2 c;
    int sc;
};
template <int EK, int SK, typename WT, bool REF>
__device__ __forceinline__ void gram_load(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int B,
                                          const WT *__restrict__ W, int64_t e0, GramRaw &r)
{
    r.w0 = *reinterpret_cast<const uint4 *>(W + e0);
    if (sizeof(WT) == 4) r.w1 = *reinterpret_cast<const uint4 *>(W + e0 + 4);
    if (REF) return;
    const int64_t bi = e0 >> (31 - __builtin_clz((unsigned)B));
    r.sc = scale_bytes(SK) == 2 ? (int)reinterpret_cast<const uint16_t *>(scales)[bi] : (int)scales[bi];
    if (elem_4bit(EK))
        r.c.x = *reinterpret_cast<const uint32_t *>(codes + e0 / 2);
    else
        r.c = *reinterpret_cast<const uint2 *>(codes + e0);
}

// d = Wq - W for a loaded chunk (REF: d = W), with Wq the float32 values
// dequantize() gives (fl32(s val(q)); invalid codes give 0).  stab: the INT8
// grid's scale values per code (0 for invalid codes), unused on the other
// grids.
template <int EK, int SK, typename WT, bool REF>
__device__ __forceinline__ void gram_decode(const GramRaw &r, float d[8], const float *stab)
{
    float w[8];
    if (sizeof(WT) == 2) {
        const uint32_t u[4] = {r.w0.x, r.w0.y, r.w0.z, r.w0.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w[2 * j] = bf16_to_f32(u[j] & 0xFFFFu);
            w[2 * j + 1] = bf16_to_f32(u[j] >> 16);
        }
    } else {
        const uint32_t u[8] = {r.w0.x, r.w0.y, r.w0.z, r.w0.w, r.w1.x, r.w1.y, r.w1.z, r.w1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = __builtin_bit_cast(float, u[j]);
    }
    if (REF) {
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = w[j];
        return;
    }
    const int sc = r.sc;
    const float s = SK == SCALE_INT8 ? stab[sc & 127] * (sc < 128 ? 1.0f : 0.0f)
                                     : (scale_code_valid(SK, sc) ? scale_value(SK, sc) : 0.0f);
    uint32_t c[8];
    if (elem_4bit(EK)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (r.c.x >> (4 * j)) & 15u;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = (r.c.x >> (8 * j)) & 255u;
            c[4 + j] = (r.c.y >> (8 * j)) & 255u;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float q;
        if (EK == ELEM_INT8) {
            const int i = (int)(int8_t)(uint8_t)c[j];
            q = i == -128 ? 0.0f : s * (float)i;
        } else if (EK == ELEM_INT4) {
            const int i = (int)((c[j] ^ 8u) & 15u) - 8;
            q = i == -8 ? 0.0f : s * (float)i;
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
            q = neg ? -mag : mag;
        }
        d[j] = q - w[j];
    }
}

// One workgroup per row n: e = d sqrt(h) as float16 under the row exponent
// erow[n] (largest |e| scaled into [2^14, 2^15); 0 for a zero row), and
// dsum[n] = sum_j d_j^2 h_j in float64; rows n >= nvalid (the padding of E
// to whole 256-row tiles) are written as zeros.  RC > 0: the row's e values stay in
// registers (RC chunks of 8 per thread, K <= 2048 RC) between the row maximum
// and the float16 stores; RC = 0: a second pass recomputes them.
template <int EK, int SK, typename WT, bool REF, int RC>
__device__ __forceinline__ void gram_operand_row(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 int B, const WT *__restrict__ W, int64_t K,
                                                 const float *__restrict__ sq, const float *__restrict__ h,
                                                 uint16_t *__restrict__ E, int *__restrict__ erow,
                                                 double *__restrict__ dsum, int64_t nvalid, int64_t n)
{
    __shared__ double sh[4];
    __shared__ int shm[4];
    __shared__ float stab[128];  // the INT8 grid's scale values fl32(val / 127)
    if (n >= nvalid) {  // padding row of E: zeros
        for (int64_t c = threadIdx.x; c < K / 8; c += 256)
            *reinterpret_cast<uint4 *>(E + n * K + c * 8) = make_uint4(0u, 0u, 0u, 0u);
        if (threadIdx.x == 0) {
            erow[n] = 0;
            dsum[n] = 0.0;
        }
        return;
    }
    if (SK == SCALE_INT8 && !REF) {
        if (threadIdx.x < 128)
            stab[threadIdx.x] = scale_code_valid(SK, threadIdx.x) ? scale_value(SK, threadIdx.x) : 0.0f;
        __syncthreads();
    }
    const int64_t nch = K / 8;
    int mx = 0;  // largest |e| as float bits (monotone for non-negative floats)
    double ds = 0.0;
    float ek[RC > 0 ? RC : 1][8];
    // sqrt(h) and h of chunk c
    struct SqH {
        float4 q0, q1, h0, h1;
    };
    auto load_sqh = [&](int64_t c) {
        SqH v;
        v.q0 = *reinterpret_cast<const float4 *>(sq + c * 8);
        v.q1 = *reinterpret_cast<const float4 *>(sq + c * 8 + 4);
        v.h0 = *reinterpret_cast<const float4 *>(h + c * 8);
        v.h1 = *reinterpret_cast<const float4 *>(h + c * 8 + 4);
        return v;
    };
    // e = d sqrt(h) of a chunk from its loaded memory, into the row maximum
    // and the diagonal sum
    auto chunk = [&](const GramRaw &r, const SqH &v, float *e) {
        float d[8];
        gram_decode<EK, SK, WT, REF>(r, d, stab);
        const float qv[8] = {v.q0.x, v.q0.y, v.q0.z, v.q0.w, v.q1.x, v.q1.y, v.q1.z, v.q1.w};
        const float hv[8] = {v.h0.x, v.h0.y, v.h0.z, v.h0.w, v.h1.x, v.h1.y, v.h1.z, v.h1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            e[j] = d[j] * qv[j];
            mx = max(mx, __builtin_bit_cast(int, fabsf(e[j])));
            ds = __builtin_fma((double)d[j] * (double)d[j], (double)hv[j], ds);
        }
    };
    if (RC > 0) {
        // every chunk's weights, codes and scale first, then the chunks in
        // order, each one's sqrt(h) and h loaded while the one before is
        // decoded (chunk indices past the row are clamped to its last chunk
        // for the loads; their values go unused)
        GramRaw raw[RC > 0 ? RC : 1];
#pragma unroll
        for (int it = 0; it < RC; ++it)
            if (256 * it < nch)
                gram_load<EK, SK, WT, REF>(codes, scales, B, W, n * K + min<int64_t>(threadIdx.x + 256 * it, nch - 1) * 8,
                                           raw[it]);
        SqH nxt = load_sqh(min<int64_t>(threadIdx.x, nch - 1));
#pragma unroll
        for (int it = 0; it < RC; ++it) {
            const SqH cur = nxt;
            if (it + 1 < RC && 256 * (it + 1) < nch) nxt = load_sqh(min<int64_t>(threadIdx.x + 256 * (it + 1), nch - 1));
            if (threadIdx.x + 256 * it < nch) chunk(raw[it], cur, ek[it]);
        }
    } else {
        for (int64_t c = threadIdx.x; c < nch; c += 256) {
            GramRaw r;
            gram_load<EK, SK, WT, REF>(codes, scales, B, W, n * K + c * 8, r);
            chunk(r, load_sqh(c), ek[0]);
        }
    }
    mx = wave_max_int(mx);
    if ((threadIdx.x & 63) == 0) shm[threadIdx.x >> 6] = mx;
    ds = block_sum_256(ds, sh);  // synchronises, so shm is complete
    mx = max(max(shm[0], shm[1]), max(shm[2], shm[3]));
    int ex = 0;
    if (mx != 0) {
        int f;
        frexpf(__builtin_bit_cast(float, mx), &f);  // max = g 2^f, g in [0.5, 1)
        ex = f - 1 - 14;
    }
    if (threadIdx.x == 0) {
        erow[n] = ex;
        dsum[n] = ds;
    }
    uint16_t *orow = E + n * K;
    auto store = [&](int64_t c, const float *e) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const _Float16 lo = (_Float16)ldexpf(e[2 * j], -ex);
            const _Float16 hi = (_Float16)ldexpf(e[2 * j + 1], -ex);
            o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4 *>(orow + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    };
    if (RC > 0) {
#pragma unroll
        for (int it = 0; it < RC; ++it) {
            const int64_t c = threadIdx.x + 256 * it;
            if (c < nch) store(c, ek[it]);
        }
    } else {
        for (int64_t c = threadIdx.x; c < nch; c += 256) {
            float e[8];
            const int mx0 = mx;
            const double ds0 = ds;
            GramRaw r;
            gram_load<EK, SK, WT, REF>(codes, scales, B, W, n * K + c * 8, r);
            chunk(r, load_sqh(c), e);  // recomputes e (mx and ds are not used again)
            mx = mx0;
            ds = ds0;
            store(c, e);
        }
    }
}

template <int EK, int SK, typename WT, bool REF, int RC>
__global__ __launch_bounds__(256) void gram_operand_kernel(const uint8_t *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales, int B,
                                                           const WT *__restrict__ W, int64_t K,
                                                           const float *__restrict__ sq, const float *__restrict__ h,
                                                           uint16_t *__restrict__ E, int *__restrict__ erow,
                                                           double *__restrict__ dsum, int64_t nvalid)
{
    gram_operand_row<EK, SK, WT, REF, RC>(codes, scales, B, W, K, sq, h, E, erow, dsum, nvalid, blockIdx.x);
}

// Up to GRAM_OPS quantisations of one format in one launch: workgroup b does
// row n of quantisation q with, for b = 8 (n_q i + q) + x (x < 8),
// n = 8 i + x: consecutive workgroups go to the 8 XCDs in turn, so the n_q
// workgroups of one row of W run on one XCD, 8 dispatches apart, and share
// the row in its L2.  rpq (a multiple of 256) rows per quantisation;
// quantisation q's E, erow and dsum start at row q rpq.
constexpr int GRAM_OPS = 16;
struct GramOps {
    const uint8_t *codes[GRAM_OPS];
    const uint8_t *scales[GRAM_OPS];
    int B[GRAM_OPS];
    int n;
};
template <int EK, int SK, typename WT>
__global__ __launch_bounds__(256) void gram_operand_multi_kernel(const GramOps ob, const WT *__restrict__ W, int64_t K,
                                                                 const float *__restrict__ sq,
                                                                 const float *__restrict__ h, uint16_t *__restrict__ E,
                                                                 int *__restrict__ erow, double *__restrict__ dsum,
                                                                 int64_t nvalid, int64_t rpq)
{
    const unsigned rest = blockIdx.x / 8u;
    const int q = (int)(rest % (unsigned)ob.n);
    const int64_t n = (int64_t)(rest / (unsigned)ob.n) * 8 + (blockIdx.x & 7u), o = q * rpq;
    gram_operand_row<EK, SK, WT, false, 8>(ob.codes[q], ob.scales[q], ob.B[q], W, K, sq, h, E + o * K, erow + o,
                                           dsum + o, nvalid, n);
}

// This thread's share of v[0 .. n - 1] in a 256-thread workgroup (elements
// threadIdx.x + 256 i) as 8 running sums over i mod 8, added in a fixed order
// at the end: the 8 loads of a round are in flight together (indices past n
// are clamped for the load and contribute 0).
__device__ __forceinline__ double strided_sum8(const double *__restrict__ v, int64_t n)
{
    double a[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 2048) {
        double x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = v[min<int64_t>(i0 + 256 * u, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += i0 + 256 * u < n ? x[u] : 0.0;
    }
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// One workgroup per quantisation q: total = the slots part[(t mt + band) qg
// + x] of its E tiles t = q tpq .. q tpq + tpq - 1 (every band and gang) plus
// the diagonal sum b = dsum of its rows q rpq .. q rpq + nvalid - 1, in a
// fixed order.  ysq == NULL: ysq_out[q] = total.  Otherwise out[q] =
// sqrt(total) / sqrt(*ysq) and sums[3 q .. 3 q + 2] = {total, *ysq, b} (b /
// total says how much the float16 off-diagonal part cancels the exact
// diagonal one).
__global__ __launch_bounds__(256) void gram_final(const double *__restrict__ part, int tpq, int mt, int qg,
                                                  const double *__restrict__ dsum, int64_t rpq, int64_t nvalid,
                                                  const double *__restrict__ ysq, double *__restrict__ ysq_out,
                                                  double *__restrict__ out, double *__restrict__ sums)
{
    __shared__ double sh[4];
    const int q = blockIdx.x;
    const int64_t ns = (int64_t)tpq * mt * qg;
    const double *ps = part + (int64_t)q * ns;
    double a = strided_sum8(ps, ns), b = strided_sum8(dsum + q * rpq, nvalid);
    a = block_sum_256(a, sh);
    b = block_sum_256(b, sh);
    if (threadIdx.x == 0) {
        const double t = a + b;
        if (ysq == nullptr) {
            ysq_out[q] = t;
        } else {
            const double y = *ysq;
            out[q] = sqrt(t) / sqrt(y);
            if (sums) {
                sums[3 * q] = t;
                sums[3 * q + 1] = y;
                sums[3 * q + 2] = b;
            }
        }
    }
}

__global__ __launch_bounds__(256) void gram_zero_f64(double *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0;
}

GramLayout output_gram_layout(int64_t K)
{
    GramLayout L;
    L.h = 0;
    L.sq = al256(K * 4);
    L.r = L.sq + al256(K * 4);
    L.c = L.r + al256(K * 4);
    L.bytes = L.c + al256(K * K * 2);
    return L;
}

size_t output_gram_ws(int64_t M, int64_t K) { return (size_t)std::max<int64_t>(256, (int64_t)hdiag_ws(M, K)); }

// Schedule of the C E^T walk (the QUAD mode's gangs) over nt E tiles: with
// P = CUs / 8 workgroups per XCD, the E tiles per group qe (and qa = min(4,
// P / qe) bands per panel) that keep the largest share of the XCD busy on
// real tiles, 8 gangs of P slots, when that share is at least 90%;
// otherwise gangs of all nt tiles with one band per panel, CUs / nt of them.
// The schedule setting HD_SCHED_GRAM_GANGS = g > 0 forces the second form
// with g gangs; HD_SCHED_GRAM_BANDS = a > 0 the first with qa = a and qe =
// max(1, P / a) (at most nt).
struct GramPlan {
    int qa, qe, qg, qper;
    int64_t qcpg, qcols, wgs;
};
static GramPlan gram_plan(int64_t nt, int64_t K)
{
    const int64_t mt = (K + GE_TM - 1) / GE_TM, cus = device_cus(), per = cus / 8;
    const int64_t forced = std::min<int64_t>(schedule_setting(HD_SCHED_GRAM_GANGS), cus);
    GramPlan g;
    double best = 0.0;
    int64_t bqe = 0, bqa = 0;
    for (int64_t qe = 1; qe <= per; ++qe) {
        const int64_t qa = std::min<int64_t>(4, per / qe), ngr = (nt + qe - 1) / qe;
        const double eff = (double)nt / (double)(ngr * qe) * (double)(qa * qe) / (double)per;
        if (eff > best + 1e-9) {
            best = eff;
            bqe = qe;
            bqa = qa;
        }
    }
    const int64_t bands = std::min<int64_t>(schedule_setting(HD_SCHED_GRAM_BANDS), std::max<int64_t>(mt, 1));
    if (forced <= 0 && bands > 0) {
        best = 1.0;
        bqa = bands;
        bqe = std::min<int64_t>(std::max<int64_t>(1, per / bands), std::max<int64_t>(nt, 1));
    }
    if (forced <= 0 && best >= 0.9) {
        g.qa = (int)bqa;
        g.qe = (int)bqe;
        g.qg = 8;
        g.qper = (int)per;
    } else {
        g.qa = 1;
        g.qe = (int)nt;
        g.qg = (int)std::max<int64_t>(1, forced > 0 ? forced : cus / std::max<int64_t>(nt, 1));
        g.qper = (int)nt;
    }
    g.qcpg = 0;
    for (int64_t i = 0; i * g.qa < mt; ++i) g.qcpg += mt - g.qa * i;
    g.qcols = g.qcpg * ((nt + g.qe - 1) / g.qe);
    g.qg = (int)std::min<int64_t>(g.qg, g.qcols);
    g.wgs = (int64_t)g.qg * g.qper;
    return g;
}

// Rows of E per quantisation (N padded to whole 256-row tiles).
static int64_t gram_rows(int64_t N) { return (N + GE_TN - 1) / GE_TN * GE_TN; }

size_t output_error_gram_ws(int64_t count, int64_t N, int64_t K)
{
    const int64_t R = count * gram_rows(N), nt = R / GE_TN, mt = (K + GE_TM - 1) / GE_TM;
    const int64_t slots = nt * mt * std::max<int64_t>(device_cus(), 8);
    return (size_t)(al256(R * K * 2) + al256(R * 4) + al256(R * 8) + al256(slots * 8));
}

hipError_t launch_output_gram(const void *X, int64_t M, int64_t K, const float *h, void *gram, void *ws,
                              hipStream_t st)
{
    const GramLayout L = output_gram_layout(K);
    char *g = static_cast<char *>(gram);
    float *gh = reinterpret_cast<float *>(g + L.h);
    float *sq = reinterpret_cast<float *>(g + L.sq);
    float *r = reinterpret_cast<float *>(g + L.r);
    uint16_t *C = reinterpret_cast<uint16_t *>(g + L.c);
    if (K == 0) return hipSuccess;
    hipError_t e;
    if (h == nullptr) {
        e = launch_hdiag(X, HD_BF16, M, K, gh, ws, st);
        if (e != hipSuccess) return e;
        h = gh;
    }
    gram_prep_kernel<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(h, K, gh, sq, r);
    if (M == 0) {
        gram_zero_kernel<<<1024, 256, 0, st>>>(C, K * K);
        return hipGetLastError();
    }
    // X^T X straight from row-major X (the GRAM mode's transposed LDS reads)
    const uint16_t *Xb = static_cast<const uint16_t *>(X);
    GeArgs ga = ge_args(Xb, Xb, K, K, M);
    const int64_t items = (int64_t)ga.mt * (ga.mt + 1) / 2;
    ga.nlin = (int)items;
    ga.r = r;
    ga.C = C;
    return ge_launch<false, GE_GRAM, 8 / HD_GE_WN>(ga, items, st);
}

// H = X^T X in float32 [K][K] for bf16 X [M][K] (K % 8 == 0, M > 0): the
// lower tile triangle of the transposed-read product, each element written
// with its mirror.
hipError_t launch_gram_store(const void *X, int64_t M, int64_t K, float *H, hipStream_t st)
{
    const uint16_t *Xb = static_cast<const uint16_t *>(X);
    GeArgs ga = ge_args(Xb, Xb, K, K, M);
    const int64_t items = (int64_t)ga.mt * (ga.mt + 1) / 2;
    ga.nlin = (int)items;
    ga.Y = H;
    return ge_launch<false, GE_SYRK, 8 / HD_GE_WN>(ga, items, st);
}

template <int EK, int SK, bool REF>
static void launch_gram_operand(const uint8_t *codes, const uint8_t *scales, int B, const void *W, int wdt, int64_t N,
                                int64_t rows, int64_t K, const float *sq, const float *h, uint16_t *E, int *erow,
                                double *dsum, hipStream_t st)
{
    const bool regs = K <= 2048 * 8;
    if (wdt == HD_BF16) {
        if (regs)
            gram_operand_kernel<EK, SK, uint16_t, REF, 8><<<(unsigned)rows, 256, 0, st>>>(
                codes, scales, B, static_cast<const uint16_t *>(W), K, sq, h, E, erow, dsum, N);
        else
            gram_operand_kernel<EK, SK, uint16_t, REF, 0><<<(unsigned)rows, 256, 0, st>>>(
                codes, scales, B, static_cast<const uint16_t *>(W), K, sq, h, E, erow, dsum, N);
    } else {
        if (regs)
            gram_operand_kernel<EK, SK, float, REF, 8><<<(unsigned)rows, 256, 0, st>>>(
                codes, scales, B, static_cast<const float *>(W), K, sq, h, E, erow, dsum, N);
        else
            gram_operand_kernel<EK, SK, float, REF, 0><<<(unsigned)rows, 256, 0, st>>>(
                codes, scales, B, static_cast<const float *>(W), K, sq, h, E, erow, dsum, N);
    }
}

template <int F>
static void gram_operand_fmt(const uint8_t *codes, const uint8_t *scales, int B, const void *W, int wdt, int64_t N,
                             int64_t rows, int64_t K, const float *sq, const float *h, uint16_t *E, int *erow,
                             double *dsum, hipStream_t st)
{
    launch_gram_operand<elem_kind(F), scale_kind(F), false>(codes, scales, B, W, wdt, N, rows, K, sq, h, E, erow,
                                                            dsum, st);
}

template <int F>
static void gram_operand_multi_fmt(const GramOps &ob, const void *W, int wdt, int64_t N, int64_t rows, int64_t K,
                                   const float *sq, const float *h, uint16_t *E, int *erow, double *dsum,
                                   hipStream_t st)
{
    if (wdt == HD_BF16)
        gram_operand_multi_kernel<elem_kind(F), scale_kind(F), uint16_t><<<(unsigned)(rows * ob.n), 256, 0, st>>>(
            ob, static_cast<const uint16_t *>(W), K, sq, h, E, erow, dsum, N, rows);
    else
        gram_operand_multi_kernel<elem_kind(F), scale_kind(F), float><<<(unsigned)(rows * ob.n), 256, 0, st>>>(
            ob, static_cast<const float *>(W), K, sq, h, E, erow, dsum, N, rows);
}

// Partial slots of one walk over `count` quantisations of N x K weights.
static int64_t gram_walk_slots(int count, int64_t N, int64_t K)
{
    const int64_t nt = count * gram_rows(N) / GE_TN, mt = (K + GE_TM - 1) / GE_TM;
    return N > 0 && K > 0 ? nt * mt * gram_plan(nt, K).qg : 0;
}

// One walk over `count` quantisations (fmt[q], B[q], codes[q], scales[q]) of
// one W: out[q] = sqrt(||X (Wq_q - W)^T||^2) / sqrt(*ysq); fmt == NULL: the
// reference ||X W^T||^2 into ysq_out[0] (count 1).  E, erow and dsum are the
// walk's rows, part its gram_walk_slots() slots, zeroed beforehand.
static hipError_t gram_walk(int count, const int *fmt, const int *B, const uint8_t *const *codes,
                            const uint8_t *const *scales, const void *W, int wdt, int64_t N, int64_t K,
                            const void *gram, const double *ysq, double *ysq_out, double *out, double *sums,
                            uint16_t *E, int *erow, double *dsum, double *part, hipStream_t st)
{
    const GramLayout L = output_gram_layout(K);
    const char *g = static_cast<const char *>(gram);
    const float *gh = reinterpret_cast<const float *>(g + L.h);
    const float *sq = reinterpret_cast<const float *>(g + L.sq);
    const uint16_t *C = reinterpret_cast<const uint16_t *>(g + L.c);
    const int64_t rpq = gram_rows(N), R = count * rpq, nt = R / GE_TN, mt = (K + GE_TM - 1) / GE_TM;
    const bool work = N > 0 && K > 0;
    const GramPlan plan = gram_plan(nt, K);
    bool fused = false;
    if (work && fmt != nullptr && K <= 2048 * 8 && rpq * GRAM_OPS < ((int64_t)1 << 31)) {
        fused = true;
        for (int q = 1; q < count; ++q) fused = fused && fmt[q] == fmt[0];
    }
    if (work && fused) {
        for (int q0 = 0; q0 < count; q0 += GRAM_OPS) {
            GramOps ob = {};
            ob.n = std::min(GRAM_OPS, count - q0);
            for (int k = 0; k < ob.n; ++k) {
                ob.codes[k] = codes[q0 + k];
                ob.scales[k] = scales[q0 + k];
                ob.B[k] = B[q0 + k];
            }
            uint16_t *Eq = E + q0 * rpq * K;
            int *eq = erow + q0 * rpq;
            double *dq = dsum + q0 * rpq;
            switch (fmt[0]) {
            case HD_INT8_E4M3: gram_operand_multi_fmt<HD_INT8_E4M3>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4: gram_operand_multi_fmt<HD_NVFP4>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_MXFP4: gram_operand_multi_fmt<HD_MXFP4>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_MXFP8: gram_operand_multi_fmt<HD_MXFP8>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_FP8_E4M3S: gram_operand_multi_fmt<HD_FP8_E4M3S>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4_UE4M4: gram_operand_multi_fmt<HD_NVFP4_UE4M4>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4_UE5M3: gram_operand_multi_fmt<HD_NVFP4_UE5M3>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVINT4: gram_operand_multi_fmt<HD_NVINT4>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_FP4_F16: gram_operand_multi_fmt<HD_FP4_F16>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_INT4_F16: gram_operand_multi_fmt<HD_INT4_F16>(ob, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            default: return hipErrorInvalidValue;
            }
        }
    }
    if (work) {
        for (int q = 0; q < count && !fused; ++q) {
            uint16_t *Eq = E + q * rpq * K;
            int *eq = erow + q * rpq;
            double *dq = dsum + q * rpq;
            const uint8_t *cq = codes ? codes[q] : nullptr;
            const uint8_t *sq8 = scales ? scales[q] : nullptr;
            switch (fmt ? fmt[q] : -1) {
            case -1: launch_gram_operand<ELEM_INT8, SCALE_INT8, true>(cq, sq8, 8, W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_INT8_E4M3: gram_operand_fmt<HD_INT8_E4M3>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4: gram_operand_fmt<HD_NVFP4>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_MXFP4: gram_operand_fmt<HD_MXFP4>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_MXFP8: gram_operand_fmt<HD_MXFP8>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_FP8_E4M3S: gram_operand_fmt<HD_FP8_E4M3S>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4_UE4M4: gram_operand_fmt<HD_NVFP4_UE4M4>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVFP4_UE5M3: gram_operand_fmt<HD_NVFP4_UE5M3>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_NVINT4: gram_operand_fmt<HD_NVINT4>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_FP4_F16: gram_operand_fmt<HD_FP4_F16>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            case HD_INT4_F16: gram_operand_fmt<HD_INT4_F16>(cq, sq8, B[q], W, wdt, N, rpq, K, sq, gh, Eq, eq, dq, st); break;
            default: return hipErrorInvalidValue;
            }
        }
        GeArgs ga = ge_args(C, E, K, R, K);
        ga.nlin = (int)plan.wgs;
        ga.qa = plan.qa;
        ga.qe = plan.qe;
        ga.qg = plan.qg;
        ga.qper = plan.qper;
        ga.qcpg = plan.qcpg;
        ga.qcols = plan.qcols;
        ga.erow = erow;
        ga.part = part;
        const hipError_t e = ge_launch<true, GE_QUAD, 8 / HD_GE_WN>(ga, plan.wgs, st);
        if (e != hipSuccess) return e;
    }
    gram_final<<<(unsigned)count, 256, 0, st>>>(part, work ? (int)(rpq / GE_TN) : 0, (int)mt, plan.qg, dsum, rpq,
                                                work ? N : 0, fmt ? ysq : nullptr, ysq_out, out, sums);
    return hipGetLastError();
}

// Quantisations per walk: the walk re-reads the stacked operand E once per
// panel of C's bands and C once per group of E tiles, from the Infinity Cache
// when C's upper block triangle and the walk's E fit in it together
// (GRAM_CACHE_BYTES); a batch whose whole E does not fit is cut into walks of
// as many quantisations as do (at least one).  When C alone does not fit
// there is nothing to gain and the batch stays one walk.
static constexpr int64_t GRAM_CACHE_BYTES = (int64_t)224 << 20;
static int gram_sub_batch(int count, int64_t N, int64_t K)
{
    const int64_t mt = (K + GE_TM - 1) / GE_TM;
    const int64_t cbytes = mt * (mt + 1) / 2 * (int64_t)GE_TM * GE_TM * 2;
    const int64_t ebytes = gram_rows(N) * K * 2;
    if (cbytes + ebytes > GRAM_CACHE_BYTES || ebytes == 0) return count;
    return (int)std::max<int64_t>(1, std::min<int64_t>(count, (GRAM_CACHE_BYTES - cbytes) / ebytes));
}

// count quantisations of one W, in walks of gram_sub_batch quantisations
// that take consecutive slices of the workspace (E rows, row exponents,
// diagonal sums, partial slots); fmt == NULL: the reference (count 1).
hipError_t launch_output_error_gram(int count, const int *fmt, const int *B, const uint8_t *const *codes,
                                    const uint8_t *const *scales, const void *W, int wdt, int64_t N, int64_t K,
                                    const void *gram, const double *ysq, double *ysq_out, double *out, double *sums,
                                    void *ws, hipStream_t st)
{
    const int64_t rpq = gram_rows(N), R = count * rpq;
    char *w = static_cast<char *>(ws);
    uint16_t *E = reinterpret_cast<uint16_t *>(w);
    int *erow = reinterpret_cast<int *>(w + al256(R * K * 2));
    double *dsum = reinterpret_cast<double *>(w + al256(R * K * 2) + al256(R * 4));
    double *part = reinterpret_cast<double *>(w + al256(R * K * 2) + al256(R * 4) + al256(R * 8));
    const int sb = fmt == nullptr ? 1 : gram_sub_batch(count, N, K);
    // the walks' slots packed one after another, all zeroed by one launch
    const int last = count - (count - 1) / sb * sb;  // quantisations of the last walk
    const int64_t full_slots = gram_walk_slots(sb, N, K), slots = (int64_t)((count - 1) / sb) * full_slots +
                                                               gram_walk_slots(last, N, K);
    if (slots > 0)
        gram_zero_f64<<<(unsigned)std::min<int64_t>((slots + 255) / 256, 1024), 256, 0, st>>>(part, slots);
    for (int q0 = 0; q0 < count; q0 += sb) {
        const int n = std::min(sb, count - q0);
        const hipError_t e = gram_walk(n, fmt ? fmt + q0 : nullptr, B ? B + q0 : nullptr,
                                       codes ? codes + q0 : nullptr, scales ? scales + q0 : nullptr, W, wdt, N, K,
                                       gram, ysq, ysq_out, out ? out + q0 : nullptr, sums ? sums + 3 * q0 : nullptr,
                                       E + q0 * rpq * K, erow + q0 * rpq, dsum + q0 * rpq,
                                       part + (int64_t)(q0 / sb) * full_slots, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hd
