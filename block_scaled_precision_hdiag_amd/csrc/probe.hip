// probe.hip - streaming kernels with the memory access patterns of the
// HBM-bound stages and next to no arithmetic: what a kernel with those loads
// and stores reaches at best, beside which the stages' own rates are read.
//
// Every kind walks n 16-bit elements (n % 8192 == 0) in the encode's layout:
// a wave owns 2048 consecutive elements, lane l of it the 8-element chunks
// 512 k + 8 l (k = 0..3), loaded as 16 bytes each with the non-temporal hint.
//   READ    (0): in0 = n bf16; out0[w] = XOR of the 32-bit words of
//                workgroup w's 8192 elements (one store per workgroup).
//   ENCODE  (1): in0 = n bf16; out0 = n / 2 bytes, one 32-bit word per chunk
//                (the XOR of its four words), out1 = n / 16 bytes, one per
//                pair of chunks (the low byte of the first one's word): the
//                NVFP4 B = 16 byte mix, gathered in LDS and written with 16-byte
//                (codes) and 4-byte (scale) stores like the encode.
//   WRITE   (2): out0 = n bf16, 32-bit word i = i.
//   DEQUANT (3): in0 = n / 2 bytes (a 32-bit word c per chunk), in1 = n / 16
//                bytes (a byte s per pair of chunks); out0 = n bf16, the chunk's
//                four words {c ^ s, c + s, 3 c, c >> 3}: the dequantize-to-
//                bfloat16 byte mix.
#include "common.hpp"
#include "hdiag.h"
#include "kernels.hpp"

namespace hd {

static constexpr int PR_SUB = 4;  // chunks per lane

__global__ __launch_bounds__(256) void probe_read(const uint16_t *__restrict__ in, uint32_t *__restrict__ out)
{
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wbase = ((int64_t)blockIdx.x * 4 + wv) * (64 * 8 * PR_SUB);
    uint4 v[PR_SUB];
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) v[k] = load16_nt(in + wbase + 512 * k + 8 * lane);
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if (lane == 0) red[wv] = x;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void probe_encode(const uint16_t *__restrict__ in, uint8_t *__restrict__ codes,
                                                    uint8_t *__restrict__ sc)
{
    __shared__ uint32_t lc[4][64 * PR_SUB];
    __shared__ uint32_t ls[4][8 * PR_SUB];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wbase = ((int64_t)blockIdx.x * 4 + wv) * (64 * 8 * PR_SUB);
    uint4 v[PR_SUB];
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) v[k] = load16_nt(in + wbase + 512 * k + 8 * lane);
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) {
        const uint32_t x = v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
        lc[wv][64 * k + lane] = x;
        if ((lane & 1) == 0) reinterpret_cast<uint8_t *>(ls[wv])[32 * k + lane / 2] = (uint8_t)x;
    }
    __syncthreads();
    const hd_u32x4 *src = reinterpret_cast<const hd_u32x4 *>(lc[wv]);
    hd_u32x4 *dst = reinterpret_cast<hd_u32x4 *>(codes + wbase / 2);
#pragma unroll
    for (int i = lane; i < 16 * PR_SUB; i += 64) __builtin_nontemporal_store(src[i], dst + i);
    if (lane < 8 * PR_SUB) reinterpret_cast<uint32_t *>(sc + wbase / 16)[lane] = ls[wv][lane];
}

__global__ __launch_bounds__(256) void probe_write(uint16_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wbase = ((int64_t)blockIdx.x * 4 + wv) * (64 * 8 * PR_SUB);
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        const uint32_t i = (uint32_t)(e / 2);
        __builtin_nontemporal_store(hd_u32x4{i, i + 1, i + 2, i + 3}, reinterpret_cast<hd_u32x4 *>(out + e));
    }
}

__global__ __launch_bounds__(256) void probe_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ sc,
                                                     uint16_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wbase = ((int64_t)blockIdx.x * 4 + wv) * (64 * 8 * PR_SUB);
    uint32_t c[PR_SUB], s[PR_SUB];
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        c[k] = *reinterpret_cast<const uint32_t *>(codes + e / 2);
        s[k] = sc[e / 16];
    }
#pragma unroll
    for (int k = 0; k < PR_SUB; ++k) {
        const int64_t e = wbase + 512 * k + 8 * lane;
        *reinterpret_cast<uint4 *>(out + e) = make_uint4(c[k] ^ s[k], c[k] + s[k], 3u * c[k], c[k] >> 3);
    }
}

hipError_t launch_stream_probe(int kind, int64_t n, const void *in0, const void *in1, void *out0, void *out1,
                               hipStream_t st)
{
    const unsigned grid = (unsigned)(n / (256 * 8 * PR_SUB));
    if (grid == 0) return hipSuccess;
    switch (kind) {
    case HD_PROBE_READ:
        probe_read<<<grid, 256, 0, st>>>(static_cast<const uint16_t *>(in0), static_cast<uint32_t *>(out0));
        break;
    case HD_PROBE_ENCODE:
        probe_encode<<<grid, 256, 0, st>>>(static_cast<const uint16_t *>(in0), static_cast<uint8_t *>(out0),
                                           static_cast<uint8_t *>(out1));
        break;
    case HD_PROBE_WRITE: probe_write<<<grid, 256, 0, st>>>(static_cast<uint16_t *>(out0)); break;
    case HD_PROBE_DEQUANT:
        probe_dequant<<<grid, 256, 0, st>>>(static_cast<const uint8_t *>(in0), static_cast<const uint8_t *>(in1),
                                            static_cast<uint16_t *>(out0));
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hd
