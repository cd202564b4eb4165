// common.hpp - small device helpers shared by the kernels of libhdiag.so.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace hd {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16, round to nearest even (finite and infinite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as float.
template <typename T>
__device__ __forceinline__ void load8(const T *p, float *v);

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t *p, float *v)
{
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float *p, float *v)
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// load8 with the non-temporal hint: for data streamed once (the copy of it
// need not stay in L2 / MALL); measured ~10% more read bandwidth on gfx950.
typedef uint32_t hd_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void *p)
{
    const hd_u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const hd_u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

template <typename T>
__device__ __forceinline__ void load8_nt(const T *p, float *v);

template <>
__device__ __forceinline__ void load8_nt<bf16_t>(const bf16_t *p, float *v)
{
    const uint4 q = load16_nt(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8_nt<float>(const float *p, float *v)
{
    const uint4 a = load16_nt(p), b = load16_nt(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// Sum over the `width` consecutive lanes of an aligned lane group (butterfly:
// every lane of the group ends with the same value, added in the same order).
template <int WIDTH>
__device__ __forceinline__ double group_sum(double v)
{
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_max_int(int v)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

// Deterministic sum of one double per thread over a 256-thread workgroup.
__device__ __forceinline__ double block_sum_256(double v, double *sh /* [4] */)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

}  // namespace hd
