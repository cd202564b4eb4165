// tscale.hip - per-tensor scaling over E4M3 block scales ("Is Finer Better?"
// §5.1 and Table 1, UE4M3-S).  The tensor scale s_T = amax_T / (C 448) (C the
// element maximum, 1 for INT8 whose block scale is amax itself; 1 for an
// all-zero tensor) maps the largest block scale onto the top of the E4M3
// grid; the blocks then quantise W' = fl32(W / s_T) as the format does, and
// dequantize multiplies by s_T once more.
//
// Kernels: a grid-stride max |w| (16-byte loads, per-workgroup LDS reduction,
// one atomic max on the float's bits: non-negative floats order like their
// bit patterns), the scale, and an elementwise pass writing W' in float32.
#include <algorithm>

#include "encode.hpp"
#include "kernels.hpp"

namespace hd {

__global__ __launch_bounds__(256) void tscale_init_kernel(uint32_t *__restrict__ amax_bits)
{
    if (threadIdx.x == 0) amax_bits[0] = 0u;
}

template <typename T>
__global__ __launch_bounds__(256) void tscale_amax_kernel(const T *__restrict__ W, int64_t total,
                                                          uint32_t *__restrict__ amax_bits)
{
    __shared__ float red[256];
    float m = 0.0f;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; e < total; e += (int64_t)gridDim.x * 256 * 8) {
        float w[8];
        load8<T>(W + e, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(w[j]));
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(red[0]));
}

// s_T = fl32(amax / ct448), or 1 when amax = 0 (ct448 = C * 448, exact).
__global__ __launch_bounds__(256) void tscale_final_kernel(const uint32_t *__restrict__ amax_bits, float ct448,
                                                           float *__restrict__ tscale)
{
    if (threadIdx.x == 0) {
        const float amax = __uint_as_float(amax_bits[0]);
        tscale[0] = amax == 0.0f ? 1.0f : amax / ct448;  // IEEE division
    }
}

// Wp = fl32(W / s_T), sign kept (IEEE division).
template <typename T>
__global__ __launch_bounds__(256) void tscale_apply_kernel(const T *__restrict__ W, int64_t total,
                                                           const float *__restrict__ tscale, float *__restrict__ Wp)
{
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= total) return;
    const float t = tscale[0];
    float w[8];
    load8<T>(W + e, w);
    float4 *p = reinterpret_cast<float4 *>(Wp + e);
    p[0] = make_float4(w[0] / t, w[1] / t, w[2] / t, w[3] / t);
    p[1] = make_float4(w[4] / t, w[5] / t, w[6] / t, w[7] / t);
}

hipError_t launch_tensor_scale(int fmt, const void *W, int wdt, int64_t N, int64_t K, float *tscale, float *Wp,
                               void *ws, hipStream_t st)
{
    const int64_t total = N * K;  // a multiple of 8 (K % B == 0, B >= 8)
    uint32_t *amax_bits = static_cast<uint32_t *>(ws);
    const float ct = scale_kind(fmt) == SCALE_INT8 ? 1.0f : elem_max(elem_kind(fmt));
    const unsigned g = (unsigned)std::min<int64_t>((total / 8 + 255) / 256, 4096);
    tscale_init_kernel<<<1, 64, 0, st>>>(amax_bits);
    if (wdt == HD_BF16)
        tscale_amax_kernel<bf16_t><<<g, 256, 0, st>>>(static_cast<const bf16_t *>(W), total, amax_bits);
    else
        tscale_amax_kernel<float><<<g, 256, 0, st>>>(static_cast<const float *>(W), total, amax_bits);
    tscale_final_kernel<<<1, 64, 0, st>>>(amax_bits, ct * 448.0f, tscale);
    const unsigned ga = (unsigned)((total / 8 + 255) / 256);
    if (wdt == HD_BF16)
        tscale_apply_kernel<bf16_t><<<ga, 256, 0, st>>>(static_cast<const bf16_t *>(W), total, tscale, Wp);
    else
        tscale_apply_kernel<float><<<ga, 256, 0, st>>>(static_cast<const float *>(W), total, tscale, Wp);
    return hipGetLastError();
}

}  // namespace hd
