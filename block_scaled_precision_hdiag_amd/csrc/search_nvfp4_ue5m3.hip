// search_nvfp4_ue5m3.hip - scale-search kernels for one format (one translation unit
// per format keeps the build parallel).
#include "search_impl.hpp"

namespace hd {

hipError_t launch_search_nvfp4_ue5m3(int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                           uint8_t *codes, uint8_t *scales, float *block_obj, hipStream_t st)
{
    return search_fmt<ELEM_E2M1, SCALE_UE5M3>(B, W, wdt, N, K, h, codes, scales, block_obj, st);
}

}  // namespace hd
