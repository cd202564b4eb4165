// search_e2m1_elems.hip - the scale-search kernels of the formats with E2M1 elements (NVFP4 on the E4M3, UE4M4 and UE5M3 grids, MXFP4)
// (search_impl.hpp), one translation unit per element family so the build
// compiles them in parallel.
#include "hdiag.h"
#include "search_impl.hpp"

namespace hd {

hipError_t launch_search_e2m1_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                    uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals, hipStream_t st)
{
    switch (fmt) {
    case HD_NVFP4: return search_fmt<ELEM_E2M1, SCALE_E4M3>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_MXFP4: return search_fmt<ELEM_E2M1, SCALE_E8M0>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_NVFP4_UE4M4: return search_fmt<ELEM_E2M1, SCALE_UE4M4>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_NVFP4_UE5M3: return search_fmt<ELEM_E2M1, SCALE_UE5M3>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hd
