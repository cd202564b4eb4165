// search_e4m3_elems.hip - the scale-search kernels of the formats with E4M3 elements (MXFP8, FP8_E4M3S)
// (search_impl.hpp), one translation unit per element family so the build
// compiles them in parallel.
#include "hdiag.h"
#include "search_impl.hpp"

namespace hd {

hipError_t launch_search_e4m3_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                    uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals, hipStream_t st)
{
    switch (fmt) {
    case HD_MXFP8: return search_fmt<ELEM_E4M3, SCALE_E8M0>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_FP8_E4M3S: return search_fmt<ELEM_E4M3, SCALE_E4M3>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hd
