// search_int_elems.hip - the scale-search kernels of the formats with integer elements (INT8, INT4)
// (search_impl.hpp), one translation unit per element family so the build
// compiles them in parallel.
#include "hdiag.h"
#include "search_impl.hpp"

namespace hd {

hipError_t launch_search_int_elems(int fmt, int B, const void *W, int wdt, int64_t N, int64_t K, const float *h,
                                   uint8_t *codes, uint8_t *scales, float *block_obj, unsigned long long *evals, hipStream_t st)
{
    switch (fmt) {
    case HD_INT8_E4M3: return search_fmt<ELEM_INT8, SCALE_INT8>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    case HD_NVINT4: return search_fmt<ELEM_INT4, SCALE_E4M3>(B, W, wdt, N, K, h, codes, scales, block_obj, evals, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hd
