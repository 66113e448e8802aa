// Row-gather GEMV instantiations reading LN(x) of an x accumulated in place (moments summed
// by the kernel): __half weights, 256-thread blocks and 1024-thread blocks with long-row
// selections in the first blocks.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16_own(const GemvArgs& a, hipStream_t s) {
    return (a.nattn > 0 || a.nside > 0) ? gemv_detail::dispatch<__half, 1, false, true>(a, s)
                                         : gemv_detail::dispatch<__half, 0, false, true>(a, s);
}

hipError_t launch_gemv_f16_side_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 2, false, true>(a, s);
}

}  // namespace djv
