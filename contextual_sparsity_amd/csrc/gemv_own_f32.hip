// Row-gather GEMV instantiations reading LN(x) of an x accumulated in place (moments summed
// by the kernel): float weights, 256-thread blocks and 1024-thread blocks with long-row
// selections in the first blocks.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32_own(const GemvArgs& a, hipStream_t s) {
    return (a.nattn > 0 || a.nside > 0) ? gemv_detail::dispatch<float, 1, false, true>(a, s)
                                         : gemv_detail::dispatch<float, 0, false, true>(a, s);
}

hipError_t launch_gemv_f32_side_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 2, false, true>(a, s);
}

}  // namespace djv
