// Row-gather GEMV instantiations with the dynamic segment split reading LN(x) of an x
// accumulated in place (moments summed by the kernel): float weights, plain (256-thread
// blocks) and with long-row selections in the first blocks (1024-thread blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32_dyn_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 0, true, true>(a, s);
}

hipError_t launch_gemv_f32_side_dyn_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 2, true, true>(a, s);
}

}  // namespace djv
