// Row-gather GEMV instantiations with the dynamic segment split reading LN(x) of an x
// accumulated in place (moments summed by the kernel): __half weights, plain (256-thread
// blocks) and with long-row selections in the first blocks (1024-thread blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16_dyn_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 0, true, true>(a, s);
}

hipError_t launch_gemv_f16_side_dyn_own(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 2, true, true>(a, s);
}

}  // namespace djv
