// Row-gather GEMV instantiations with the dynamic segment split (segments that read the
// same input, with device counts): float weights, plain (256-thread blocks) and with
// long-row selections in the first blocks (1024-thread blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32_dyn(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 0, true>(a, s);
}

hipError_t launch_gemv_f32_side_dyn(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 2, true>(a, s);
}

}  // namespace djv
