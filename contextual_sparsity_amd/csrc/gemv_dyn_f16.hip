// Row-gather GEMV instantiations with the dynamic segment split (segments that read the
// same input, with device counts): __half weights, plain (256-thread blocks) and with
// long-row selections in the first blocks (1024-thread blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16_dyn(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 0, true>(a, s);
}

hipError_t launch_gemv_f16_side_dyn(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 2, true>(a, s);
}

}  // namespace djv
