// Row-gather GEMV instantiations: float weights, 1024-thread blocks whose first blocks run
// selections of long rows.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32_side(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, 2>(a, s);
}

}  // namespace djv
