// Row-gather GEMV instantiations: float weights, with side-block selections.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32_side(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, true>(a, s);
}

}  // namespace djv
