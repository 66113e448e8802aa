// Row-gather GEMV instantiations: float weights, no side blocks.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<float, false>(a, s);
}

}  // namespace djv
