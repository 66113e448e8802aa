// Row-gather GEMV instantiations: __half weights, with side-block selections.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16_side(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, true>(a, s);
}

}  // namespace djv
