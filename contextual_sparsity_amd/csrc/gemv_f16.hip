// Row-gather GEMV instantiations: __half weights, no side blocks.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, false>(a, s);
}

}  // namespace djv
