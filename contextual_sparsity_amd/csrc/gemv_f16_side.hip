// Row-gather GEMV instantiations: __half weights, 1024-thread blocks whose first blocks run
// selections of long rows.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16_side(const GemvArgs& a, hipStream_t s) {
    return gemv_detail::dispatch<__half, 2>(a, s);
}

}  // namespace djv
