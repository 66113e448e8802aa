// Row-gather GEMV instantiations: __half weights, 256-thread blocks (GEMV only, or with
// attention chunks and short-row selections in the first blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f16(const GemvArgs& a, hipStream_t s) {
    return (a.nattn > 0 || a.nside > 0) ? gemv_detail::dispatch<__half, 1>(a, s)
                                         : gemv_detail::dispatch<__half, 0>(a, s);
}

}  // namespace djv
