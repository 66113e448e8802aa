// Row-gather GEMV instantiations: float weights, 256-thread blocks (GEMV only, or with
// attention chunks and short-row selections in the first blocks).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_f32(const GemvArgs& a, hipStream_t s) {
    return (a.nattn > 0 || a.nside > 0) ? gemv_detail::dispatch<float, 1>(a, s)
                                         : gemv_detail::dispatch<float, 0>(a, s);
}

}  // namespace djv
