// Dispatch of the row-gather GEMV to its instantiations (weight dtype x with or without
// side selections, each compiled in its own translation unit).
#include "common.hpp"

namespace djv {

hipError_t launch_gemv_f32(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_side(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_side(const GemvArgs& a, hipStream_t s);

hipError_t launch_gemv(bool f16, const GemvArgs& a, hipStream_t s) {
    if (a.nseg < 1 || a.nseg > kMaxSeg || a.nside < 0 || a.nside > kMaxSide) return hipErrorInvalidValue;
    for (int i = 0; i < a.nseg; ++i)
        if (a.seg[i].epi < kEpiStore || a.seg[i].epi > kEpiQkv) return hipErrorInvalidValue;
    if (f16) return a.nside > 0 ? launch_gemv_f16_side(a, s) : launch_gemv_f16(a, s);
    return a.nside > 0 ? launch_gemv_f32_side(a, s) : launch_gemv_f32(a, s);
}

}  // namespace djv
