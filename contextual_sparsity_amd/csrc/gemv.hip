// Dispatch of the row-gather GEMV to its per-epilogue instantiations (each epilogue
// is compiled in its own translation unit and is a distinct kernel symbol).
#include "common.hpp"

namespace djv {

hipError_t launch_gemv_store(bool f16, const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_relu(bool f16, const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_bias_relu(bool f16, const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_qkv(bool f16, const GemvArgs& a, hipStream_t s);

hipError_t launch_gemv(bool f16, const GemvArgs& a, hipStream_t s) {
    switch (a.epi) {
    case kEpiStore: return launch_gemv_store(f16, a, s);
    case kEpiRelu: return launch_gemv_relu(f16, a, s);
    case kEpiBiasRelu: return launch_gemv_bias_relu(f16, a, s);
    case kEpiQkv: return launch_gemv_qkv(f16, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace djv
