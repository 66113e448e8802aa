// Row-gather GEMV instantiated for the predictor layers (ReLU hidden layer, fp32 scores).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_store(bool f16, const GemvArgs& a, hipStream_t s) {
    return f16 ? gemv_detail::dispatch<__half, kEpiStore>(a, s)
               : gemv_detail::dispatch<float, kEpiStore>(a, s);
}

hipError_t launch_gemv_relu(bool f16, const GemvArgs& a, hipStream_t s) {
    return f16 ? gemv_detail::dispatch<__half, kEpiRelu>(a, s)
               : gemv_detail::dispatch<float, kEpiRelu>(a, s);
}

}  // namespace djv
