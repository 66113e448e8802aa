// Row-gather GEMV instantiated for the MLP up-projection of the kept neurons (bias + ReLU).
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_bias_relu(bool f16, const GemvArgs& a, hipStream_t s) {
    return f16 ? gemv_detail::dispatch<__half, kEpiBiasRelu>(a, s)
               : gemv_detail::dispatch<float, kEpiBiasRelu>(a, s);
}

}  // namespace djv
