// Row-gather GEMV instantiated for the head-sparse Q/K/V projection with the KV-cache append.
#include "gemv.hpp"

namespace djv {

hipError_t launch_gemv_qkv(bool f16, const GemvArgs& a, hipStream_t s) {
    return f16 ? gemv_detail::dispatch<__half, kEpiQkv>(a, s)
               : gemv_detail::dispatch<float, kEpiQkv>(a, s);
}

}  // namespace djv
