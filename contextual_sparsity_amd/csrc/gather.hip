// The unfused gather of the fusion ablation: the kept rows copied into a contiguous buffer
// ([BLOG section 3.2 "Kernel Fusion"]: read W, write W', read W' again in the product).
// One block per output row; 16-byte vectors when the row allows, else 4- or 2-byte words
// (a bias vector is a gather of one-element rows).
#include "common.hpp"

namespace djv {
namespace {

struct GatherArgs {
    const char* W;
    char* out;
    UnitList list;
    int rpu;
    size_t row_bytes;
    unsigned* flags;
};

template <int V>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs a) {
    const int orow = blockIdx.x;                 // output row: slot * rpu + j
    const int slot = orow / a.rpu, j = orow - slot * a.rpu;
    const int count = read_count(a.list, a.flags);
    int unit = -1;
    if (slot < count) unit = unit_of(a.list, slot, a.flags);
    char* dst = a.out + (size_t)orow * a.row_bytes;
    const char* src = unit < 0 ? nullptr : a.W + ((size_t)unit * a.rpu + j) * a.row_bytes;
    const size_t n = a.row_bytes / V;
    if constexpr (V == 16) {
        for (size_t i = threadIdx.x; i < n; i += 256) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (src) v = reinterpret_cast<const uint4*>(src)[i];
            reinterpret_cast<uint4*>(dst)[i] = v;
        }
    } else if constexpr (V == 4) {
        for (size_t i = threadIdx.x; i < n; i += 256) {
            uint32_t v = 0u;
            if (src) v = reinterpret_cast<const uint32_t*>(src)[i];
            reinterpret_cast<uint32_t*>(dst)[i] = v;
        }
    } else {
        for (size_t i = threadIdx.x; i < n; i += 256) {
            unsigned short v = 0;
            if (src) v = reinterpret_cast<const unsigned short*>(src)[i];
            reinterpret_cast<unsigned short*>(dst)[i] = v;
        }
    }
}

}  // namespace

hipError_t launch_gather_rows(const void* W, void* out, const UnitList& list, int rpu, size_t row_bytes,
                              unsigned* flags, hipStream_t s) {
    GatherArgs a{static_cast<const char*>(W), static_cast<char*>(out), list, rpu, row_bytes, flags};
    const dim3 grid((unsigned)((size_t)list.cap * rpu));
    if (row_bytes % 16 == 0) hipLaunchKernelGGL(gather_rows_kernel<16>, grid, dim3(256), 0, s, a);
    else if (row_bytes % 4 == 0) hipLaunchKernelGGL(gather_rows_kernel<4>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gather_rows_kernel<2>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace djv
