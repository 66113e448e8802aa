// Standalone launches of the split-position attention (see attn.hpp) and its merge.
#include "attn.hpp"

namespace djv {
namespace {

using namespace attn;

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    attn_partial_block<T, DH>(a, blockIdx.x, blockIdx.y);
}

// H[b, u] = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c over the chunks of a head.
// One block of dh threads per (sequence, head slot); chunk maxima and weights go through
// LDS, and each thread issues its column's loads in batches of 8 before adding.
template <int DH>
__global__ __launch_bounds__(DH) void attn_merge_kernel(AttnArgs a) {
    __shared__ float cw[kAttnMaxChunks];
    __shared__ float red[DH / kWave];
    const int cap = a.list.cap;
    const int b = blockIdx.x / cap, u = blockIdx.x - b * cap;
    const int tid = threadIdx.x;
    const int count = read_count(a.list, nullptr);
    if (u >= count) return;
    float* H = a.H + ((size_t)b * cap + u) * DH;
    if (unit_of(a.list, u, nullptr) < 0) {
        H[tid] = 0.f;
        return;
    }
    const float* hp = a.part + ((size_t)b * cap + u) * a.nchunk * (DH + 2);
    float m = -INFINITY;
    for (int c = tid; c < a.nchunk; c += DH) {
        cw[c] = hp[(size_t)c * (DH + 2)];
        m = fmaxf(m, cw[c]);
    }
    m = wave_max(m);
    if (tid % kWave == 0) red[tid / kWave] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int q = 1; q < DH / kWave; ++q) M = fmaxf(M, red[q]);
    for (int c = tid; c < a.nchunk; c += DH) cw[c] = __expf(cw[c] - M);
    __syncthreads();
    float L = 0.f, acc = 0.f;
    int c = 0;
    for (; c + 8 <= a.nchunk; c += 8) {
        float lv[8], av[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lv[k] = hp[(size_t)(c + k) * (DH + 2) + 1];
            av[k] = hp[(size_t)(c + k) * (DH + 2) + 2 + tid];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            L = fmaf(lv[k], cw[c + k], L);
            acc = fmaf(av[k], cw[c + k], acc);
        }
    }
    for (; c < a.nchunk; ++c) {
        L = fmaf(hp[(size_t)c * (DH + 2) + 1], cw[c], L);
        acc = fmaf(hp[(size_t)c * (DH + 2) + 2 + tid], cw[c], acc);
    }
    H[tid] = acc / L;
}

template <typename T, int DH>
hipError_t run(const AttnArgs& a, bool merge, hipStream_t s) {
    const int blocks = a.list.cap * a.B;
    if (blocks <= 0) return hipSuccess;
    prof_begin(a.prof, s);
    hipLaunchKernelGGL((attn_partial_kernel<T, DH>), dim3(blocks, a.nchunk), dim3(256), 0, s, a);
    prof_end(a.prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !merge) return e;
    hipLaunchKernelGGL((attn_merge_kernel<DH>), dim3(blocks), dim3(DH), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Positions per chunk for a head width and element size (must match AttnGeom).
static int chunk_positions(bool f16, int dh) {
    const int E = f16 ? 8 : 4;
    return (256 / (dh / E)) * kPasses;
}

int attn_chunk_for(bool f16, int dh) { return chunk_positions(f16, dh); }

hipError_t launch_attention(bool f16, const AttnArgs& a, bool merge, hipStream_t s) {
    if (f16) {
        if (a.dh == 128) return run<__half, 128>(a, merge, s);
        if (a.dh == 64) return run<__half, 64>(a, merge, s);
    } else {
        if (a.dh == 128) return run<float, 128>(a, merge, s);
        if (a.dh == 64) return run<float, 64>(a, merge, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace djv
