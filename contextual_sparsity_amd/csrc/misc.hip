// LayerNorm of the residual stream and the per-device flag word.
#include "common.hpp"

namespace djv {

// One flag word per device (zero at load), set by kernels that meet a bad index list.
__device__ unsigned g_flags = 0u;

namespace {

constexpr int kLnThreads = 1024;
constexpr int kLnPerThread = 16;   // d <= 16384 held in registers

// y = (x - mean) / sqrt(var + eps), biased variance, no affine; one block per row with
// the row held in registers (one round trip to memory).
// Pre-LN block input: [NOTES "LLM Contextually Sparse", third finding] (residual blocks
// with a Norm); eps, gamma = 1 and beta = 0 as in OPT.
__global__ __launch_bounds__(kLnThreads) void layernorm_kernel(int d, const float* x, float* y,
                                                               float eps) {
    __shared__ float red[kLnThreads / kWave];
    const float* xr = x + (size_t)blockIdx.x * d;
    float* yr = y + (size_t)blockIdx.x * d;
    float v[kLnPerThread];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kLnPerThread; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        v[i] = c < d ? xr[c] : 0.f;
        s += v[i];
    }
    const float mean = block_sum<kLnThreads>(s, red) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kLnPerThread; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        const float t = c < d ? v[i] - mean : 0.f;
        q = fmaf(t, t, q);
    }
    const float var = block_sum<kLnThreads>(q, red) / (float)d;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < kLnPerThread; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        if (c < d) yr[c] = (v[i] - mean) * rstd;
    }
}

// (mean, M2) of each kLnTile-column slice of x; one wave per (slice, row b).  The
// LayerNorm of x is applied from these by the consuming kernel.
__global__ __launch_bounds__(kWave) void ln_stats_kernel(int d, const float* x, float2* stats) {
    const int tile = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const int c0 = tile * kLnTile, n = min(kLnTile, d - c0);
    const float v = c < n ? x[(size_t)b * d + c0 + c] : 0.f;
    const float mean = wave_sum(v) / (float)n;
    const float dv = c < n ? v - mean : 0.f;
    const float M2 = wave_sum(dv * dv);
    if (c == 0) stats[(size_t)b * gridDim.x + tile] = make_float2(mean, M2);
}

// Plain streaming read of nvec 16-byte vectors.  Each block streams one contiguous share
// of the buffer, kProbeUnroll independent non-temporal loads per thread in flight (a block
// reads kProbeUnroll x 4 KiB contiguous per round; on this device contiguous per-block
// shares read faster and more evenly than a grid-stride loop).  The data is folded into one
// word that is stored only if it equals an arbitrary value, so the loads stay and the
// kernel writes (almost) nothing.
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr uint32_t kProbeSentinel = 0x5EEDC0DEu;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const Vec16* buf, size_t nvec,
                                                                   uint32_t* out) {
    const size_t share = (nvec + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * share;
    const size_t hi = lo + share < nvec ? lo + share : nvec;
    uint32_t acc = 0u;
    size_t i = lo + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += kProbeUnroll * kProbeThreads) {
        Vec16 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = ldg16_nt(buf + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].w[0] ^ v[u].w[1] ^ v[u].w[2] ^ v[u].w[3];
    }
    for (; i < hi; i += kProbeThreads) {
        const Vec16 v = ldg16_nt(buf + i);
        acc ^= v.w[0] ^ v.w[1] ^ v.w[2] ^ v.w[3];
    }
    if (acc == kProbeSentinel) *out = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
    if (bytes == 0 || bytes % 16 != 0) return hipErrorInvalidValue;
    const int blocks = device_cus() * 8;  // 8 blocks of 4 waves per compute unit
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const Vec16*>(buf), bytes / 16, out);
    return hipGetLastError();
}

hipError_t launch_layernorm(int B, int d, const float* x, float* y, float eps, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (d > kLnThreads * kLnPerThread) return hipErrorInvalidValue;
    hipLaunchKernelGGL(layernorm_kernel, dim3(B), dim3(kLnThreads), 0, s, d, x, y, eps);
    return hipGetLastError();
}

hipError_t launch_ln_stats(int B, int d, const float* x, float2* stats, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    const int tiles = (d + kLnTile - 1) / kLnTile;
    hipLaunchKernelGGL(ln_stats_kernel, dim3(tiles, B), dim3(kWave), 0, s, d, x, stats);
    return hipGetLastError();
}

ProfHook& prof_hook() {
    static ProfHook hook;
    return hook;
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

unsigned* device_flags() {
    static unsigned* addr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_flags)) != hipSuccess) return nullptr;
        addr[dev] = reinterpret_cast<unsigned*>(p);
    }
    return addr[dev];
}

}  // namespace djv
