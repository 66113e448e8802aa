// Output norms of units across a batch, the scores of the "true" selection.
//
// [BLOG section 1 "Contextual Sparsity"]: a dense pass over the input records, per head,
// the L2 norm of that head's output matrix (tokens x d_h, before the output projection),
// and per MLP neuron the L2 norm of its row of activations across the tokens; the units
// with the largest norms are the ones that matter for that input.  Here the tokens are
// the batch rows of one decode step: score[u] = sqrt(sum_b sum_c v[b, u, c]^2), fp32.
#include "common.hpp"

namespace djv {
namespace {

constexpr int kNormThreads = 256;

// One unit of one value per batch row (neurons): a thread per unit.
__global__ __launch_bounds__(kNormThreads) void norms_narrow_kernel(const float* v, int B, int units,
                                                                    float* scores) {
    const int u = blockIdx.x * kNormThreads + threadIdx.x;
    if (u >= units) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
        const float x = v[(size_t)b * units + u];
        s = fmaf(x, x, s);
    }
    scores[u] = sqrtf(s);
}

// Units of w values per batch row (heads, w = d_h): a wave per unit, lanes over the values.
__global__ __launch_bounds__(kNormThreads) void norms_wide_kernel(const float* v, int B, int units,
                                                                  int w, float* scores) {
    const int u = blockIdx.x * (kNormThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (u >= units) return;  // uniform over the wave
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
        const float* row = v + ((size_t)b * units + u) * w;
        for (int c = lane; c < w; c += kWave) s = fmaf(row[c], row[c], s);
    }
    s = wave_sum(s);
    if (lane == 0) scores[u] = sqrtf(s);
}

}  // namespace

hipError_t launch_unit_norms(const float* v, int B, int units, int w, float* scores, hipStream_t s) {
    if (B < 1 || units < 1 || w < 1) return hipErrorInvalidValue;
    if (w == 1) {
        hipLaunchKernelGGL(norms_narrow_kernel, dim3((units + kNormThreads - 1) / kNormThreads),
                           dim3(kNormThreads), 0, s, v, B, units, scores);
    } else {
        constexpr int per = kNormThreads / kWave;
        hipLaunchKernelGGL(norms_wide_kernel, dim3((units + per - 1) / per), dim3(kNormThreads), 0, s, v, B,
                           units, w, scores);
    }
    return hipGetLastError();
}

}  // namespace djv
