// Single-query attention over the selected heads' KV cache, split over positions.
//
// [NOTES "Sparsified Attention"]: H_i(y) = D_i(y)^{-1} exp(y W_i^Q (W_i^K)^T X^T) X W_i^V,
// D_i = exp(.) 1, for each kept head i.  One decode token attends over positions 0..n of
// its sequence's cache (the new key/value were written at position n by the QKV step).
//
// A kept head has only n+1 keys, and a few dozen heads cannot fill 256 compute units,
// so the positions are cut into chunks: block (sequence b, head slot u, chunk c)
// computes for its positions the running max m, the sum l of exp(s - m) and the
// weighted value sum; a merge kernel (one block per head) rescales the chunks to the
// global max, divides and writes H_i.  Scores use max subtraction, which cancels exactly
// between numerator and D.  Keys and values of the chunk are all requested before the
// first score is formed.
//
// Lanes: a key/value row is dh elements = LPP lanes x one 16-byte vector; a block of 256
// threads covers 256/LPP positions per pass and makes 8 passes per chunk.
#include "common.hpp"

namespace djv {
namespace {

constexpr int kPasses = 8;

template <typename T, int DH>
struct AttnGeom {
    static constexpr int E = WTraits<T>::kPerVec;
    static constexpr int LPP = DH / E;          // lanes per position
    static constexpr int PPI = 256 / LPP;       // positions per pass
    static constexpr int CH = PPI * kPasses;    // positions per chunk
};

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    using G = AttnGeom<T, DH>;
    constexpr int E = G::E, LPP = G::LPP, PPI = G::PPI, CH = G::CH;
    __shared__ float sc[CH];
    __shared__ float wred[4];
    __shared__ float vred[PPI][DH];

    const int tid = threadIdx.x;
    const int cap = a.list.cap;
    const int b = blockIdx.x / cap, u = blockIdx.x - b * cap;
    const int chunk = blockIdx.y;
    const int count = read_count(a.list, a.flags);
    if (u >= count) return;
    const int unit = unit_of(a.list, u, a.flags);
    if (unit < 0) return;
    const int t0 = chunk * CH;
    const int t1 = min(t0 + CH, a.n + 1);
    const int grp = tid / LPP, sl = tid % LPP;

    const size_t head = ((size_t)b * a.h + unit) * a.n_cap;
    const char* Kb = reinterpret_cast<const char*>(a.Kc) + head * DH * sizeof(T);
    const char* Vb = reinterpret_cast<const char*>(a.Vc) + head * DH * sizeof(T);
    const float* q = a.q + ((size_t)b * cap + u) * DH + sl * E;
    float qs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qs[e] = q[e] * a.scale;

    // keys and values of this chunk, all in flight at once
    Vec16 kv[kPasses], vv[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int t = t0 + p * PPI + grp;
        kv[p] = t < t1 ? ldg16_nt(Kb + (size_t)t * DH * sizeof(T) + sl * 16) : Vec16{{0u, 0u, 0u, 0u}};
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int t = t0 + p * PPI + grp;
        vv[p] = t < t1 ? ldg16_nt(Vb + (size_t)t * DH * sizeof(T) + sl * 16) : Vec16{{0u, 0u, 0u, 0u}};
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float f[E];
        unpack<T>(kv[p], f);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(qs[e], f[e], s);
#pragma unroll
        for (int o = LPP / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
        const int t = t0 + p * PPI + grp;
        if (sl == 0) sc[p * PPI + grp] = t < t1 ? s : -INFINITY;
    }
    __syncthreads();

    // chunk max and exp weights
    float m = -INFINITY;
    for (int i = tid; i < CH; i += 256) m = fmaxf(m, sc[i]);
    m = wave_max(m);
    if (tid % kWave == 0) wred[tid / kWave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    __syncthreads();
    float l = 0.f;
    for (int i = tid; i < CH; i += 256) {
        const float w = (t0 + i < t1) ? __expf(sc[i] - m) : 0.f;
        sc[i] = w;
        l += w;
    }
    l = wave_sum(l);
    if (tid % kWave == 0) wred[tid / kWave] = l;
    __syncthreads();
    l = wred[0] + wred[1] + wred[2] + wred[3];

    // weighted values
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float f[E];
        unpack<T>(vv[p], f);
        const float w = sc[p * PPI + grp];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(w, f[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) vred[grp][sl * E + e] = acc[e];
    __syncthreads();
    float* part = a.part + (((size_t)b * cap + u) * a.nchunk + chunk) * (DH + 2);
    if (tid < DH) {
        float s = 0.f;
        for (int g = 0; g < PPI; ++g) s += vred[g][tid];
        part[2 + tid] = s;
    }
    if (tid == 0) {
        part[0] = m;
        part[1] = l;
    }
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
hipError_t run(const AttnArgs& a, hipStream_t s) {
    const int blocks = a.list.cap * a.B;
    if (blocks <= 0) return hipSuccess;
    prof_begin(a.prof, s);
    hipLaunchKernelGGL((attn_partial_kernel<T, DH>), dim3(blocks, a.nchunk), dim3(256), 0, s, a);
    prof_end(a.prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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

hipError_t launch_attention(bool f16, const AttnArgs& a, hipStream_t s) {
    if (f16) {
        if (a.dh == 128) return run<__half, 128>(a, s);
        if (a.dh == 64) return run<__half, 64>(a, s);
    } else {
        if (a.dh == 128) return run<float, 128>(a, s);
        if (a.dh == 64) return run<float, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace djv
