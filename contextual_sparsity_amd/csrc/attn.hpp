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
#pragma once
#include "common.hpp"

namespace djv {
namespace attn {

constexpr int kPasses = 8;

template <typename T, int DH>
struct AttnGeom {
    static constexpr int E = WTraits<T>::kPerVec;
    static constexpr int LPP = DH / E;          // lanes per position
    static constexpr int PPI = 256 / LPP;       // positions per pass
    static constexpr int CH = PPI * kPasses;    // positions per chunk
};

// One block of 256 threads: positions of chunk `chunk` of head slot u of sequence b
// (bu = b * cap + u).  Writes (m, l, weighted value sum) of the chunk.
template <typename T, int DH>
__device__ __forceinline__ void attn_partial_block(const AttnArgs& a, int bu, int chunk) {
    using G = AttnGeom<T, DH>;
    constexpr int E = G::E, LPP = G::LPP, PPI = G::PPI, CH = G::CH;
    __shared__ float sc[CH];
    __shared__ float wred[4];
    __shared__ float vred[PPI][DH];

    const int tid = threadIdx.x;
    const int cap = a.list.cap;
    const int b = bu / cap, u = bu - b * cap;
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

// Blocks of a launch running attention chunks: block i covers (bu, chunk) =
// (i / nchunk, i % nchunk), over B * cap head slots.
__device__ __forceinline__ int attn_blocks(const AttnArgs& a) { return a.B * a.list.cap * a.nchunk; }

template <typename T>
__device__ __forceinline__ void attn_block(const AttnArgs& a, int i) {
    const int bu = i / a.nchunk, chunk = i - bu * a.nchunk;
    if (a.dh == 128) attn_partial_block<T, 128>(a, bu, chunk);
    else attn_partial_block<T, 64>(a, bu, chunk);
}

}  // namespace attn
}  // namespace djv
