// Lazy K/V for the heads a step does not select.
//
// [NOTES "Sparsity operator for Attention"]: a step computes and stores K/V only for the
// predicted heads S_A, and keeps a copy of its attention input y for the other heads;
// when a head that skipped earlier steps is selected again, its missing K/V are computed
// from the saved inputs before it attends.  The cache then holds, for every head, what
// computing all heads' K/V at every step would have stored.
//
// One launch per layer and step at position n, before the layer's Q/K/V launch:
//   blocks [0, B):      Y[b, n] = y[b] (the normalised input, as the Q/K/V GEMV forms it);
//   block B:            kv_next[i] = n + 1 for the selected heads, kv_prev[i] otherwise;
//   the other blocks:   for each selected head i and each position p in [kv_prev[i], n),
//                       K[b, i, p] = W_i^K Y[b, p] and V[b, i, p] = W_i^V Y[b, p], rounded
//                       to the cache type; a block per four output rows (K or V columns),
//                       its waves taking every fourth position, two per pass.
// kv_len holds two buffers of h entries read and written alternately by the parity of n,
// so no block reads an entry that another block of the same launch writes.
#include "gemv.hpp"

namespace djv {

namespace {

constexpr int kLazyThreads = 256;
constexpr int kLazyRows = kLazyThreads / kWave;  // waves per block: position phases of a row tile
constexpr int kSaveBatch = 16;  // values of the saved input per thread in flight
constexpr int kSaveVals = 16384 / kLazyThreads;  // a whole row per thread set (d <= 16384)
constexpr int kRowTile = 4;     // output rows per catch-up block
constexpr int kPosTile = 2;     // positions per catch-up wave and pass
constexpr int kChunkVec = 256;  // weight vectors per row staged in LDS at a time (16 KiB per tile)

template <typename T>
__global__ __launch_bounds__(kLazyThreads) void lazy_kv_kernel(LazyKvArgs a) {
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int bid = blockIdx.x;
    if (bid < a.B) {
        // save this step's input row b, normalised as the Q/K/V launch normalises it
        // (loads batched ahead of the stores: the source and Y may not be assumed apart,
        // so a plain copy loop would wait for each load in turn)
        const int b = bid;
        float* dst = a.Y + ((size_t)b * a.n_cap + a.n) * a.d;
        const float* src = (a.in.y ? a.in.y : a.in.x) + (size_t)b * a.d;
        float mean = 0.f, rstd = 1.f;
        if (a.in.own_stats) {
            // LN of x with its moments summed here, the form the GEMVs that read the in-place
            // residual stream use (one pass of deviations from the row's first element).  The
            // row stays in registers: one round of loads (addresses clamped into the row), the
            // block's sums, then the normalised values stored.
            __shared__ float part[2][kLazyThreads / kWave];
            const float sh = src[0];
            float v[kSaveVals];
#pragma unroll
            for (int k = 0; k < kSaveVals; ++k) v[k] = src[min(tid + k * kLazyThreads, a.d - 1)];
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int k = 0; k < kSaveVals; ++k) {
                const float t = tid + k * kLazyThreads < a.d ? v[k] - sh : 0.f;
                s1 += t;
                s2 = fmaf(t, t, s2);
            }
            s1 = wave_sum(s1);
            s2 = wave_sum(s2);
            if (lane == 0) {
                part[0][wv] = s1;
                part[1][wv] = s2;
            }
            __syncthreads();
            float t1 = 0.f, t2 = 0.f;
#pragma unroll
            for (int w = 0; w < kLazyThreads / kWave; ++w) {
                t1 += part[0][w];
                t2 += part[1][w];
            }
            const float inv_n = 1.0f / (float)a.d, md = t1 * inv_n;
            mean = sh + md;
            rstd = 1.0f / sqrtf(fmaxf(t2 * inv_n - md * md, 0.f) + a.in.eps);
#pragma unroll
            for (int k = 0; k < kSaveVals; ++k) {
                const int e = tid + k * kLazyThreads;
                if (e < a.d) dst[e] = (v[k] - mean) * rstd;
            }
            return;
        }
        if (!a.in.y) gemv_detail::row_moments(a.in, a.d, b, mean, rstd);
        for (int e0 = tid; e0 < a.d; e0 += kLazyThreads * kSaveBatch) {
            float v[kSaveBatch];
#pragma unroll
            for (int k = 0; k < kSaveBatch; ++k) {
                const int e = e0 + k * kLazyThreads;
                v[k] = e < a.d ? src[e] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < kSaveBatch; ++k) {
                const int e = e0 + k * kLazyThreads;
                if (e < a.d) dst[e] = (v[k] - mean) * rstd;
            }
        }
        return;
    }
    const int count = read_count(a.heads, a.flags);
    if (bid == a.B) {
        for (int i = tid; i < a.h; i += kLazyThreads) a.kv_next[i] = a.kv_prev[i];
        __syncthreads();
        for (int u = tid; u < count; u += kLazyThreads) {
            const int i = unit_of(a.heads, u, a.flags);
            if (i >= 0) a.kv_next[i] = a.n + 1;
        }
        return;
    }
    // catch-up: block g owns kRowTile consecutive output rows j0 .. j0+3 of head slot u
    // (j < dh: K column j, else V column j - dh; a tile never straddles the two since
    // dh % 4 == 0), and its wave w the positions start + w, start + w + 4, ..., kPosTile of
    // them per pass: each weight vector serves kPosTile positions and each input vector
    // kRowTile rows, and the four waves walk a head's skipped positions side by side.  The
    // tile's weights pass through LDS in chunks of kChunkVec vectors per row, each chunk read
    // from memory once for all four waves.  Every test before the first barrier depends
    // only on the block's tile, so the block takes the same path throughout.
    __shared__ Vec16 wsh[kRowTile][kChunkVec];
    const int tiles_per_head = 2 * a.dh / kRowTile;
    const int g = bid - a.B - 1;
    const int u = g / tiles_per_head, j0 = (g - u * tiles_per_head) * kRowTile;
    if (u >= count) return;  // uniform over the block
    const int i = unit_of(a.heads, u, a.flags);
    if (i < 0) return;
    const int part = 1 + j0 / a.dh, c0 = j0 % a.dh;
    const int start = max(a.kv_prev[i], 0);
    if (start >= a.n) return;
    constexpr int E = WTraits<T>::kPerVec;
    const Vec16* W = reinterpret_cast<const Vec16*>(reinterpret_cast<const T*>(a.Wqkv) +
                                                    (((size_t)i * 3 + part) * a.dh + c0) * a.d);
    T* cache = reinterpret_cast<T*>(part == 1 ? a.Kc : a.Vc);
    const int nvec = a.d / E;  // 16-byte weight vectors per row (d % 8 == 0)
    const int passes = (a.n - start + kLazyRows * kPosTile - 1) / (kLazyRows * kPosTile);
    constexpr int kLaneVec = kChunkVec / kWave;  // a lane's vectors of a chunk, per row
    for (int ps = 0; ps < passes; ++ps) {
        const int p0 = start + wv + ps * kLazyRows * kPosTile;  // positions p0 + 4t
        for (int b = 0; b < a.B; ++b) {
            const float* yb = a.Y + (size_t)b * a.n_cap * a.d;
            // per (row, position): the lane's vectors v = lane, lane + 64, ... in order
            float acc[kRowTile][kPosTile];
#pragma unroll
            for (int r = 0; r < kRowTile; ++r)
#pragma unroll
                for (int t = 0; t < kPosTile; ++t) acc[r][t] = 0.f;
            for (int cv = 0; cv < nvec; cv += kChunkVec) {
                __syncthreads();  // the previous chunk's readers are done
                // the tile's weights of the chunk and this wave's inputs of it, all requested
                // before either is used (one round trip per chunk)
                Vec16 st[kRowTile * kChunkVec / kLazyThreads];
#pragma unroll
                for (int k = 0; k < kRowTile * kChunkVec / kLazyThreads; ++k) {
                    const int e = tid + k * kLazyThreads, r = e / kChunkVec, v = e - r * kChunkVec;
                    st[k] = W[(size_t)r * nvec + min(cv + v, nvec - 1)];  // clamped; unused past the end
                }
                float yf[kPosTile][kLaneVec][8];
#pragma unroll
                for (int t = 0; t < kPosTile; ++t) {
                    const int p = min(p0 + t * kLazyRows, a.n - 1);  // clamped; not stored past n
#pragma unroll
                    for (int k = 0; k < kLaneVec; ++k) {
                        const int v = min(cv + lane + k * kWave, nvec - 1);
                        const float* y = yb + (size_t)p * a.d + (size_t)v * E;
#pragma unroll
                        for (int q = 0; q < E / 4; ++q) {
                            const float4 f = *reinterpret_cast<const float4*>(y + 4 * q);
                            yf[t][k][4 * q] = f.x; yf[t][k][4 * q + 1] = f.y;
                            yf[t][k][4 * q + 2] = f.z; yf[t][k][4 * q + 3] = f.w;
                        }
                    }
                }
#pragma unroll
                for (int k = 0; k < kRowTile * kChunkVec / kLazyThreads; ++k) {
                    const int e = tid + k * kLazyThreads, r = e / kChunkVec, v = e - r * kChunkVec;
                    wsh[r][v] = st[k];
                }
                // the inputs in the form the dot products take (packed fp16 pairs against fp16
                // weights, as the Q/K/V GEMV rounds them; fp32 against fp32 weights); a vector
                // past the row end gets zero inputs and adds exact zeros (weights are finite)
                gemv_detail::YSlice<T> ysl[kPosTile][kLaneVec];
#pragma unroll
                for (int t = 0; t < kPosTile; ++t)
#pragma unroll
                    for (int k = 0; k < kLaneVec; ++k) {
                        if (cv + lane + k * kWave < nvec) ysl[t][k].set(yf[t][k], 0);
                        else ysl[t][k].zero();
                    }
                __syncthreads();
#pragma unroll
                for (int k = 0; k < kLaneVec; ++k)
#pragma unroll
                    for (int r = 0; r < kRowTile; ++r) {
                        const Vec16 w = wsh[r][lane + k * kWave];
#pragma unroll
                        for (int t = 0; t < kPosTile; ++t) acc[r][t] = ysl[t][k].dot(w, acc[r][t]);
                    }
            }
#pragma unroll
            for (int r = 0; r < kRowTile; ++r)
#pragma unroll
                for (int t = 0; t < kPosTile; ++t) {
                    const float v = wave_sum(acc[r][t]);
                    const int p = p0 + t * kLazyRows;
                    if (lane == 0 && p < a.n)
                        cache[(((size_t)b * a.h + i) * a.n_cap + p) * a.dh + c0 + r] = to_store<T>(v);
                }
        }
    }
}

}  // namespace

hipError_t launch_lazy_kv(bool f16, const LazyKvArgs& a, hipStream_t s) {
    // an empty head list (top-k with k = 0) still saves the step's input and carries the
    // valid lengths over; there is nothing to catch up
    if (a.B < 1 || a.d < 1 || a.h < 1 || a.n < 0 || a.n >= a.n_cap || a.heads.cap < 0 ||
        (a.in.own_stats && (!a.in.x || a.in.y)))
        return hipErrorInvalidValue;
    const long long tiles = (long long)a.heads.cap * 2 * a.dh / kRowTile;  // dh % 4 == 0
    const dim3 grid((unsigned)(a.B + 1 + tiles));
    if (f16)
        hipLaunchKernelGGL(lazy_kv_kernel<__half>, grid, dim3(kLazyThreads), 0, s, a);
    else
        hipLaunchKernelGGL(lazy_kv_kernel<float>, grid, dim3(kLazyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace djv
