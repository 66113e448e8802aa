// Row-gather GEMV: for each visited weight row, dot it with every batch row of y.
//
// This is the fused "gather + multiply" step: a kept unit's rows are read straight
// from the full weight tensor (neuron-major W1, head-major Wqkv, predictor rows) and
// multiplied in the same pass, with no gathered copy written or read back.
//   [BLOG section 3.2 "Kernel Fusion"]: unfused, the gather costs three passes (read W,
//   write the gathered W', read W'); fused, one.  [BLOG section 3.3 "Memory coalescing"]
//   names coalescing without detail; here every kept unit is one or more contiguous
//   rows, so each wave reads contiguous 1 KiB spans with 16-byte loads.
//
// Work decomposition (gfx950, wave64, 256-thread blocks):
//   * A "team" of TS threads (64 = one wave, or 256 = the whole block) owns one row at a
//     time; thread t of the team owns the 16-byte vectors t, t+TS, t+2TS, ... of every
//     row, so its slice of y is the same for all rows and stays in registers.
//   * A team processes G rows together: G*NV independent 16-byte loads are in flight per
//     thread before any arithmetic, which is what keeps HBM busy.
//   * Dot products: fp32 weights use fp32 FMA; fp16 weights use v_dot2_f32_f16 with y
//     packed to fp16 pairs (fp32 accumulation).
//   * Team reduction: wave butterfly, then (TS = 256) a 4-entry LDS combine.
#pragma once
#include "common.hpp"

namespace djv {
namespace gemv_detail {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <typename T> struct YSlice;
template <> struct YSlice<float> {
    float v[4];
    __device__ __forceinline__ void load(const float* y, int e0) {
        float4 t = *reinterpret_cast<const float4*>(y + e0);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
    __device__ __forceinline__ float dot(const Vec16& w, float acc) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(w.w[i]), v[i], acc);
        return acc;
    }
};
template <> struct YSlice<__half> {
    h2_t v[4];
    __device__ __forceinline__ void load(const float* y, int e0) {
        float4 a = *reinterpret_cast<const float4*>(y + e0);
        float4 b = *reinterpret_cast<const float4*>(y + e0 + 4);
        v[0] = h2_t{(_Float16)a.x, (_Float16)a.y};
        v[1] = h2_t{(_Float16)a.z, (_Float16)a.w};
        v[2] = h2_t{(_Float16)b.x, (_Float16)b.y};
        v[3] = h2_t{(_Float16)b.z, (_Float16)b.w};
    }
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 4; ++i) v[i] = h2_t{(_Float16)0.f, (_Float16)0.f};
    }
    __device__ __forceinline__ float dot(const Vec16& w, float acc) const {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.w[i]), v[i], acc, false);
        return acc;
    }
};

// Resolve visited row r to (unit slot, unit, weight row); row < 0 when skipped.
struct RowRef {
    int u, unit, sub;
    long long row;
};

__device__ __forceinline__ RowRef resolve(const GemvArgs& a, int r) {
    RowRef rr;
    rr.u = r / a.rpu;
    rr.sub = r - rr.u * a.rpu;
    rr.unit = unit_of(a.list, rr.u, a.flags);
    rr.row = rr.unit < 0 ? -1 : (long long)rr.unit * a.rpu + rr.sub;
    return rr;
}

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int r, int b, float acc) {
    const RowRef rr = resolve(a, r);
    switch (EPI) {
    case kEpiStore:
        a.out[(size_t)b * a.ld + r] = acc;
        break;
    case kEpiRelu:
        a.out[(size_t)b * a.ld + r] = fmaxf(acc, 0.f);
        break;
    case kEpiBiasRelu: {
        float v = 0.f;
        if (rr.unit >= 0)
            v = fmaxf(acc + to_f32<T>(reinterpret_cast<const T*>(a.bias)[rr.unit]), 0.f);
        a.out[(size_t)b * a.ld + rr.u] = v;
        break;
    }
    case kEpiQkv: {
        if (rr.unit < 0) break;
        const int part = rr.sub / a.dh, c = rr.sub - part * a.dh;
        if (part == 0) {
            a.out[((size_t)b * a.list.cap + rr.u) * a.dh + c] = acc;
        } else {
            T* cache = reinterpret_cast<T*>(part == 1 ? a.Kc : a.Vc);
            cache[(((size_t)b * a.h + rr.unit) * a.n_cap + a.n) * a.dh + c] = to_store<T>(acc);
        }
        break;
    }
    default:
        break;
    }
}

template <typename T, int TS, int NV, int NB, int G, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    constexpr int E = WTraits<T>::kPerVec;
    constexpr int NT = 256 / TS;
    constexpr int NW = TS / kWave;  // waves per team
    __shared__ float red[4][G * NB];

    const int tid = threadIdx.x;
    const int tm = tid / TS, lt = tid % TS, wv = lt / kWave, ln = tid % kWave;
    const int nvec = a.cols / E;
    const int count = read_count(a.list, a.flags);
    const int rows = count * a.rpu;
    const int groups = (rows + G - 1) / G;
    const char* Wb = reinterpret_cast<const char*>(a.W);
    const size_t row_bytes = (size_t)a.cols * sizeof(T);

    // this thread's slice of every batch row of y
    YSlice<T> ys[NB][NV];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = lt + TS * i;
            if (b < a.B && v < nvec) ys[b][i].load(a.y + (size_t)b * a.cols, v * E);
            else ys[b][i].zero();
        }

    for (int grp = blockIdx.x * NT + tm; grp < groups; grp += gridDim.x * NT) {
        Vec16 w[G][NV];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int r = grp * G + g;
            long long row = -1;
            if (r < rows) row = resolve(a, r).row;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int v = lt + TS * i;
                if (row >= 0 && v < nvec)
                    w[g][i] = ldg16_nt(Wb + (size_t)row * row_bytes + (size_t)v * 16);
                else
                    w[g][i] = Vec16{{0u, 0u, 0u, 0u}};
            }
        }
        float acc[G][NB];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < NV; ++i) s = ys[b][i].dot(w[g][i], s);
                acc[g][b] = wave_sum(s);
            }
        if constexpr (NW == 1) {
            if (ln < G * NB) {
                // lane j of the wave writes result j (all lanes hold every sum)
                float v = 0.f;
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        if (ln == g * NB + b) v = acc[g][b];
                const int g = ln / NB, b = ln % NB;
                const int r = grp * G + g;
                if (r < rows && b < a.B) epilogue<T, EPI>(a, r, b, v);
            }
        } else {
            if (ln == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int b = 0; b < NB; ++b) red[wv][g * NB + b] = acc[g][b];
            }
            __syncthreads();
            if (tid < G * NB) {
                float v = 0.f;
#pragma unroll
                for (int q = 0; q < NW; ++q) v += red[q][tid];
                const int g = tid / NB, b = tid % NB;
                const int r = grp * G + g;
                if (r < rows && b < a.B) epilogue<T, EPI>(a, r, b, v);
            }
            __syncthreads();
        }
    }
}

template <typename T, int TS, int NB, int EPI>
hipError_t dispatch_nv(const GemvArgs& a, int nv, dim3 grid, hipStream_t s) {
#define DJV_GEMV_CASE(NVV, GG)                                                                 \
    case NVV:                                                                                  \
        prof_begin(a.prof, s);                                                                 \
        hipLaunchKernelGGL((gemv_kernel<T, TS, NVV, NB, GG, EPI>), grid, dim3(256), 0, s, a);   \
        prof_end(a.prof, s);                                                                   \
        break;
    if constexpr (TS == 64) {
        switch (nv) {
            DJV_GEMV_CASE(1, 4)
            DJV_GEMV_CASE(2, 4)
            DJV_GEMV_CASE(3, 4)
        default:
            return hipErrorInvalidValue;
        }
    } else {
        switch (nv) {
            DJV_GEMV_CASE(1, 4)
            DJV_GEMV_CASE(2, 4)
            DJV_GEMV_CASE(3, 3)
            DJV_GEMV_CASE(4, 3)
            DJV_GEMV_CASE(5, 2)
            DJV_GEMV_CASE(6, 2)
            DJV_GEMV_CASE(7, 2)
            DJV_GEMV_CASE(8, 2)
        default:
            return hipErrorInvalidValue;
        }
    }
#undef DJV_GEMV_CASE
    return hipGetLastError();
}

template <typename T, int EPI>
hipError_t dispatch(const GemvArgs& a, hipStream_t s) {
    constexpr int E = WTraits<T>::kPerVec;
    const int nvec = a.cols / E;
    const int rows_cap = a.list.cap * a.rpu;
    if (rows_cap <= 0) return hipSuccess;
    const bool small = nvec <= 3 * 64;
    const int TS = small ? 64 : 256;
    const int nv = (nvec + TS - 1) / TS;
    int G;
    if (small) G = 4;
    else G = nv <= 2 ? 4 : (nv <= 4 ? 3 : 2);
    const int NT = 256 / TS;
    const int groups = (rows_cap + G - 1) / G;
    int blocks = (groups + NT - 1) / NT;
    const int max_blocks = 256 * 8;
    if (blocks > max_blocks) blocks = max_blocks;
    dim3 grid(blocks);
    const int nb = a.B <= 1 ? 1 : (a.B <= 2 ? 2 : 4);
    if (small) {
        if (nb == 1) return dispatch_nv<T, 64, 1, EPI>(a, nv, grid, s);
        if (nb == 2) return dispatch_nv<T, 64, 2, EPI>(a, nv, grid, s);
        return dispatch_nv<T, 64, 4, EPI>(a, nv, grid, s);
    }
    if (nb == 1) return dispatch_nv<T, 256, 1, EPI>(a, nv, grid, s);
    if (nb == 2) return dispatch_nv<T, 256, 2, EPI>(a, nv, grid, s);
    return dispatch_nv<T, 256, 4, EPI>(a, nv, grid, s);
}

}  // namespace gemv_detail
}  // namespace djv
