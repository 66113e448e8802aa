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
//   * The activation rows are either given, or LayerNorm(x) is applied while the slice is
//     loaded, from per-slice (mean, M2) statistics written by the kernel that produced x,
//     so no separate normalisation pass runs.
//   * One launch may serve two weight matrices of the same row length (the head and the
//     neuron predictor): blocks [0, seg[0].blocks) serve the first, the rest the second.
#pragma once
#include "common.hpp"

namespace djv {
namespace gemv_detail {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <typename T> struct YSlice;
template <> struct YSlice<float> {
    float v[4];
    __device__ __forceinline__ void set(const float (&f)[8], int o) {
        v[0] = f[o]; v[1] = f[o + 1]; v[2] = f[o + 2]; v[3] = f[o + 3];
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
    __device__ __forceinline__ void set(const float (&f)[8], int) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = h2_t{(_Float16)f[2 * i], (_Float16)f[2 * i + 1]};
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = h2_t{(_Float16)0.f, (_Float16)0.f};
    }
    __device__ __forceinline__ float dot(const Vec16& w, float acc) const {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.w[i]), v[i], acc, false);
        return acc;
    }
};

// Loads the E activation values at column e0 of row b (y, or x before normalisation).
template <typename T>
__device__ __forceinline__ void load_raw(const RowInput& in, int cols, int b, int e0, float (&f)[8]) {
    constexpr int E = WTraits<T>::kPerVec;
    const float* src = (in.y ? in.y : in.x) + (size_t)b * cols + e0;
#pragma unroll
    for (int i = 0; i < E; i += 4) {
        const float4 t = *reinterpret_cast<const float4*>(src + i);
        f[i] = t.x; f[i + 1] = t.y; f[i + 2] = t.z; f[i + 3] = t.w;
    }
}

// LayerNorm moments of row b from its slice statistics; each lane loads its (at most
// four) slices at once.  cols <= 16384, so ntiles <= 256.
__device__ __forceinline__ void row_moments(const RowInput& in, int cols, int b, float& mean,
                                            float& rstd) {
    const int lane = threadIdx.x % kWave;
    const float2* st = in.stats + (size_t)b * in.ntiles;
    float2 v[4];
    float nt[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = lane + kWave * q;
        v[q] = st[min(t, in.ntiles - 1)];
        nt[q] = t < in.ntiles ? (float)min(kLnTile, cols - t * kLnTile) : 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s = fmaf(nt[q], v[q].x, s);
    const float m = wave_sum(s) / (float)cols;
    float qs = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float dm = v[q].x - m;
        qs += nt[q] > 0.f ? v[q].y + nt[q] * dm * dm : 0.f;
    }
    mean = m;
    rstd = 1.0f / sqrtf(wave_sum(qs) / (float)cols + in.eps);
}

// Resolve visited row r to (unit slot, unit, weight row); row < 0 when skipped.
struct RowRef {
    int u, unit, sub;
    long long row;
};

__device__ __forceinline__ RowRef resolve(const GemvSeg& S, int r, unsigned* flags) {
    RowRef rr;
    rr.u = r / S.rpu;
    rr.sub = r - rr.u * S.rpu;
    rr.unit = unit_of(S.list, rr.u, flags);
    rr.row = rr.unit < 0 ? -1 : (long long)rr.unit * S.rpu + rr.sub;
    return rr;
}

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, const GemvSeg& S, int r, int b, float acc) {
    const RowRef rr = resolve(S, r, a.flags);
    switch (EPI) {
    case kEpiStore:
        S.out[(size_t)b * S.ld + r] = acc;
        break;
    case kEpiRelu:
        S.out[(size_t)b * S.ld + r] = fmaxf(acc, 0.f);
        break;
    case kEpiBiasRelu: {
        float v = 0.f;
        if (rr.unit >= 0)
            v = fmaxf(acc + to_f32<T>(reinterpret_cast<const T*>(a.bias)[rr.unit]), 0.f);
        S.out[(size_t)b * S.ld + rr.u] = v;
        break;
    }
    case kEpiQkv: {
        if (rr.unit < 0) break;
        const int part = rr.sub / a.dh, c = rr.sub - part * a.dh;
        if (part == 0) {
            S.out[((size_t)b * S.list.cap + rr.u) * a.dh + c] = acc;
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
    const int sg = (a.nseg > 1 && (int)blockIdx.x >= a.seg[0].blocks) ? 1 : 0;
    const GemvSeg S = a.seg[sg];
    const int bid = (int)blockIdx.x - (sg ? a.seg[0].blocks : 0);
    const int nvec = a.cols / E;
    const int count = read_count(S.list, a.flags);
    const int rows = count * S.rpu;
    const int groups = (rows + G - 1) / G;
    const char* Wb = reinterpret_cast<const char*>(S.W);
    const size_t row_bytes = (size_t)a.cols * sizeof(T);

    // all rows of a group are resolved (index loads) before any weight load is issued, so
    // one round trip covers the indices and one the weights
    auto load_group = [&](Vec16 (&w)[G][NV], int grp) {
        long long row[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int r = grp * G + g;
            row[g] = r < rows ? resolve(S, r, a.flags).row : -1;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int v = lt + TS * i;
                if (row[g] >= 0 && v < nvec)
                    w[g][i] = ldg16_nt(Wb + (size_t)row[g] * row_bytes + (size_t)v * 16);
                else
                    w[g][i] = Vec16{{0u, 0u, 0u, 0u}};
            }
    };

    // the first group's weights are requested before the activation slice is read
    int grp = bid * NT + tm;
    Vec16 w[G][NV];
    if (grp < groups) load_group(w, grp);

    // this thread's slice of every batch row (loads clamped in range, then masked)
    float raw[NB][NV][8];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = min(lt + TS * i, nvec - 1);
            load_raw<T>(S.in, a.cols, min(b, a.B - 1), v * E, raw[b][i]);
        }
    YSlice<T> ys[NB][NV];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float mean = 0.f, rstd = 1.f;
        if (!S.in.y) row_moments(S.in, a.cols, min(b, a.B - 1), mean, rstd);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool ok = b < a.B && lt + TS * i < nvec;
#pragma unroll
            for (int e = 0; e < E; ++e) raw[b][i][e] = ok ? (raw[b][i][e] - mean) * rstd : 0.f;
            ys[b][i].set(raw[b][i], 0);
        }
    }

    while (grp < groups) {
        float acc[G][NB];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < NV; ++i) s = ys[b][i].dot(w[g][i], s);
                acc[g][b] = s;
            }
        // the next group's loads go out before this group's reduction
        const int cur = grp;
        grp += S.blocks * NT;
        if (grp < groups) load_group(w, grp);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[g][b] = wave_sum(acc[g][b]);
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
                const int r = cur * G + g;
                if (r < rows && b < a.B) epilogue<T, EPI>(a, S, r, b, v);
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
                const int r = cur * G + g;
                if (r < rows && b < a.B) epilogue<T, EPI>(a, S, r, b, v);
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

// Chooses the team size, vectors per thread and rows per team, sizes each segment's
// share of the grid, and launches.
template <typename T, int EPI>
hipError_t dispatch(const GemvArgs& a_in, hipStream_t s) {
    constexpr int E = WTraits<T>::kPerVec;
    GemvArgs a = a_in;
    const int nvec = a.cols / E;
    const bool small = nvec <= 3 * 64;
    const int TS = small ? 64 : 256;
    const int nv = (nvec + TS - 1) / TS;
    int G;
    if (small) G = 4;
    else G = nv <= 2 ? 4 : (nv <= 4 ? 3 : 2);
    const int NT = 256 / TS;
    const int max_blocks = 256 * 64;
    int total = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const int rows_cap = a.seg[i].list.cap * a.seg[i].rpu;
        const int groups = (rows_cap + G - 1) / G;
        int blocks = (groups + NT - 1) / NT;
        if (blocks > max_blocks) blocks = max_blocks;
        if (blocks < 1) blocks = 1;
        a.seg[i].blocks = blocks;
        total += blocks;
    }
    if (total <= 0) return hipSuccess;
    dim3 grid(total);
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
