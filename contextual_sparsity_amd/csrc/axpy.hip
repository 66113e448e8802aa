// Row-axpy: out[b] = resid[b] + sum over visited rows r of coef[b, r] * W[row(r), :].
//
// Serves the two "down" products of the layer, both of which consume whole weight rows
// selected by a unit list:
//   * MLP down-projection: rows W2[j] of the kept neurons, coefficients a_j
//     ([NOTES "Sparsified MLP"]: (W^2_{S_M})^T applied to the kept activations);
//   * attention output projection: rows of W_i^O of the kept heads, coefficients H_i[c]
//     ([NOTES "Sparsified Attention"]: sum over kept heads of H_i(y) W_i^O).
// The kept rows are read in place ([BLOG section 3.2]: gather fused with the product).
//
// Decomposition: a block owns a column tile of 64 lanes x one 16-byte vector (512 fp16
// or 256 fp32 columns) and a chunk of consecutive visited rows; its four waves split the
// chunk's rows and combine in LDS, giving one partial tile per (chunk, tile).  A second
// kernel adds the partial tiles in chunk order plus the residual, so the result does not
// depend on scheduling (no atomics).
#include "common.hpp"

namespace djv {
namespace {

constexpr int kUnroll = 8;      // rows in flight per wave
constexpr int kWavesPerBlock = 4;

template <typename T, int NB>
__global__ __launch_bounds__(256) void axpy_partial_kernel(AxpyArgs a) {
    constexpr int E = WTraits<T>::kPerVec;
    __shared__ float red[kWavesPerBlock - 1][NB][kWave * E];

    const int tid = threadIdx.x, wv = tid / kWave, ln = tid % kWave;
    const int nvec = a.cols / E;
    const int v = blockIdx.x * kWave + ln;  // this lane's column vector
    const bool col_ok = v < nvec;
    const int count = read_count(a.list, a.flags);
    const int rows = count * a.rpu;
    const int r0 = blockIdx.y * a.rows_per_chunk;
    if (r0 >= rows) return;
    const int r1 = min(rows, r0 + a.rows_per_chunk);
    const char* Wb = reinterpret_cast<const char*>(a.W);
    const size_t row_bytes = (size_t)a.cols * sizeof(T);

    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;

    for (int rb = r0 + wv; rb < r1; rb += kWavesPerBlock * kUnroll) {
        Vec16 w[kUnroll];
        float cf[kUnroll][NB];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            const int r = rb + q * kWavesPerBlock;
            long long row = -1;
            if (r < r1) {
                const int u = r / a.rpu, sub = r - u * a.rpu;
                const int unit = unit_of(a.list, u, a.flags);
                if (unit >= 0) row = (long long)unit * a.rpu + sub;
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                cf[q][b] = (row >= 0 && b < a.B) ? a.coef[(size_t)b * a.ldc + r] : 0.f;
            if (row >= 0 && col_ok)
                w[q] = ldg16_nt(Wb + (size_t)row * row_bytes + (size_t)v * 16);
            else
                w[q] = Vec16{{0u, 0u, 0u, 0u}};
        }
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            float f[E];
            unpack<T>(w[q], f);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[b][e] = fmaf(cf[q][b], f[e], acc[b][e]);
        }
    }

    if (wv > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < E; ++e) red[wv - 1][b][ln * E + e] = acc[b][e];
    }
    __syncthreads();
    if (wv == 0 && col_ok) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b >= a.B) break;
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float s = acc[b][e];
#pragma unroll
                for (int q = 0; q < kWavesPerBlock - 1; ++q) s += red[q][b][ln * E + e];
                o[e] = s;
            }
            float* dst = a.partial + ((size_t)blockIdx.y * a.B + b) * a.cols + (size_t)v * E;
#pragma unroll
            for (int e = 0; e < E; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
        }
    }
}

// out = resid + sum of the used partial tiles, in chunk order.
__global__ __launch_bounds__(256) void axpy_finalize_kernel(AxpyArgs a) {
    const int count = read_count(a.list, nullptr);
    const int rows = count * a.rpu;
    const int nch = (rows + a.rows_per_chunk - 1) / a.rows_per_chunk;
    const size_t total4 = (size_t)a.B * a.cols / 4;
    const size_t plane = (size_t)a.B * a.cols;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total4;
         i += (size_t)gridDim.x * blockDim.x) {
        float4 s = a.resid ? reinterpret_cast<const float4*>(a.resid)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int c = 0; c < nch; ++c) {
            const float4 p = reinterpret_cast<const float4*>(a.partial + c * plane)[i];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        reinterpret_cast<float4*>(a.out)[i] = s;
    }
}

template <typename T>
hipError_t dispatch(const AxpyArgs& a, hipStream_t s) {
    constexpr int E = WTraits<T>::kPerVec;
    const int nvec = a.cols / E;
    const int tiles = (nvec + kWave - 1) / kWave;
    const int rows_cap = a.list.cap * a.rpu;
    const int nch = rows_cap > 0 ? (rows_cap + a.rows_per_chunk - 1) / a.rows_per_chunk : 0;
    if (nch > 0) {
        dim3 grid(tiles, nch);
        prof_begin(a.prof, s);
        if (a.B <= 1) hipLaunchKernelGGL((axpy_partial_kernel<T, 1>), grid, dim3(256), 0, s, a);
        else if (a.B <= 2) hipLaunchKernelGGL((axpy_partial_kernel<T, 2>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((axpy_partial_kernel<T, 4>), grid, dim3(256), 0, s, a);
        prof_end(a.prof, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t total4 = (size_t)a.B * a.cols / 4;
    int blocks = (int)((total4 + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(axpy_finalize_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int axpy_chunks(int rows_cap, int cols, bool f16, int* rows_per_chunk) {
    const int E = f16 ? 8 : 4;
    const int tiles = (cols / E + kWave - 1) / kWave;
    const int step = kWavesPerBlock * kUnroll;  // 32 rows: one pass of the block
    if (rows_cap <= 0) {
        *rows_per_chunk = step;
        return 0;
    }
    int chunks = (1024 + tiles - 1) / tiles;
    const int max_chunks = (rows_cap + step - 1) / step;
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks < 1) chunks = 1;
    int rpc = (rows_cap + chunks - 1) / chunks;
    rpc = ((rpc + step - 1) / step) * step;
    *rows_per_chunk = rpc;
    return (rows_cap + rpc - 1) / rpc;
}

hipError_t launch_axpy(bool f16, const AxpyArgs& a, hipStream_t s) {
    return f16 ? dispatch<__half>(a, s) : dispatch<float>(a, s);
}

}  // namespace djv
