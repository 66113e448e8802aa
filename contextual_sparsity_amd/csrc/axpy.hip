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
// Kernel 1 (partial): a block owns a column tile of 64 lanes x one 16-byte vector (512
// fp16 or 256 fp32 columns) and a chunk of consecutive visited rows.  It stages the
// chunk's row numbers and coefficients in LDS (one round trip for the whole chunk), then
// its four waves stream their rows with kUnroll independent 16-byte loads in flight per
// lane, combine in LDS and write one partial tile.
// Kernel 2 (finalize): out = resid + the partial tiles summed in a fixed order, so the
// result does not depend on scheduling (no atomics); a thread issues its loads in
// batches before adding.  It also writes (mean, M2) of every 64-column slice of out, from
// which the next GEMV applies LayerNorm while loading.  The kernel boundary between the
// two is what makes the partial tiles of all XCDs visible; no device-wide fence is used.
#include "common.hpp"

namespace djv {
namespace {

constexpr int kUnroll = 8;      // rows in flight per wave
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 256;

template <typename T, int NB>
__global__ __launch_bounds__(kThreads) void axpy_partial_kernel(AxpyArgs a) {
    constexpr int E = WTraits<T>::kPerVec;
    constexpr int TC = kWave * E;                       // columns per tile
    extern __shared__ float dyn[];                      // [NB][rpc] coefs, then [rpc] rows
    __shared__ float red[kWavesPerBlock - 1][NB][TC];

    const int tid = threadIdx.x, wv = tid / kWave, ln = tid % kWave;
    const int chunk = blockIdx.y;
    const int nvec = a.cols / E;
    const int v = blockIdx.x * kWave + ln;              // this lane's column vector
    const bool col_ok = v < nvec;
    const int count = read_count(a.list, a.flags);
    const int rows = count * a.rpu;
    const int r0 = chunk * a.rows_per_chunk;
    if (r0 >= rows) return;
    const int nr = min(rows, r0 + a.rows_per_chunk) - r0;
    float* cf_s = dyn;
    int* row_s = reinterpret_cast<int*>(dyn + NB * a.rows_per_chunk);

    // stage row numbers and coefficients of the chunk
    for (int i = tid; i < nr; i += kThreads) {
        const int r = r0 + i;
        const int u = r / a.rpu, sub = r - u * a.rpu;
        const int unit = unit_of(a.list, u, a.flags);
        row_s[i] = unit < 0 ? -1 : unit * a.rpu + sub;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            cf_s[b * a.rows_per_chunk + i] = (unit >= 0 && b < a.B) ? a.coef[(size_t)b * a.ldc + r] : 0.f;
    }
    __syncthreads();

    const char* Wb = reinterpret_cast<const char*>(a.W);
    const size_t row_bytes = (size_t)a.cols * sizeof(T);
    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;

    for (int i0 = wv; i0 < nr; i0 += kWavesPerBlock * kUnroll) {
        Vec16 w[kUnroll];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            const int i = i0 + q * kWavesPerBlock;
            const int row = i < nr ? row_s[i] : -1;
            if (row >= 0 && col_ok)
                w[q] = ldg16_nt(Wb + (size_t)row * row_bytes + (size_t)v * 16);
            else
                w[q] = Vec16{{0u, 0u, 0u, 0u}};
        }
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            const int i = i0 + q * kWavesPerBlock;
            if (i >= nr) break;
            float f[E];
            unpack<T>(w[q], f);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float c = cf_s[b * a.rows_per_chunk + i];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[b][e] = fmaf(c, f[e], acc[b][e]);
            }
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
            float* dst = a.partial + ((size_t)chunk * a.B + b) * a.cols + (size_t)v * E;
#pragma unroll
            for (int e = 0; e < E; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
        }
    }
}

// out = resid + sum of the used partial tiles in a fixed order, per 64-column slice, and
// the slice's (mean, M2).  Block (slice, b): four groups of 64 threads split the chunks
// (group g adds chunks g, g+4, ...), then wave 0 adds the four group sums in order.
constexpr int kFinGroups = 4;
constexpr int kFinUnroll = 4;

__global__ __launch_bounds__(kWave * kFinGroups) void axpy_finalize_kernel(AxpyArgs a) {
    __shared__ float red[kFinGroups - 1][kWave];
    const int slice = blockIdx.x, b = blockIdx.y;
    const int g = threadIdx.x / kWave, c = threadIdx.x % kWave;
    const int col = slice * kWave + c;
    const bool ok = col < a.cols;
    const int count = read_count(a.list, nullptr);
    const int rows = count * a.rpu;
    const int nch = (rows + a.rows_per_chunk - 1) / a.rows_per_chunk;
    const size_t plane = (size_t)a.B * a.cols;
    const float* p = a.partial + (size_t)b * a.cols + (ok ? col : 0);
    float s = 0.f;
    for (int ch = g; ch < nch; ch += kFinGroups * kFinUnroll) {
        float t[kFinUnroll];
#pragma unroll
        for (int k = 0; k < kFinUnroll; ++k) {
            const int cc = ch + k * kFinGroups;
            t[k] = (ok && cc < nch) ? p[(size_t)cc * plane] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kFinUnroll; ++k) s += t[k];
    }
    if (g > 0) red[g - 1][c] = s;
    __syncthreads();
    if (g != 0) return;
#pragma unroll
    for (int q = 0; q < kFinGroups - 1; ++q) s += red[q][c];
    const size_t o = (size_t)b * a.cols + col;
    if (ok && a.resid) s += a.resid[o];
    if (ok) a.out[o] = s;
    if (a.stats) {
        const int n = min(kWave, a.cols - slice * kWave);
        const float mean = wave_sum(ok ? s : 0.f) / (float)n;
        const float dv = ok ? s - mean : 0.f;
        const float M2 = wave_sum(dv * dv);
        if (c == 0) a.stats[(size_t)b * gridDim.x + slice] = make_float2(mean, M2);
    }
}

template <typename T>
hipError_t dispatch(const AxpyArgs& a, hipStream_t s) {
    constexpr int E = WTraits<T>::kPerVec;
    const int tiles = (a.cols / E + kWave - 1) / kWave;
    const int rows_cap = a.list.cap * a.rpu;
    const int nch = rows_cap > 0 ? (rows_cap + a.rows_per_chunk - 1) / a.rows_per_chunk : 0;
    if (nch > 0) {
        const int nb = a.B <= 1 ? 1 : (a.B <= 2 ? 2 : 4);
        const size_t dyn = (size_t)a.rows_per_chunk * (nb * sizeof(float) + sizeof(int));
        dim3 grid(tiles, nch);
        prof_begin(a.prof, s);
        if (nb == 1) hipLaunchKernelGGL((axpy_partial_kernel<T, 1>), grid, dim3(kThreads), dyn, s, a);
        else if (nb == 2) hipLaunchKernelGGL((axpy_partial_kernel<T, 2>), grid, dim3(kThreads), dyn, s, a);
        else hipLaunchKernelGGL((axpy_partial_kernel<T, 4>), grid, dim3(kThreads), dyn, s, a);
        prof_end(a.prof, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 fgrid((a.cols + kWave - 1) / kWave, a.B);
    hipLaunchKernelGGL(axpy_finalize_kernel, fgrid, dim3(kWave * kFinGroups), 0, s, a);
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
    const int min_chunks = (rows_cap + kAxpyMaxChunkRows - 1) / kAxpyMaxChunkRows;
    if (chunks < min_chunks) chunks = min_chunks;
    if (chunks < 1) chunks = 1;
    int rpc = (rows_cap + chunks - 1) / chunks;
    rpc = ((rpc + step - 1) / step) * step;
    if (rpc > kAxpyMaxChunkRows) rpc = kAxpyMaxChunkRows;
    *rows_per_chunk = rpc;
    return (rows_cap + rpc - 1) / rpc;
}

hipError_t launch_axpy(bool f16, const AxpyArgs& a, hipStream_t s) {
    return f16 ? dispatch<__half>(a, s) : dispatch<float>(a, s);
}

}  // namespace djv
