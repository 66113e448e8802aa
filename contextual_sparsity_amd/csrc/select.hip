// Selection of kept units from predictor scores, with ties resolved by index.
//
// [BLOG section 2]: each predictor output is a select / skip decision made by a sigmoid;
// [BLOG section 1]: the best-scoring ~20% of heads and ~5% of neurons are kept.  Sigmoid
// is monotone, so both rules work on the fp32 scores directly:
//   top-k:     the k best under (score descending, index ascending);
//   threshold: score > tau with tau = fp32(logit t).
// -0 counts as +0 and NaN as -inf, so every result is a unique function of the score
// bits.  A batch computes with the union of its rows' sets, listed in ascending order.
//
// Scores are mapped to order-preserving uint32 keys; the k-th largest key is found by a
// four-pass 8-bit radix select in one 1024-thread block per row (histograms in LDS),
// then the keys equal to it are taken in index order with a block-wide prefix count.
// Each row writes a bitmap; a second kernel ORs the rows' bitmaps and compacts the set
// bits into an ascending index list and a device-side count.  Integer work only.
#include "common.hpp"

namespace djv {
namespace {

constexpr int kThreads = 1024;
constexpr int kKeysPerThread = 64;                 // n_out <= 65536
constexpr int kMaxWords = kThreads * 2;            // 65536 bits

struct SelectJobs {
    SelectJob j[2];
};

__device__ __forceinline__ uint32_t score_key(float z) {
    uint32_t u = __float_as_uint(z);
    if (z != z) u = 0xFF800000u;                    // NaN ranks as -inf
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;            // -0 equals +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block; also returns the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wtot, int* total) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wtot[w] = x;
    __syncthreads();
    int base = 0, tot = 0;
    for (int q = 0; q < kThreads / kWave; ++q) {
        const int t = wtot[q];
        if (q < w) base += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

__global__ __launch_bounds__(kThreads) void select_rows_kernel(SelectJobs jobs) {
    const SelectJob& J = jobs.j[blockIdx.y];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int n = J.n_out, words = (n + 31) / 32;
    __shared__ uint32_t hist[256];
    __shared__ uint32_t selw[kMaxWords];
    __shared__ uint32_t tiew[kMaxWords];
    __shared__ int sh[2];
    __shared__ int wtot[kThreads / kWave];
    const float* z = J.z + (size_t)b * n;

    for (int w = tid; w < words; w += kThreads) {
        selw[w] = 0u;
        tiew[w] = 0u;
    }
    __syncthreads();

    if (J.mode == 1) {
        for (int j = tid; j < n; j += kThreads)
            if (score_key(z[j]) > J.tau_key) atomicOr(&selw[j >> 5], 1u << (j & 31));
    } else if (J.k >= n) {
        for (int j = tid; j < n; j += kThreads) atomicOr(&selw[j >> 5], 1u << (j & 31));
    } else if (J.k > 0) {
        uint32_t key[kKeysPerThread];
#pragma unroll
        for (int i = 0; i < kKeysPerThread; ++i) {
            const int j = tid + kThreads * i;
            key[i] = j < n ? score_key(z[j]) : 0u;
        }
        uint32_t prefix = 0u, pmask = 0u;
        int rem = J.k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kKeysPerThread; ++i) {
                const int j = tid + kThreads * i;
                if (j < n && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < kWave) {
                // lane L holds digits 255-4L .. 252-4L (descending digit order across lanes)
                int c[4], s = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    c[q] = (int)hist[255 - 4 * tid - q];
                    s += c[q];
                }
                int x = s;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const int y = __shfl_up(x, o, kWave);
                    if (tid >= o) x += y;
                }
                int cum = x - s;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (cum < rem && rem <= cum + c[q]) {
                        sh[0] = 255 - 4 * tid - q;
                        sh[1] = rem - cum;
                    }
                    cum += c[q];
                }
            }
            __syncthreads();
            prefix |= (uint32_t)sh[0] << shift;
            pmask |= 0xFFu << shift;
            rem = sh[1];
            __syncthreads();
        }
        // prefix is now the k-th largest key; rem keys equal to it are still to take
#pragma unroll
        for (int i = 0; i < kKeysPerThread; ++i) {
            const int j = tid + kThreads * i;
            if (j < n) {
                if (key[i] > prefix) atomicOr(&selw[j >> 5], 1u << (j & 31));
                else if (key[i] == prefix) atomicOr(&tiew[j >> 5], 1u << (j & 31));
            }
        }
        __syncthreads();
        const int w0 = 2 * tid, w1 = 2 * tid + 1;
        uint32_t t0 = w0 < words ? tiew[w0] : 0u, t1 = w1 < words ? tiew[w1] : 0u;
        int total;
        const int base = block_exclusive_scan(__popc(t0) + __popc(t1), wtot, &total);
        int take = rem - base;
        uint32_t add0 = 0u, add1 = 0u;
        while (take > 0 && t0) {
            const uint32_t low = t0 & (~t0 + 1u);
            add0 |= low;
            t0 ^= low;
            --take;
        }
        while (take > 0 && t1) {
            const uint32_t low = t1 & (~t1 + 1u);
            add1 |= low;
            t1 ^= low;
            --take;
        }
        if (w0 < words) selw[w0] |= add0;
        if (w1 < words) selw[w1] |= add1;
    }
    __syncthreads();
    uint32_t* out = J.bits + (size_t)b * words;
    for (int w = tid; w < words; w += kThreads) out[w] = selw[w];
}

__global__ __launch_bounds__(kThreads) void compact_kernel(SelectJobs jobs, int B) {
    const SelectJob& J = jobs.j[blockIdx.x];
    const int tid = threadIdx.x;
    const int words = (J.n_out + 31) / 32;
    __shared__ int wtot[kThreads / kWave];
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    uint32_t m0 = 0u, m1 = 0u;
    for (int b = 0; b < B; ++b) {
        const uint32_t* bits = J.bits + (size_t)b * words;
        if (w0 < words) m0 |= bits[w0];
        if (w1 < words) m1 |= bits[w1];
    }
    int total;
    int pos = block_exclusive_scan(__popc(m0) + __popc(m1), wtot, &total);
    while (m0) {
        const int bit = __ffs(m0) - 1;
        J.idx[pos++] = w0 * 32 + bit;
        m0 &= m0 - 1u;
    }
    while (m1) {
        const int bit = __ffs(m1) - 1;
        J.idx[pos++] = w1 * 32 + bit;
        m1 &= m1 - 1u;
    }
    if (tid == 0) *J.count = total;
}

}  // namespace

hipError_t launch_select(const SelectJob* jobs, int njobs, int B, hipStream_t s, int prof) {
    if (njobs < 1 || njobs > 2 || B < 1) return hipErrorInvalidValue;
    SelectJobs js{};
    for (int i = 0; i < njobs; ++i) js.j[i] = jobs[i];
    prof_begin(prof, s);
    hipLaunchKernelGGL(select_rows_kernel, dim3(B, njobs), dim3(kThreads), 0, s, js);
    prof_end(prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(compact_kernel, dim3(njobs), dim3(kThreads), 0, s, js, B);
    return hipGetLastError();
}

}  // namespace djv
