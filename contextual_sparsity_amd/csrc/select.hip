// Selection kernels: one block per row (bitmaps ORed by a second kernel when there are
// several rows), two selections per launch.  The block-level algorithm is in select.hpp.
#include "select.hpp"

namespace djv {
namespace {

using namespace sel;

struct SelectJobs {
    SelectJob j[2];
};

__global__ __launch_bounds__(kThreads) void select_rows_kernel(SelectJobs jobs, int B) {
    __shared__ RowShared S;
    const SelectJob& J = jobs.j[blockIdx.y];
    select_row_full(S, J, blockIdx.x);
    finish_row(S, J, blockIdx.x, B, (J.n_out + 31) / 32);
}

// Rows of at most kShortRows scores: one block per selection over all B rows (small B), or
// one block per row writing the row's bitmap for compact_kernel (larger B).  Rank counting
// is n^2 comparisons on one compute unit (about 40 us at n = 1024), so longer rows take the
// candidate radix path of select_rows_kernel (about 8 us at n = 1024).
__global__ __launch_bounds__(kThreads) void select_small_kernel(SelectJobs jobs, int B) {
    __shared__ SmallShared<kThreads> S;
    select_small_block<kThreads>(S, jobs.j[blockIdx.x], B);
}
__global__ __launch_bounds__(kThreads) void select_small_rows_kernel(SelectJobs jobs) {
    __shared__ SmallShared<kThreads> S;
    select_small_row_bits<kThreads>(S, jobs.j[blockIdx.y], blockIdx.x);
}
constexpr int kSmallRowsFrom = 4;  // batches from which the per-row form is used

__global__ __launch_bounds__(kThreads) void compact_kernel(SelectJobs jobs, int B) {
    const SelectJob& J = jobs.j[blockIdx.x];
    const int tid = threadIdx.x;
    const int words = (J.n_out + 31) / 32;
    __shared__ int wtot[kThreads / kWave];
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    uint32_t m0 = 0u, m1 = 0u;
    // rows in groups of 8, their loads issued together
    for (int b0 = 0; b0 < B; b0 += 8) {
        uint32_t v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t* bits = J.bits + (size_t)min(b0 + k, B - 1) * words;
            v0[k] = w0 < words ? bits[w0] : 0u;
            v1[k] = w1 < words ? bits[w1] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            m0 |= v0[k];
            m1 |= v1[k];
        }
    }
    const int total = compact_words(m0, m1, J.idx, wtot, J.lo, J.hi);
    if (tid == 0) *J.count = total;
}

}  // namespace

hipError_t launch_select(const SelectJob* jobs, int njobs, int B, hipStream_t s, int prof) {
    if (njobs < 1 || njobs > 2 || B < 1) return hipErrorInvalidValue;
    SelectJobs js{};
    bool small = true;
    for (int i = 0; i < njobs; ++i) {
        js.j[i] = jobs[i];
        small = small && jobs[i].n_out <= kShortRows;
    }
    if (small && B < kSmallRowsFrom) {
        prof_begin(prof, s);
        hipLaunchKernelGGL(select_small_kernel, dim3(njobs), dim3(kThreads), 0, s, js, B);
        prof_end(prof, s);
        return hipGetLastError();
    }
    if (small) {
        prof_begin(prof, s);
        hipLaunchKernelGGL(select_small_rows_kernel, dim3(B, njobs), dim3(kThreads), 0, s, js);
        prof_end(prof, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(compact_kernel, dim3(njobs), dim3(kThreads), 0, s, js, B);
        return hipGetLastError();
    }
    prof_begin(prof, s);
    hipLaunchKernelGGL(select_rows_kernel, dim3(B, njobs), dim3(kThreads), 0, s, js, B);
    prof_end(prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 1) return e;
    hipLaunchKernelGGL(compact_kernel, dim3(njobs), dim3(kThreads), 0, s, js, B);
    return hipGetLastError();
}

}  // namespace djv
