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
// Scores become order-preserving uint32 keys.  The k-th largest key is found by a radix
// select on digits of 12, 10 and 10 bits (the wide first digit spreads the sign and
// exponent bits, where predictor scores crowd, over many bins); keys above it are kept,
// and keys equal to it are taken in index order with a block-wide prefix count.
//
// One 1024-thread block per row reads its keys in rounds of 32 per thread (all loads of a
// round in flight together), histograms the first digit, marks the keys above the k-th
// key's first digit and gathers the few keys sharing it into LDS, where the last two
// digits are resolved.  With one row the block compacts the result into the ascending
// index list and the device-side count; with several rows each row writes a bitmap and a
// second kernel ORs and compacts them.  Two selections (the head and the neuron predictor)
// run in one launch.  Bitmaps are built from wave ballots: lanes of a wave hold
// consecutive indices, so a ballot is exactly two bitmap words and no shared word is
// updated atomically.
#include "common.hpp"

namespace djv {
namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 32;                         // keys per thread held in registers at once
constexpr int kMaxWords = kThreads * 2;            // 65536 bits
constexpr int kMaxBins = 4096;                     // first digit: the top 12 bits of a key
constexpr int kMaxCand = 2048;                     // candidates refined in LDS

struct SelectJobs {
    SelectJob j[2];
};

// Exclusive prefix sum over a block of NT threads; also returns the block total.
template <int NT>
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
#pragma unroll
    for (int q = 0; q < NT / kWave; ++q) {
        const int t = wtot[q];
        if (q < w) base += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// The digit of the rem-th largest key among histogrammed keys.  Thread t owns the PER
// bins nbins-1-PER*t .. nbins-PER*t, so thread order is descending digit order.  rem
// (in: rank among the keys, out: rank inside the returned bin) is updated in every thread.
template <int NT, int PER>
__device__ __forceinline__ int find_bin_counts(const int (&c)[PER], int nbins, int& rem, int* wtot,
                                               int* sh) {
    const int tid = threadIdx.x;
    int s = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) s += c[q];
    int total;
    int cum = block_exclusive_scan<NT>(s, wtot, &total);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (cum < rem && rem <= cum + c[q]) {
            sh[0] = nbins - 1 - PER * tid - q;
            sh[1] = rem - cum;
        }
        cum += c[q];
    }
    __syncthreads();
    const int d = sh[0];
    rem = sh[1];
    __syncthreads();
    return d;
}

template <int NT, int PER>
__device__ __forceinline__ int find_bin(const uint32_t* hist, int nbins, int& rem, int* wtot, int* sh) {
    int c[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int bin = nbins - 1 - PER * (int)threadIdx.x - q;
        c[q] = bin >= 0 ? (int)hist[bin] : 0;
    }
    return find_bin_counts<NT, PER>(c, nbins, rem, wtot, sh);
}

// Lanes of a wave hold 64 consecutive indices starting at index j0 (a multiple of 64):
// one ballot is the two bitmap words j0/32 and j0/32 + 1.
__device__ __forceinline__ void ballot_words(uint32_t* words, int nwords, int j0, bool pred) {
    const unsigned long long m = __ballot(pred);
    const int w0 = j0 >> 5;
    if ((threadIdx.x % kWave) == 0) {
        if (w0 < nwords) words[w0] = (uint32_t)m;
        if (w0 + 1 < nwords) words[w0 + 1] = (uint32_t)(m >> 32);
    }
}

// Writes the set bits of words 2t, 2t+1 (t = thread) as ascending indices; returns the
// total count.
__device__ __forceinline__ int compact_words(uint32_t m0, uint32_t m1, int32_t* idx, int* wtot) {
    const int w0 = 2 * threadIdx.x, w1 = w0 + 1;
    int total;
    int pos = block_exclusive_scan<kThreads>(__popc(m0) + __popc(m1), wtot, &total);
    while (m0) {
        idx[pos++] = w0 * 32 + (__ffs(m0) - 1);
        m0 &= m0 - 1u;
    }
    while (m1) {
        idx[pos++] = w1 * 32 + (__ffs(m1) - 1);
        m1 &= m1 - 1u;
    }
    return total;
}

// Shared LDS of the 1024-thread row kernels.
struct RowShared {
    uint32_t hist[kMaxBins + kWave];
    uint32_t selw[kMaxWords];
    uint32_t tiew[kMaxWords];
    uint32_t cand[kMaxCand];
    int cand_j[kMaxCand];
    int sh[3];
    int wtot[kThreads / kWave];
};

// Resolves the last two digits over candidate keys in LDS (prefix/pmask: digits so far)
// and marks the candidates above the k-th key in selw and equal to it in tiew.
__device__ __forceinline__ void resolve_candidates(RowShared& S, int ncand, uint32_t& prefix,
                                                   uint32_t& pmask, int& rem) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 10 : 0;
        for (int i = tid; i < 1024; i += kThreads) S.hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < ncand; i += kThreads)
            if ((S.cand[i] & pmask) == prefix) atomicAdd(&S.hist[(S.cand[i] >> shift) & 1023u], 1u);
        __syncthreads();
        prefix |= (uint32_t)find_bin<kThreads, 4>(S.hist, 1024, rem, S.wtot, S.sh) << shift;
        pmask |= 1023u << shift;
    }
    for (int i = tid; i < ncand; i += kThreads) {
        const int j = S.cand_j[i];
        if (S.cand[i] > prefix) atomicOr(&S.selw[j >> 5], 1u << (j & 31));
        else if (S.cand[i] == prefix) atomicOr(&S.tiew[j >> 5], 1u << (j & 31));
    }
}

// Adds to selw the first `rem` indices (ascending) of the tie bitmap.
__device__ __forceinline__ void take_ties(RowShared& S, int words, int rem) {
    const int tid = threadIdx.x;
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    uint32_t t0 = w0 < words ? S.tiew[w0] : 0u, t1 = w1 < words ? S.tiew[w1] : 0u;
    int total;
    const int base = block_exclusive_scan<kThreads>(__popc(t0) + __popc(t1), S.wtot, &total);
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
    if (w0 < words) S.selw[w0] |= add0;
    if (w1 < words) S.selw[w1] |= add1;
}

// Emits the row's final bitmap: compacted into idx/count when B == 1, else written to
// the row's bitmap for the union kernel.
__device__ __forceinline__ void finish_row(RowShared& S, const SelectJob& J, int b, int B, int words) {
    const int tid = threadIdx.x;
    __syncthreads();
    if (B == 1) {
        const int w0 = 2 * tid, w1 = 2 * tid + 1;
        const int total = compact_words(w0 < words ? S.selw[w0] : 0u, w1 < words ? S.selw[w1] : 0u,
                                        J.idx, S.wtot);
        if (tid == 0) *J.count = total;
        return;
    }
    uint32_t* out = J.bits + (size_t)b * words;
    for (int w = tid; w < words; w += kThreads) out[w] = S.selw[w];
}

// The whole selection of row b in one block (keys from z).
__device__ __forceinline__ void select_row_full(RowShared& S, const SelectJob& J, int b) {
    const int tid = threadIdx.x, lane = tid % kWave;
    const int n = J.n_out, words = (n + 31) / 32;
    const float* z = J.z + (size_t)b * n;
    const int slots = (n + kThreads - 1) / kThreads;   // key slots in use (uniform)
    const int rounds = (slots + kChunk - 1) / kChunk;
    const int wbase = (tid / kWave) * kWave;            // first index of this wave in a slot

    // keys of slots [rr*kChunk, rr*kChunk + kChunk) of this thread (index tid + 1024 * slot),
    // all requested at once; a slot past n reads the last score and becomes key 0, below
    // every real key (-inf and NaN map to 0x007FFFFF)
    auto load_keys = [&](uint32_t (&kk)[kChunk], int rr) {
        float v[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) v[c] = z[min(tid + kThreads * (rr * kChunk + c), n - 1)];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int j = tid + kThreads * (rr * kChunk + c);
            kk[c] = score_key(v[c]) & (0u - (uint32_t)(j < n));
        }
    };

    for (int w = tid; w < words; w += kThreads) {
        S.selw[w] = 0u;
        S.tiew[w] = 0u;
    }
    __syncthreads();

    if (J.mode == 1) {
        for (int rr = 0; rr < rounds; ++rr) {
            uint32_t kk[kChunk];
            load_keys(kk, rr);
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int i = rr * kChunk + c;
                if (i >= slots) break;
                ballot_words(S.selw, words, kThreads * i + wbase, tid + kThreads * i < n && kk[c] > J.tau_key);
            }
        }
    } else if (J.k >= n) {
        for (int i = 0; i < slots; ++i) ballot_words(S.selw, words, kThreads * i + wbase, tid + kThreads * i < n);
    } else if (J.k > 0) {
        // first digit: histogram of the top 12 bits of the real keys (slots past n go to one
        // of 64 spare bins, one per lane, so they neither count nor collide)
        for (int i = tid; i < kMaxBins + kWave; i += kThreads) S.hist[i] = 0u;
        __syncthreads();
        for (int rr = 0; rr < rounds; ++rr) {
            uint32_t kk[kChunk];
            load_keys(kk, rr);
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int i = rr * kChunk + c;
                if (i >= slots) break;
                const bool ok = tid + kThreads * i < n;
                atomicAdd(&S.hist[ok ? (kk[c] >> 20) : (uint32_t)(kMaxBins + lane)], 1u);
            }
        }
        __syncthreads();
        int rem = J.k;
        const uint32_t top = (uint32_t)find_bin<kThreads, 4>(S.hist, kMaxBins, rem, S.wtot, S.sh);
        uint32_t prefix = top << 20, pmask = 0xFFF00000u;
        const int ncand = (int)S.hist[top];
        __syncthreads();  // every thread has read ncand before either branch rewrites hist
        if (ncand <= kMaxCand) {
            // keys above the first digit are kept now; the few sharing it are gathered (key
            // and index; one LDS atomic per wave and slot) and finished alone
            if (tid == 0) S.sh[2] = 0;
            __syncthreads();
            for (int rr = 0; rr < rounds; ++rr) {
                uint32_t kk[kChunk];
                load_keys(kk, rr);
#pragma unroll
                for (int c = 0; c < kChunk; ++c) {
                    const int i = rr * kChunk + c;
                    if (i >= slots) break;
                    const int j = tid + kThreads * i;
                    const bool ok = j < n;
                    ballot_words(S.selw, words, kThreads * i + wbase, ok && (kk[c] >> 20) > top);
                    const bool pred = ok && (kk[c] >> 20) == top;
                    const unsigned long long m = __ballot(pred);
                    if (m) {
                        int base = 0;
                        if (lane == 0) base = atomicAdd(&S.sh[2], __popcll(m));
                        base = __shfl(base, 0, kWave);
                        if (pred) {
                            const int at = base + __popcll(m & ((1ull << lane) - 1ull));
                            S.cand[at] = kk[c];
                            S.cand_j[at] = j;
                        }
                    }
                }
            }
            __syncthreads();
            resolve_candidates(S, ncand, prefix, pmask, rem);
        } else {
            // many equal top bits (heavy ties): refine over all keys, then mark
#pragma unroll
            for (int pass = 1; pass < 3; ++pass) {
                const int shift = pass == 1 ? 10 : 0;
                for (int i = tid; i < 1024; i += kThreads) S.hist[i] = 0u;
                __syncthreads();
                for (int rr = 0; rr < rounds; ++rr) {
                    uint32_t kk[kChunk];
                    load_keys(kk, rr);
#pragma unroll
                    for (int c = 0; c < kChunk; ++c) {
                        const int i = rr * kChunk + c;
                        if (i >= slots) break;
                        if (tid + kThreads * i < n && (kk[c] & pmask) == prefix)
                            atomicAdd(&S.hist[(kk[c] >> shift) & 1023u], 1u);
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)find_bin<kThreads, 4>(S.hist, 1024, rem, S.wtot, S.sh) << shift;
                pmask |= 1023u << shift;
            }
            for (int rr = 0; rr < rounds; ++rr) {
                uint32_t kk[kChunk];
                load_keys(kk, rr);
#pragma unroll
                for (int c = 0; c < kChunk; ++c) {
                    const int i = rr * kChunk + c;
                    if (i >= slots) break;
                    const bool ok = tid + kThreads * i < n;
                    ballot_words(S.selw, words, kThreads * i + wbase, ok && kk[c] > prefix);
                    ballot_words(S.tiew, words, kThreads * i + wbase, ok && kk[c] == prefix);
                }
            }
        }
        // prefix is now the k-th largest key; rem keys equal to it are still to take
        __syncthreads();
        take_ties(S, words, rem);
    }
}

__global__ __launch_bounds__(kThreads) void select_rows_kernel(SelectJobs jobs, int B) {
    __shared__ RowShared S;
    const SelectJob& J = jobs.j[blockIdx.y];
    select_row_full(S, J, blockIdx.x);
    finish_row(S, J, blockIdx.x, B, (J.n_out + 31) / 32);
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
    const int total = compact_words(m0, m1, J.idx, wtot);
    if (tid == 0) *J.count = total;
}

}  // namespace

hipError_t launch_select(const SelectJob* jobs, int njobs, int B, hipStream_t s, int prof) {
    if (njobs < 1 || njobs > 2 || B < 1) return hipErrorInvalidValue;
    SelectJobs js{};
    for (int i = 0; i < njobs; ++i) js.j[i] = jobs[i];
    prof_begin(prof, s);
    hipLaunchKernelGGL(select_rows_kernel, dim3(B, njobs), dim3(kThreads), 0, s, js, B);
    prof_end(prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 1) return e;
    hipLaunchKernelGGL(compact_kernel, dim3(njobs), dim3(kThreads), 0, s, js, B);
    return hipGetLastError();
}

}  // namespace djv
