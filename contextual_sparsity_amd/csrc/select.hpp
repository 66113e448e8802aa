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
// Scores become order-preserving uint32 keys.  One 1024-thread block per row holds all
// of the row's keys in registers (one round of loads; n <= 49152).  For top-k the k-th
// largest key is bracketed from a sample: 2048 scores spread evenly over the row are
// histogrammed on their top 12 bits, and the bins holding the sample ranks k*2048/n -+ 4
// standard deviations give a digit range [b_lo, b_hi].  Exact counts over all keys then
// check the bracket (fewer than k keys above b_hi, at least k at or above b_lo, and at
// most 4096 inside); keys above are kept (wave ballots: lanes of a wave hold consecutive
// indices, so a ballot is exactly two bitmap words), keys inside are gathered into LDS at
// offsets from a block prefix count, and a radix select over their digits (12, 10, 10
// bits) finds the k-th key; keys equal to it are taken in index order.  The bracket only
// decides how much work is done, never the result: when the check fails (a sample far
// off, or heavy ties), and for rows above 49152, the row falls back to a radix select
// over all keys, reloading them per pass.  Rows of 4097 to 16384 scores skip the sample:
// every key's top 12 bits go into an exact histogram (16 LDS atomics per thread), which
// gives the first digit of the k-th key at once; the keys sharing that digit are gathered
// with their full keys from registers, and two radix passes finish (select_row_hist; one
// search, no bracket check, no re-read of the candidates, one radix pass fewer).  Threshold
// rows are ballots of key > tau.
// Every search for the bin holding a rank is done by one wave over the threads' bin sums
// (find_bin).  With one row the block compacts the result into the ascending index list
// and the device-side count; several rows are ORed (in LDS for a side block, or by a
// second kernel).  Rows of at most 256 scores (the head predictor) take a smaller path:
// one key per thread, ranks by counting (select_small_block).  A tensor-parallel shard lists
// only the kept units of its own range [lo, hi), rebased to its rows (j - lo): the
// selection itself is over all units, as every shard computes it alike.
//
// This header holds the block-level device code; it is used by the selection kernels
// and by GEMV launches that run a selection in a side block.
#pragma once
#include "common.hpp"

namespace djv {
namespace sel {

constexpr int kThreads = 1024;
constexpr int kChunk = 8;                          // keys per thread per round (radix path)
constexpr int kMaxWords = kThreads * 2;            // 65536 bits
constexpr int kMaxBins = 4096;                     // first digit: the top 12 bits of a key
constexpr int kMaxCand = 4096;                     // candidates refined in LDS
constexpr int kSample = 2048;                      // sample scores that bracket the k-th key

// Exclusive prefix sum over a block of NT threads; also returns the block total.  T is
// int, or uint32_t for sums of two packed 16-bit counts (modular, no carry between them
// while the low count's total stays below 2^16).
template <typename T> struct NoDeduce { using type = T; };
template <int NT, typename T = int>
__device__ __forceinline__ T block_exclusive_scan(typename NoDeduce<T>::type v, T* wtot, T* total) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    T x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const T y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wtot[w] = x;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < NT / kWave; ++q) {
        const T t = wtot[q];
        if (q < w) base += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// The digit of the rem-th largest key among histogrammed keys.  Thread t owns the PER
// bins nbins-1-PER*t .. nbins-PER*t, so thread order is descending digit order.  rem (in:
// rank among the keys, from 1; out: rank inside the returned bin) is updated in every
// thread.  The threads' bin sums go to LDS and one wave finds the bin: each lane sums 16
// threads' sums, a wave scan finds the lane where the rank falls, that lane walks its
// threads and then the found thread's bins.  Two block barriers in all (a block-wide scan
// takes four and a longer chain of LDS round trips).
template <int PER>
__device__ __forceinline__ int find_bin(const uint32_t* hist, int nbins, int& rem, int* part, int* sh) {
    constexpr int kPerLane = kThreads / kWave;  // thread sums per lane
    const int tid = threadIdx.x;
    int s = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int bin = nbins - 1 - PER * tid - q;
        s += bin >= 0 ? (int)hist[bin] : 0;
    }
    part[tid] = s;
    __syncthreads();
    if (tid < kWave) {
        const int l = tid;
        int v[kPerLane];
        const int4* p4 = reinterpret_cast<const int4*>(part + l * kPerLane);
#pragma unroll
        for (int i = 0; i < kPerLane / 4; ++i) {
            const int4 t = p4[i];
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
        int tot = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) tot += v[i];
        int inc = tot;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(inc, o, kWave);
            if (l >= o) inc += y;
        }
        const int exc = inc - tot;
        if (exc < rem && rem <= inc) {  // one lane (when rem is within the total)
            int cum = exc, t = -1, cum_t = 0;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) {
                if (t < 0 && rem <= cum + v[i]) {
                    t = l * kPerLane + i;
                    cum_t = cum;
                }
                cum += v[i];
            }
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int bin = nbins - 1 - PER * t - q;
                const int c = bin >= 0 ? (int)hist[bin] : 0;
                if (cum_t < rem && rem <= cum_t + c) {
                    sh[0] = bin;
                    sh[1] = rem - cum_t;
                }
                cum_t += c;
            }
        }
    }
    __syncthreads();
    const int d = sh[0];
    rem = sh[1];
    __syncthreads();  // every thread has read sh (and part) before either is written again
    return d;
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

// Bits of word w (indices 32w .. 32w+31) that lie in [lo, hi).
__device__ __forceinline__ uint32_t range_mask(int w, int lo, int hi) {
    const int a = lo - 32 * w, b = hi - 32 * w;  // the range inside the word: [a, b)
    const uint32_t below_b = b >= 32 ? ~0u : (b <= 0 ? 0u : (1u << b) - 1u);
    const uint32_t from_a = a <= 0 ? ~0u : (a >= 32 ? 0u : ~((1u << a) - 1u));
    return below_b & from_a;
}

// Writes the set bits of words 2t, 2t+1 (t = thread) that lie in [lo, hi) as ascending
// indices j - lo; returns the total count.
__device__ __forceinline__ int compact_words(uint32_t m0, uint32_t m1, int32_t* idx, int* wtot, int lo,
                                             int hi) {
    const int w0 = 2 * threadIdx.x, w1 = w0 + 1;
    m0 &= range_mask(w0, lo, hi);
    m1 &= range_mask(w1, lo, hi);
    int total;
    int pos = block_exclusive_scan<kThreads>(__popc(m0) + __popc(m1), wtot, &total);
    while (m0) {
        idx[pos++] = w0 * 32 + (__ffs(m0) - 1) - lo;
        m0 &= m0 - 1u;
    }
    while (m1) {
        idx[pos++] = w1 * 32 + (__ffs(m1) - 1) - lo;
        m1 &= m1 - 1u;
    }
    return total;
}

// Shared LDS of the 1024-thread row kernels.
struct RowShared {
    uint32_t hist[kMaxBins + kWave];
    uint32_t selw[kMaxWords];
    uint32_t tiew[kMaxWords];
    uint32_t uni[kMaxWords];              // union over rows (side-block selection)
    uint32_t cand[kMaxCand];
    int cand_j[kMaxCand];
    int sh[4];
    int wtot[kThreads / kWave];
    __align__(16) int part[kThreads];     // per-thread bin sums of find_bin
};

// Radix select over candidate keys in LDS, from digit `first` (0: the top 12 bits, 1 and
// 2: the next two 10-bit digits; prefix/pmask hold the digits already fixed): leaves in
// prefix the key of rank rem among the candidates and in rem its rank among the keys
// equal to it, and marks the candidates above it in selw and equal to it in tiew.
__device__ __forceinline__ void resolve_candidates(RowShared& S, int ncand, uint32_t& prefix,
                                                   uint32_t& pmask, int& rem, int first) {
    const int tid = threadIdx.x;
    for (int pass = first; pass < 3; ++pass) {  // uniform
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 0 ? kMaxBins : 1024;
        const uint32_t dmask = (uint32_t)nbins - 1u;
        for (int i = tid; i < nbins; i += kThreads) S.hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < ncand; i += kThreads)
            if ((S.cand[i] & pmask) == prefix) atomicAdd(&S.hist[(S.cand[i] >> shift) & dmask], 1u);
        __syncthreads();
        const uint32_t d = pass == 0 ? (uint32_t)find_bin<4>(S.hist, kMaxBins, rem, S.part, S.sh)
                                     : (uint32_t)find_bin<1>(S.hist, 1024, rem, S.part, S.sh);
        prefix |= d << shift;
        pmask |= dmask << shift;
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
                                        J.idx, S.wtot, J.lo, J.hi);
        if (tid == 0) *J.count = total;
        return;
    }
    uint32_t* out = J.bits + (size_t)b * words;
    for (int w = tid; w < words; w += kThreads) out[w] = S.selw[w];
}

// The whole selection of row b in one block by a radix select over all keys, reloaded
// from z per pass (the fallback of select_row_fast).
__device__ __forceinline__ void select_row_radix(RowShared& S, const SelectJob& J, int b) {
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
#pragma unroll 1
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
#pragma unroll 1
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
        const uint32_t top = (uint32_t)find_bin<4>(S.hist, kMaxBins, rem, S.part, S.sh);
        uint32_t prefix = top << 20, pmask = 0xFFF00000u;
        const int ncand = (int)S.hist[top];
        __syncthreads();  // every thread has read ncand before either branch rewrites hist
        if (ncand <= kMaxCand) {
            // keys above the first digit are kept now; the few sharing it are gathered (key
            // and index; one LDS atomic per wave and slot) and finished alone
            if (tid == 0) S.sh[2] = 0;
            __syncthreads();
    #pragma unroll 1
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
            resolve_candidates(S, ncand, prefix, pmask, rem, 1);
        } else {
            // many equal top bits (heavy ties): refine over all keys, then mark
#pragma unroll
            for (int pass = 1; pass < 3; ++pass) {
                const int shift = pass == 1 ? 10 : 0;
                for (int i = tid; i < 1024; i += kThreads) S.hist[i] = 0u;
                __syncthreads();
        #pragma unroll 1
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
                prefix |= (uint32_t)find_bin<4>(S.hist, 1024, rem, S.part, S.sh) << shift;
                pmask |= 1023u << shift;
            }
    #pragma unroll 1
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

// Score j of a row at a wave-uniform base.
__device__ __forceinline__ float load_score(gchar* zb, int j) {
    return *reinterpret_cast<const __attribute__((address_space(1))) float*>(zb + (uint32_t)j * 4u);
}

// The selection of row b from one read of the row (KPT scores per thread, n <= 1024 *
// KPT); returns false, having written nothing the radix path does not rewrite, when the
// sample bracket fails its check.  After the bracket only the top 16 bits of each key are
// kept (two per register); the full keys of the few candidates are read again.
template <int KPT>
__device__ __forceinline__ bool select_row_fast(RowShared& S, const SelectJob& J, int b) {
    const int tid = threadIdx.x;
    const int n = J.n_out, words = (n + 31) / 32, k = J.k;
    gchar* zb = uniform_ptr(J.z + (size_t)b * n);
    const int slots = (n + kThreads - 1) / kThreads;   // key slots in use (uniform, <= KPT)
    const int wbase = (tid / kWave) * kWave;            // first index of this wave in a slot
    // slot c of this thread (index tid + 1024 c) is in the row iff c < mine; tests against
    // this one register keep the compiler from holding an index per slot
    const int mine = (n - tid + kThreads - 1) / kThreads;

    // one round of loads: every score of the row (slots past n re-read the last one) and
    // two sample scores per thread
    float v[KPT];
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c) v[c] = load_score(zb, min(tid + kThreads * c, n - 1));
    // (n <= 65536 and tid + 1024 < 2048, so these products fit in 32 bits)
    const float sv0 = load_score(zb, (int)(((uint32_t)tid * (uint32_t)n) / kSample));
    const float sv1 = load_score(zb, (int)(((uint32_t)(tid + kThreads) * (uint32_t)n) / kSample));

    for (int w = tid; w < words; w += kThreads) {
        S.selw[w] = 0u;
        S.tiew[w] = 0u;
    }
    __syncthreads();

    if (J.mode == 1 || k >= n || k <= 0) {
        // threshold: key > tau; k >= n: every index; k == 0: none
        if (J.mode == 1 || k >= n) {
#pragma clang loop unroll(full)
            for (int c = 0; c < KPT; ++c) {
                if (c < slots)
                    ballot_words(S.selw, words, kThreads * c + wbase,
                                 c < mine && (J.mode != 1 || score_key(v[c]) > J.tau_key));
            }
        }
        return true;
    }

    if (n <= kMaxCand) {
        // every key is a candidate (slot j holds index j); the thread index is made opaque
        // so the compiler does not keep each slot's index (computed for the loads) alive
        int t_op = tid;
        asm volatile("" : "+v"(t_op));
#pragma clang loop unroll(full)
        for (int c = 0; c < KPT; ++c) {
            if (c < mine) {
                const int j = t_op + kThreads * c;
                S.cand[j] = score_key(v[c]);
                S.cand_j[j] = j;
            }
        }
        __syncthreads();
        int rem = k;
        uint32_t prefix = 0u, pmask = 0u;
        resolve_candidates(S, n, prefix, pmask, rem, 0);
        __syncthreads();
        take_ties(S, words, rem);
        return true;
    }

    // top 16 bits of every key, two per register (0 for slots past n: below every real
    // key, whose top 16 bits are at least 0x007F)
    uint32_t hk[KPT / 2];
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; c += 2) {
        const uint32_t k0 = score_key(v[c]) >> 16, k1 = score_key(v[c + 1]) >> 16;
        hk[c / 2] = (c < mine ? k0 : 0u) | ((c + 1 < mine ? k1 : 0u) << 16);
        // pin the packing here: left to itself the compiler sinks it to the first use,
        // after the bracket, and holds all KPT scores (twice the registers) until then
        asm volatile("" : "+v"(hk[c / 2]));
    }

    // bracket from the sample's top-12-bit histogram
    for (int i = tid; i < kMaxBins; i += kThreads) S.hist[i] = 0u;
    __syncthreads();
    atomicAdd(&S.hist[score_key(sv0) >> 20], 1u);
    atomicAdd(&S.hist[score_key(sv1) >> 20], 1u);
    __syncthreads();
    const int rho = (int)(((uint32_t)k * kSample + (uint32_t)n - 1u) / (uint32_t)n);
    const float sd = sqrtf((float)rho * (1.f - (float)rho / (float)kSample));
    const int margin = (int)(4.f * sd) + 2;
    uint32_t b_hi = kMaxBins - 1, b_lo = 0x7;  // 0x7: the lowest digit of a real key (NaN, -inf)
    if (rho - margin >= 1) {
        int r = rho - margin;
        b_hi = (uint32_t)find_bin<4>(S.hist, kMaxBins, r, S.part, S.sh);
    }
    if (rho + margin <= kSample) {
        int r = rho + margin;
        b_lo = (uint32_t)find_bin<4>(S.hist, kMaxBins, r, S.part, S.sh);
    }
    // as 16-bit bounds: above means hk > hi16, inside means lo16 <= hk <= hi16
    const uint32_t hi16 = (b_hi << 4) | 15u, lo16 = b_lo << 4;

    // exact counts above and inside the bracket
    int ca = 0, cm = 0;
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c) {
        // slots past the row hold 0, below lo16 (lo16 is the bin of a real sample key)
        const uint32_t h = (hk[c / 2] >> (16 * (c & 1))) & 0xFFFFu;
        ca += h > hi16 ? 1 : 0;
        cm += (h >= lo16 && h <= hi16) ? 1 : 0;
    }
    if (tid == 0) {
        S.sh[2] = (int)hi16;
        S.sh[3] = (int)lo16;
    }
    // both counts in one scan: above in the low 16 bits, inside in the high 16 (each at most
    // the row's 49152 keys, so neither part carries into the other)
    uint32_t tot2;
    const uint32_t at2 = block_exclusive_scan<kThreads, uint32_t>((uint32_t)ca | ((uint32_t)cm << 16),
                                                                 reinterpret_cast<uint32_t*>(S.wtot), &tot2);
    const int above = (int)(tot2 & 0xFFFFu), inside = (int)(tot2 >> 16);
    int at = (int)(at2 >> 16);
    if (!(above < k && k <= above + inside && inside <= kMaxCand)) return false;  // uniform

    // keys above the bracket are kept; the indices inside are gathered.  The bounds are
    // read back from LDS so the per-key tests are recomputed here rather than kept live
    // across the scans above.
    const uint32_t h_hi = (uint32_t)((volatile int*)S.sh)[2];
    const uint32_t h_lo = (uint32_t)((volatile int*)S.sh)[3];
    // the thread index, opaque to the compiler: without this it keeps every slot's index
    // (computed for the loads) alive until here
    int t_op = tid;
    asm volatile("" : "+v"(t_op));
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c) {
        if (c < slots) {
            const uint32_t h = (hk[c / 2] >> (16 * (c & 1))) & 0xFFFFu;
            ballot_words(S.selw, words, kThreads * c + wbase, h > h_hi);
            if (h >= h_lo && h <= h_hi) S.cand_j[at++] = t_op + kThreads * c;
        }
    }
    __syncthreads();
    // full keys of the candidates (the row was just read, so these hit in cache)
    {
        constexpr int kPer = kMaxCand / kThreads;
        float cv[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = min(tid + kThreads * q, inside - 1);
            cv[q] = load_score(zb, S.cand_j[i]);
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            if (tid + kThreads * q < inside) S.cand[tid + kThreads * q] = score_key(cv[q]);
    }
    __syncthreads();
    int rem = k - above;
    uint32_t prefix = 0u, pmask = 0u;
    resolve_candidates(S, inside, prefix, pmask, rem, 0);
    __syncthreads();
    take_ties(S, words, rem);
    return true;
}

// Top-k of row b (0 < k < n, kMaxCand < n <= 1024 * KPT, KPT <= 16) from one read of the
// row, the first digit from an exact histogram instead of a sample bracket: the top 12
// bits of every key (held in registers) are histogrammed, the bin holding the k-th largest
// key is found, keys above that bin are kept and the keys inside it are gathered into LDS
// with their full keys for the radix passes over the two lower digits.  Returns false,
// having written nothing the radix path does not rewrite, when that bin holds more than
// kMaxCand keys (heavy ties).  (For rows of 48 keys per thread the 48 LDS atomics per
// thread cost as much as the sample bracket saves, and more where the scores cluster.)
template <int KPT>
__device__ __forceinline__ bool select_row_hist(RowShared& S, const SelectJob& J, int b) {
    static_assert(KPT <= 16, "the full keys stay in registers");
    const int tid = threadIdx.x, lane = tid % kWave;
    const int n = J.n_out, words = (n + 31) / 32;
    gchar* zb = uniform_ptr(J.z + (size_t)b * n);
    const int slots = (n + kThreads - 1) / kThreads;   // key slots in use (uniform, <= KPT)
    const int wbase = (tid / kWave) * kWave;            // first index of this wave in a slot
    const int mine = (n - tid + kThreads - 1) / kThreads;  // slot c is in the row iff c < mine

    uint32_t key[KPT];
    {
        float v[KPT];
#pragma clang loop unroll(full)
        for (int c = 0; c < KPT; ++c) v[c] = load_score(zb, min(tid + kThreads * c, n - 1));
#pragma clang loop unroll(full)
        for (int c = 0; c < KPT; ++c) key[c] = score_key(v[c]);
    }
    for (int i = tid; i < kMaxBins + kWave; i += kThreads) S.hist[i] = 0u;
    for (int w = tid; w < words; w += kThreads) {
        S.selw[w] = 0u;
        S.tiew[w] = 0u;
    }
    __syncthreads();
    // slots past the row go to one of the 64 spare bins (one per lane), outside the search
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c)
        if (c < slots) atomicAdd(&S.hist[c < mine ? (key[c] >> 20) : (uint32_t)(kMaxBins + lane)], 1u);
    __syncthreads();
    int rem = J.k;
    const uint32_t top = (uint32_t)find_bin<4>(S.hist, kMaxBins, rem, S.part, S.sh);
    const int ncand = (int)S.hist[top];
    if (ncand > kMaxCand) return false;  // uniform

    // candidates take consecutive LDS slots from a block prefix count of each thread's own
    int mc = 0;
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c) mc += (c < mine && (key[c] >> 20) == top) ? 1 : 0;
    int total;
    int at = block_exclusive_scan<kThreads>(mc, S.wtot, &total);
    // the thread index, opaque to the compiler: without this it keeps every slot's index
    // (computed for the loads) alive until here
    int t_op = tid;
    asm volatile("" : "+v"(t_op));
#pragma clang loop unroll(full)
    for (int c = 0; c < KPT; ++c) {
        if (c < slots) {
            const uint32_t d = key[c] >> 20;
            ballot_words(S.selw, words, kThreads * c + wbase, c < mine && d > top);
            if (c < mine && d == top) {
                S.cand[at] = key[c];
                S.cand_j[at] = t_op + kThreads * c;
                ++at;
            }
        }
    }
    __syncthreads();
    uint32_t prefix = top << 20, pmask = 0xFFF00000u;
    resolve_candidates(S, ncand, prefix, pmask, rem, 1);
    __syncthreads();
    take_ties(S, words, rem);
    return true;
}

// The whole selection of row b in one block: keys in registers (rows up to 49152), with
// the radix path for longer rows and as the fallback.
__device__ __forceinline__ void select_row_full(RowShared& S, const SelectJob& J, int b) {
    const int n = J.n_out;
    bool done = false;
    if (n <= 16 * kThreads)
        done = (J.mode != 1 && J.k > 0 && J.k < n && n > kMaxCand) ? select_row_hist<16>(S, J, b)
                                                                     : select_row_fast<16>(S, J, b);
    else if (n <= 48 * kThreads) done = select_row_fast<48>(S, J, b);
    if (!done) {
        __syncthreads();
        select_row_radix(S, J, b);
    }
}

// Selection of a single row in this block, compacted into J.idx / J.count.
__device__ __forceinline__ void select_one_row_block(RowShared& S, const SelectJob& J) {
    const int tid = threadIdx.x;
    const int words = (J.n_out + 31) / 32;
    select_row_full(S, J, 0);
    __syncthreads();
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    const int total = compact_words(w0 < words ? S.selw[w0] : 0u, w1 < words ? S.selw[w1] : 0u, J.idx,
                                    S.wtot, J.lo, J.hi);
    if (tid == 0) *J.count = total;
}

// Selection over all B rows of J in this block, the union compacted into J.idx / J.count
// (rows one after another; a row's set is ORed into the union bitmap).  One row takes a
// loop-free path: inside the row loop the compiler keeps more registers live.
__device__ __forceinline__ void select_union_block(RowShared& S, const SelectJob& J, int B) {
    const int tid = threadIdx.x;
    const int words = (J.n_out + 31) / 32;
    const uint32_t* src = S.selw;
    if (B == 1) {
        select_row_full(S, J, 0);
        __syncthreads();
    } else {
#pragma nounroll
        for (int b = 0; b < B; ++b) {
            select_row_full(S, J, b);
            __syncthreads();
            for (int w = tid; w < words; w += kThreads) S.uni[w] = (b == 0 ? 0u : S.uni[w]) | S.selw[w];
            __syncthreads();
        }
        src = S.uni;
    }
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    const int total = compact_words(w0 < words ? src[w0] : 0u, w1 < words ? src[w1] : 0u, J.idx, S.wtot,
                                    J.lo, J.hi);
    if (tid == 0) *J.count = total;
}

// ---------------------------------------------------------------------------------
// Rows of at most NT scores (the head predictor): one key per thread, ranks by counting
// (keys above, plus equal keys at smaller indices), the union over the B rows, and an
// ascending compaction from wave ballots.  Any block size NT.
// ---------------------------------------------------------------------------------
template <int NT>
struct SmallShared {
    __align__(16) uint32_t keys[NT];
    int wtot[NT / kWave];
};

// Rank of `key` (thread tid's) among the n keys in LDS: keys above it plus equal keys at
// smaller indices.  Entries n .. NT-1 hold 0, below every real key (NaN and -inf map to
// 0x007FFFFF), so they never count.  Sixteen keys per step, four per 16-byte broadcast
// read, so the reads of a step are in flight together.
template <int NT>
__device__ __forceinline__ int small_rank(const SmallShared<NT>& S, uint32_t key, int n) {
    static_assert(NT % 16 == 0, "whole steps of sixteen keys");
    const uint4* k4 = reinterpret_cast<const uint4*>(S.keys);
    const int tid = threadIdx.x;
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 16) {  // j0 + 16 <= NT
        uint4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = k4[j0 / 4 + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t kj[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 4 * u + e;
                rank += (kj[e] > key || (kj[e] == key && j < tid)) ? 1 : 0;
            }
        }
    }
    return rank;
}

template <int NT>
__device__ __forceinline__ void select_small_block(SmallShared<NT>& S, const SelectJob& J, int B) {
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int n = J.n_out;
    bool sel = false;
    for (int b = 0; b < B; ++b) {
        const uint32_t key = score_key(J.z[(size_t)b * n + min(tid, n - 1)]);
        if (J.mode == 1) {
            sel = sel || (tid < n && key > J.tau_key);
        } else {
            S.keys[tid] = tid < n ? key : 0u;
            __syncthreads();
            const int rank = small_rank<NT>(S, key, n);
            sel = sel || (tid < n && rank < J.k);
            __syncthreads();
        }
    }
    sel = sel && tid >= J.lo && tid < J.hi;
    const unsigned long long m = __ballot(sel);
    if (lane == 0) S.wtot[w] = __popcll(m);
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int q = 0; q < NT / kWave; ++q) {
        const int t = S.wtot[q];
        if (q < w) base += t;
        total += t;
    }
    if (sel) J.idx[base + __popcll(m & ((1ull << lane) - 1ull))] = tid - J.lo;
    if (tid == 0) *J.count = total;
}

// Row b alone (n <= NT): the same rank test as select_small_block, written as the row's
// bitmap words (lane 0 of each wave stores its wave's 64 bits) for a union pass.
template <int NT>
__device__ __forceinline__ void select_small_row_bits(SmallShared<NT>& S, const SelectJob& J, int b) {
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int n = J.n_out, words = (n + 31) / 32;
    const uint32_t key = score_key(J.z[(size_t)b * n + min(tid, n - 1)]);
    bool sel;
    if (J.mode == 1) {
        sel = tid < n && key > J.tau_key;
    } else {
        S.keys[tid] = tid < n ? key : 0u;
        __syncthreads();
        const int rank = small_rank<NT>(S, key, n);
        sel = tid < n && rank < J.k;
    }
    const unsigned long long m = __ballot(sel);
    uint32_t* out = J.bits + (size_t)b * words;
    if (lane == 0 && 2 * w < words) out[2 * w] = (uint32_t)m;
    if (lane == 0 && 2 * w + 1 < words) out[2 * w + 1] = (uint32_t)(m >> 32);
}

}  // namespace sel
}  // namespace djv
