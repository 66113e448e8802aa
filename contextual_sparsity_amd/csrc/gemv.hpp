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
// Work decomposition (gfx950, wave64, 1024-thread blocks):
//   * A "team" of TS threads (64 = one wave, or 256 = four waves) owns one row at a
//     time; thread t of the team owns the 16-byte vectors t, t+TS, t+2TS, ... of every
//     row, so its slice of y is the same for all rows and stays in registers.
//   * A team processes G rows together: G*NV independent 16-byte loads are in flight per
//     thread before any arithmetic, and the next group's loads go out before the current
//     group is reduced, which is what keeps HBM busy.
//   * The grid is persistent: as many blocks as the device holds at once (all resident,
//     so none waits for another to finish), and team t of block b takes the groups
//     b*NT + t, b*NT + t + blocks*NT, ...; every block loads its y slice once.
//   * Dot products: fp32 weights use fp32 FMA; fp16 weights use v_dot2_f32_f16 with y
//     packed to fp16 pairs (fp32 accumulation).
//   * Team reduction: wave butterfly, then (TS = 256) a 4-entry LDS combine.
//   * The activation rows are either given, or LayerNorm(x) is applied while the slice is
//     loaded, from per-slice (mean, M2) statistics written by the kernel that produced x,
//     so no separate normalisation pass runs.  When x was accumulated in place by atomics
//     (no statistics), the team sums x's moments itself, one barrier; in 1024-thread
//     blocks the whole block loads and normalises the row once, into LDS, for its teams.
//   * One launch may serve up to three weight matrices of the same row length and input
//     (e.g. the kept heads' Q/K/V rows and both predictors' first layers, which all read
//     LN(x)), each with its own epilogue; the grid is shared in proportion to their rows.
//   * The first blocks of a launch may instead run a selection (one block over all batch
//     rows of a score vector), so a selection overlaps a long weight stream rather than
//     running alone on one compute unit.
#pragma once
#include "common.hpp"
#include "attn.hpp"
#include "select.hpp"

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
// four) slices at once.  cols <= 16384, so ntiles <= 256.  In two parts, so a caller can
// place other loads between the statistics' loads and their use.
__device__ __forceinline__ void row_moments_load(const RowInput& in, int cols, int b, float2 (&v)[4],
                                                 float (&nt)[4]) {
    const int lane = threadIdx.x % kWave;
    const float2* st = in.stats + (size_t)b * in.ntiles;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = lane + kWave * q;
        v[q] = st[min(t, in.ntiles - 1)];
        nt[q] = t < in.ntiles ? (float)min(kLnTile, cols - t * kLnTile) : 0.f;
    }
}
__device__ __forceinline__ void row_moments_finish(const RowInput& in, int cols, const float2 (&v)[4],
                                                   const float (&nt)[4], float& mean, float& rstd) {
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
__device__ __forceinline__ void row_moments(const RowInput& in, int cols, int b, float& mean,
                                            float& rstd) {
    float2 v[4];
    float nt[4];
    row_moments_load(in, cols, b, v, nt);
    row_moments_finish(in, cols, v, nt, mean, rstd);
}

// What a group's weight loads need of its segment, and what its stores need: small
// enough to keep every segment's copy in scalar registers and pick one by a uniform select.
struct SegRows {
    const char* W;
    const int32_t* idx;
    const void* bias;
    int units, rpu, with_bias;
};
struct SegOut {
    float* out;
    int ld, epi, rpu, cap;
};
__device__ __forceinline__ SegRows seg_rows(const GemvSeg& S) {
    return {reinterpret_cast<const char*>(S.W), S.list.idx, S.bias, S.list.units, S.rpu,
            S.epi == kEpiBiasRelu};
}
__device__ __forceinline__ SegOut seg_out(const GemvSeg& S) {
    return {S.out, S.ld, S.epi, S.rpu, S.list.cap};
}
template <typename Seg>
__device__ __forceinline__ Seg pick3(int i, const Seg& s0, const Seg& s1, const Seg& s2) {
    return i == 0 ? s0 : (i == 1 ? s1 : s2);
}

// Stores v (rounded to T) as element i of the T array at global address base.
template <typename T>
__device__ __forceinline__ void store_at(uint64_t base, size_t i, float v);
template <>
__device__ __forceinline__ void store_at<float>(uint64_t base, size_t i, float v) {
    *reinterpret_cast<__attribute__((address_space(1))) float*>(base + i * 4) = v;
}
template <>
__device__ __forceinline__ void store_at<__half>(uint64_t base, size_t i, float v) {
    *reinterpret_cast<__attribute__((address_space(1))) unsigned short*>(base + i * 2) =
        __half_as_ushort(to_store<__half>(v));
}

// Writes the result of visited row r (weight unit `unit`, -1 when skipped) for batch row b.
template <typename T>
__device__ __forceinline__ void epilogue(const GemvArgs& a, const SegOut& S, int r, int b, float acc,
                                         int unit, float bias) {
    switch (S.epi) {
    case kEpiStore:
        S.out[(size_t)b * S.ld + r] = acc;
        break;
    case kEpiRelu:
        S.out[(size_t)b * S.ld + r] = fmaxf(acc, 0.f);
        break;
    case kEpiBiasRelu:
        S.out[(size_t)b * S.ld + r] = unit >= 0 ? fmaxf(acc + bias, 0.f) : 0.f;
        break;
    case kEpiQkv: {
        if (unit < 0) break;
        const int u = r / S.rpu, sub = r - u * S.rpu;
        const int part = sub / a.dh, c = sub - part * a.dh;
        if (part == 0) {
            S.out[((size_t)b * S.cap + u) * a.dh + c] = acc;
        } else {
            // both cache bases moved to scalar registers and selected there: left to itself the
            // compiler selects between the two argument fields' addresses and loads the chosen
            // one with a vector load, whose wait (the load counter is in order) is also a wait
            // for every weight load in flight
            const uint64_t kc = reinterpret_cast<uint64_t>(uniform_ptr(a.Kc));
            const uint64_t vc = reinterpret_cast<uint64_t>(uniform_ptr(a.Vc));
            store_at<T>(part == 1 ? kc : vc, (((size_t)b * a.h + unit) * a.n_cap + a.n) * a.dh + c, acc);
        }
        break;
    }
    default:
        break;
    }
}

// Per-unit bias of kEpiBiasRelu, read with a scalar load of its aligned 32-bit word.
template <typename T>
__device__ __forceinline__ float load_bias(const void* bias, int unit);
template <>
__device__ __forceinline__ float load_bias<float>(const void* bias, int unit) {
    return __uint_as_float(sload_u32(reinterpret_cast<const float*>(bias) + unit));
}
template <>
__device__ __forceinline__ float load_bias<__half>(const void* bias, int unit) {
    const uint32_t w = sload_u32(reinterpret_cast<const __half*>(bias) + (unit & ~1));
    return (unit & 1) ? hi_h(w) : lo_h(w);
}

// Launch modes.  0: GEMV only.  1: the first blocks run attention chunks and selections
// of short rows (at most 256 scores), then the GEMV.  2: the first blocks run selections of
// long rows, which need 1024-thread blocks, then the GEMV.  Modes 0 and 1 use 256-thread
// blocks, which the hardware schedules with less coupling between teams.
template <int MODE> struct BlockOf { static constexpr int value = MODE == 2 ? 1024 : 256; };

// A row of zeros as long as the longest supported row: a group slot with no row (past
// the end of the list, or a skipped unit) loads from here, so every load is issued
// unconditionally and the weight buffers keep fixed registers across loop trips.
static __device__ const Vec16 g_zero_row[2048] = {};

// Weights of one group of G rows in flight, with the rows' units and biases (scalar), and
// the group's segment and index inside it.
template <int G, int NV>
struct Group {
    Vec16 w[G][NV];
    int unit[G];
    float bias[G];
    int sg, lg;
};

// OWN: the input is LN(x) of an x accumulated in place, its moments summed here (a
// separate instantiation, so the kernels of the other inputs keep their registers).
template <typename T, int TS, int NV, int NB, int G, int MODE, bool DYN, bool OWN>
__global__ __launch_bounds__(BlockOf<MODE>::value) void gemv_kernel(GemvArgs a) {
    constexpr int kThreads = BlockOf<MODE>::value;
    int bid = (int)blockIdx.x;
    if constexpr (MODE == 2) {
        if (bid < a.nside) {
            __shared__ sel::RowShared SS;
            sel::select_one_row_block(SS, a.side[bid]);  // mode 2 runs with one batch row
            return;
        }
        bid -= a.nside;
    }
    if constexpr (MODE == 1) {
        if (bid < a.nattn) {
            attn::attn_block<T>(a.attn, bid);
            return;
        }
        if (bid < a.nattn + a.nside) {
            __shared__ sel::SmallShared<kShortRows> SS;
            sel::select_small_block<kShortRows>(SS, a.side[bid - a.nattn], a.B);
            return;
        }
        bid -= a.nattn + a.nside;
    }
    constexpr int E = WTraits<T>::kPerVec;
    constexpr int NT = kThreads / TS;
    constexpr int NW = TS / kWave;  // waves per team
    __shared__ float red[2][NT][NW][G * NB];
    // OWN with several teams of several waves (1024-thread blocks): the block loads and
    // normalises the row once, into LDS, where every team reads its slices
    constexpr bool kCoop = OWN && NT > 1 && NW > 1;
    __shared__ float mom[2][OWN ? NT : 1][OWN ? NW : 1][NB];  // wave sums of the row moments
    __shared__ YSlice<T> ylds[kCoop ? kMaxRowVecs : 1];
    __shared__ float momc[2][kCoop ? kThreads / kWave : 1];

    const int tid = threadIdx.x;
    // a team is whole waves, so its index, and with it every row, unit and row address,
    // is uniform over the wave and lives in scalar registers
    const int tm = __builtin_amdgcn_readfirstlane(tid / TS);
    const int lt = tid % TS, wv = lt / kWave, ln = tid % kWave;
    // Static split: each block belongs to one segment and its teams stride over that
    // segment's groups.  Dynamic split (DYN: segments that read the same input, with device
    // counts): all GEMV blocks form one pool whose teams stride over the groups of all
    // segments, laid end to end by the counts, so a short list does not leave its blocks
    // idle while another segment's few blocks carry the launch.
    int sg0 = 0;
    int rows_seg[kMaxSeg] = {0, 0, 0}, groups_seg[kMaxSeg] = {0, 0, 0};
    int groups, stride;
    if constexpr (DYN) {
        int pool = 0;
        groups = 0;
#pragma unroll
        for (int i = 0; i < kMaxSeg; ++i)
            if (i < a.nseg) {
                rows_seg[i] = read_count_uniform(a.seg[i].list, a.flags) * a.seg[i].rpu;
                groups_seg[i] = (rows_seg[i] + G - 1) / G;
                groups += groups_seg[i];
                pool += a.seg[i].blocks;
            }
        stride = pool * NT;
    } else {
#pragma unroll
        for (int i = 0; i + 1 < kMaxSeg; ++i)
            if (sg0 == i && i + 1 < a.nseg && bid >= a.seg[i].blocks) {
                bid -= a.seg[i].blocks;
                sg0 = i + 1;
            }
    }
    const GemvSeg S = a.seg[sg0];  // the block's segment (static), or the shared input (DYN)
    const SegRows R0 = seg_rows(S), R1 = seg_rows(a.seg[1]), R2 = seg_rows(a.seg[2]);
    const SegOut O0 = seg_out(S), O1 = seg_out(a.seg[1]), O2 = seg_out(a.seg[2]);
    if constexpr (!DYN) {
        rows_seg[0] = read_count_uniform(S.list, a.flags) * S.rpu;
        groups = (rows_seg[0] + G - 1) / G;
        stride = S.blocks * NT;  // groups between a team's consecutive groups
    }
    const int nvec = a.cols / E;
    const size_t row_bytes = (size_t)a.cols * sizeof(T);

    // units (and biases) come from scalar loads and row addresses are scalar, so the
    // weight loads of a group depend on no vector load (nothing waits for the other
    // group's weights in flight).  Vector i of a row sits at scalar base row + 16*TS*i
    // and lane offset 16*lt; only the last vector can pass the row end (when the row is
    // not a whole number of team widths), and there a lane reads the row's last vector
    // instead: its activation is zero, so it adds 0 (weights are finite).
    const uint32_t lane_off = (uint32_t)lt * 16u;
    const uint32_t last_off = (uint32_t)(min(lt + TS * (NV - 1), nvec - 1) - TS * (NV - 1)) * 16u;
    gchar* zero_row = uniform_ptr(g_zero_row);
    auto load_from = [&](Group<G, NV>& q, const SegRows& Q, int rows) {
        const UnitList list{Q.idx, nullptr, 0, Q.units};
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int r = q.lg * G + g;
            int unit = -1;
            if (r < rows) unit = unit_of_uniform(list, r / Q.rpu, a.flags);
            q.unit[g] = unit;
            q.bias[g] = (Q.with_bias && unit >= 0) ? load_bias<T>(Q.bias, unit) : 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int r = q.lg * G + g;
            const int u = r / Q.rpu;
            const size_t row = (size_t)(q.unit[g] < 0 ? 0 : q.unit[g]) * Q.rpu + (r - u * Q.rpu);
            gchar* rp = q.unit[g] < 0 ? zero_row : uniform_ptr(Q.W + row * row_bytes);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                q.w[g][i] = ldg16_nt_at(rp + (size_t)16 * TS * i, i + 1 < NV ? lane_off : last_off);
        }
    };
    auto load_group = [&](Group<G, NV>& q, int grp) {
        if constexpr (DYN) {
            // group grp of the launch -> segment and index inside it
            int sg = 0, lg = grp;
#pragma unroll
            for (int i = 0; i + 1 < kMaxSeg; ++i)
                if (sg == i && i + 1 < a.nseg && lg >= groups_seg[i]) {
                    lg -= groups_seg[i];
                    sg = i + 1;
                }
            q.sg = sg;
            q.lg = lg;
            load_from(q, pick3(sg, R0, R1, R2), pick3(sg, rows_seg[0], rows_seg[1], rows_seg[2]));
        } else {
            q.sg = 0;
            q.lg = grp;
            load_from(q, R0, rows_seg[0]);
        }
    };

    // the first group's weights are requested before the activation slice is read, the
    // second group's right after it; from then on two groups per team are in flight
    const int base0 = bid * NT;
    if (base0 >= groups) return;  // uniform over the block
    Group<G, NV> qa, qb;

    // this thread's slice of every batch row (loads clamped in range, then masked).  At one
    // batch row the activation (and statistics) loads go out before the first group's
    // weights: the load counter is in order, so a wait for activations requested after the
    // weights would wait for the weights too, and the team computes nothing before its
    // activations.  (With more rows the statistics of all rows held across the weight
    // requests would cost occupancy; there the weights go first.)
    YSlice<T> ys[NB][NV];
    if constexpr (!OWN) {
        if constexpr (NB > 1) load_group(qa, base0 + tm);
        float raw[NB][NV][8];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int v = min(lt + TS * i, nvec - 1);
                load_raw<T>(S.in, a.cols, min(b, a.B - 1), v * E, raw[b][i]);
            }
        float2 stv[4];
        float ntv[4];
        if constexpr (NB == 1) {
            if (!S.in.y) row_moments_load(S.in, a.cols, 0, stv, ntv);
            load_group(qa, base0 + tm);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float mean = 0.f, rstd = 1.f;
            if (!S.in.y) {
                if constexpr (NB == 1) row_moments_finish(S.in, a.cols, stv, ntv, mean, rstd);
                else row_moments(S.in, a.cols, min(b, a.B - 1), mean, rstd);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool ok = b < a.B && lt + TS * i < nvec;
#pragma unroll
                for (int e = 0; e < E; ++e) raw[b][i][e] = ok ? (raw[b][i][e] - mean) * rstd : 0.f;
                ys[b][i].set(raw[b][i], 0);
            }
        }
        load_group(qb, base0 + stride + tm);
    } else if constexpr (kCoop) {
        // own_stats, several teams of several waves: the block's threads share the row's
        // vectors (at most KV each), sum the row's moments over all of the block's waves
        // (as the per-team form below), and leave the normalised row in LDS, where every
        // team reads its slices.  Both groups' weights are requested right after the
        // activations, so they are in flight while the moments are formed.
        static_assert(!kCoop || NB == 1, "the block-wide prologue serves one batch row");
        constexpr int KV = (NV * TS + kThreads - 1) / kThreads;
        float raw[KV][8];
#pragma unroll
        for (int k = 0; k < KV; ++k)
            load_raw<T>(S.in, a.cols, 0, min(tid + kThreads * k, nvec - 1) * E, raw[k]);
        const float sh = S.in.x[0];
        float t1 = 0.f, t2 = 0.f;
#pragma unroll
        for (int k = 0; k < KV; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float dv = tid + kThreads * k < nvec ? raw[k][e] - sh : 0.f;
                t1 += dv;
                t2 = fmaf(dv, dv, t2);
            }
        // the sums (so the wait for the activations) before the weight requests: a wait
        // placed after them would also wait for weights, the load counter being in order
        asm volatile("" : : "v"(t1), "v"(t2) : "memory");
        load_group(qa, base0 + tm);
        load_group(qb, base0 + stride + tm);
        t1 = wave_sum(t1);
        t2 = wave_sum(t2);
        const int wb = tid / kWave;
        if (ln == 0) {
            momc[0][wb] = t1;
            momc[1][wb] = t2;
        }
        __syncthreads();
        t1 = 0.f;
        t2 = 0.f;
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) {
            t1 += momc[0][w];
            t2 += momc[1][w];
        }
        const float inv_n = 1.0f / (float)a.cols;
        const float md = t1 * inv_n;
        const float mean = sh + md;
        const float rstd = 1.0f / sqrtf(fmaxf(t2 * inv_n - md * md, 0.f) + S.in.eps);
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int v = tid + kThreads * k;
            if (v < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) raw[k][e] = (raw[k][e] - mean) * rstd;
                YSlice<T> t;
                t.set(raw[k], 0);
                ylds[v] = t;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = lt + TS * i;
            if (v < nvec) ys[0][i] = ylds[v];
            else ys[0][i].zero();
        }
    } else {
        // own_stats, per team (the team holds the whole row): the moments in one pass over
        // the deviations d = x - x[0] from the row's first element, mean = x[0] + sum(d)/n
        // and variance = (sum(d^2) - sum(d)^2/n)/n (the shift keeps the squares on the
        // scale of the spread rather than of the mean); wave sums, then (several waves per
        // team) a sum over the team's waves through LDS, one barrier.  Both groups' weights
        // are requested right after the activations, before it.
        float raw[NB][NV][8];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int v = min(lt + TS * i, nvec - 1);
                load_raw<T>(S.in, a.cols, min(b, a.B - 1), v * E, raw[b][i]);
            }
        float sd[NB], sq[NB], sh[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            sh[b] = S.in.x[(size_t)min(b, a.B - 1) * a.cols];
            float t1 = 0.f, t2 = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float dv = lt + TS * i < nvec ? raw[b][i][e] - sh[b] : 0.f;
                    t1 += dv;
                    t2 = fmaf(dv, dv, t2);
                }
            sd[b] = t1;
            sq[b] = t2;
            // the sums (so the wait for the activations) before the weight requests: a wait
            // placed after them would also wait for weights, the load counter being in order
            asm volatile("" : : "v"(t1), "v"(t2) : "memory");
        }
        load_group(qa, base0 + tm);
        load_group(qb, base0 + stride + tm);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            sd[b] = wave_sum(sd[b]);
            sq[b] = wave_sum(sq[b]);
        }
        if constexpr (NW > 1) {
            if (ln == 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    mom[0][tm][wv][b] = sd[b];
                    mom[1][tm][wv][b] = sq[b];
                }
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float t1 = 0.f, t2 = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    t1 += mom[0][tm][w][b];
                    t2 += mom[1][tm][w][b];
                }
                sd[b] = t1;
                sq[b] = t2;
            }
        }
        const float inv_n = 1.0f / (float)a.cols;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float md = sd[b] * inv_n;
            const float mean = sh[b] + md;
            const float rstd = 1.0f / sqrtf(fmaxf(sq[b] * inv_n - md * md, 0.f) + S.in.eps);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool ok = b < a.B && lt + TS * i < nvec;
#pragma unroll
                for (int e = 0; e < E; ++e) raw[b][i][e] = ok ? (raw[b][i][e] - mean) * rstd : 0.f;
                ys[b][i].set(raw[b][i], 0);
            }
        }
    }

    // One group: dot products on q, then q is refilled with the group two steps ahead
    // before the reduction.  Every team of the block runs the same number of steps (a
    // team past the end computes on stale registers and stores nothing), so the block
    // barriers stay uniform.
    auto step = [&](Group<G, NV>& q, int base, int parity) {
        const int cur = base + tm;
        const int qsg = q.sg, qlg = q.lg;  // this group's segment and index inside it
        float acc[G][NB];
        int unit[G];
        float bias[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            unit[g] = q.unit[g];
            bias[g] = q.bias[g];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < NV; ++i) s = ys[b][i].dot(q.w[g][i], s);
                acc[g][b] = s;
            }
        }
        load_group(q, cur + 2 * stride);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[g][b] = wave_sum(acc[g][b]);
        if constexpr (NW == 1) {
            if (ln < G * NB && cur < groups) {
                // lane j of the wave writes result j (all lanes hold every sum)
                float v = 0.f, bs = 0.f;
                int un = -1;
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        if (ln == g * NB + b) {
                            v = acc[g][b];
                            un = unit[g];
                            bs = bias[g];
                        }
                const int g = ln / NB, b = ln % NB;
                const int r = qlg * G + g;
                if constexpr (DYN) {
                    if (r < pick3(qsg, rows_seg[0], rows_seg[1], rows_seg[2]) && b < a.B)
                        epilogue<T>(a, pick3(qsg, O0, O1, O2), r, b, v, un, bs);
                } else {
                    if (r < rows_seg[0] && b < a.B) epilogue<T>(a, O0, r, b, v, un, bs);
                }
            }
        } else {
            // wave sums through LDS, double-buffered so one barrier per group suffices
            float (&rb)[NT][NW][G * NB] = red[parity];
            if (ln == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int b = 0; b < NB; ++b) rb[tm][wv][g * NB + b] = acc[g][b];
            }
            __syncthreads();
            if (lt < G * NB && cur < groups) {
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) v += rb[tm][w][lt];
                float bs = 0.f;
                int un = -1;
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (lt / NB == g) {
                        un = unit[g];
                        bs = bias[g];
                    }
                const int g = lt / NB, b = lt % NB;
                const int r = qlg * G + g;
                if constexpr (DYN) {
                    if (r < pick3(qsg, rows_seg[0], rows_seg[1], rows_seg[2]) && b < a.B)
                        epilogue<T>(a, pick3(qsg, O0, O1, O2), r, b, v, un, bs);
                } else {
                    if (r < rows_seg[0] && b < a.B) epilogue<T>(a, O0, r, b, v, un, bs);
                }
            }
        }
    };
    // both buffers are stepped every trip (the second step of the last trip may have no
    // group for any team and then only computes on stale registers), so the loop has one
    // exit and the buffers keep their registers across trips: no copy of a buffer whose
    // loads are still in flight
    for (int base = base0; base < groups; base += 2 * stride) {
        step(qa, base, 0);
        step(qb, base + stride, 1);
    }
}

template <typename T, int TS, int NV, int NB, int G, int MODE, bool DYN, bool OWN>
int blocks_per_cu() {
    static const int occ = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void*>(&gemv_kernel<T, TS, NV, NB, G, MODE, DYN, OWN>),
                BlockOf<MODE>::value, 0) !=
                hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    return occ;
}

// Blocks per resident slot: 1 makes the grid exactly what the device holds at once.
constexpr int kOversub = 1;

// Shares the resident blocks among the segments in proportion to their groups of rows
// (at least one each) and launches.
template <typename T, int TS, int NV, int NB, int G, int MODE, bool DYN, bool OWN>
hipError_t launch_shape(GemvArgs a, hipStream_t s) {
    constexpr int NT = BlockOf<MODE>::value / TS;
    const int slots = blocks_per_cu<T, TS, NV, NB, G, MODE, DYN, OWN>() * device_cus() * kOversub;
    if (MODE != 1) a.nattn = 0;
    if (MODE == 0) a.nside = 0;
    // the prefix blocks (attention chunks, selections) are short; when they fill most of
    // the device the GEMV still gets half of it, its blocks starting as the prefix retires
    const int nprefix = a.nattn + a.nside;
    const int avail = slots - nprefix > slots / 2 ? slots - nprefix : (slots / 2 > 1 ? slots / 2 : 1);
    int want[kMaxSeg] = {0, 0, 0}, total_want = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const long long rows_cap = (long long)a.seg[i].list.cap * a.seg[i].rpu;
        const long long groups = (rows_cap + G - 1) / G;
        want[i] = (int)((groups + NT - 1) / NT);
        if (want[i] < 1) want[i] = 1;
        total_want += want[i];
    }
    int total = 0;
    for (int i = 0; i < a.nseg; ++i) {
        int b = want[i];
        if (total_want > avail) {
            b = (int)((long long)avail * want[i] / total_want);
            if (b < 1) b = 1;
        }
        a.seg[i].blocks = b;
        total += b;
    }
    dim3 grid(total + nprefix);
    prof_begin(a.prof, s);
    hipLaunchKernelGGL((gemv_kernel<T, TS, NV, NB, G, MODE, DYN, OWN>), grid, dim3(BlockOf<MODE>::value), 0, s, a);
    prof_end(a.prof, s);
    return hipGetLastError();
}

template <typename T, int TS, int NB, int MODE, bool DYN, bool OWN>
hipError_t dispatch_nv(const GemvArgs& a, int nv, hipStream_t s) {
#define DJV_GEMV_CASE(NVV, GG) \
    case NVV:                  \
        return launch_shape<T, TS, NVV, NB, GG, MODE, DYN, OWN>(a, s);
    if constexpr (TS == 64) {
        switch (nv) {
            DJV_GEMV_CASE(1, 4)
        case 2: {
            // one row per group when the launch gives its one-wave teams fewer than six rows
            // each (the P2 rows of a 16384-neuron predictor: about three per team), so every
            // team has its rows in flight in fewer, shorter rounds; two rows per group for
            // longer lists (49152 neurons: about ten per team)
            long long rows = 0;
            for (int i = 0; i < a.nseg; ++i) rows += (long long)a.seg[i].list.cap * a.seg[i].rpu;
            const long long teams = (long long)blocks_per_cu<T, 64, 2, NB, 2, MODE, DYN, OWN>() * device_cus() *
                                    (BlockOf<MODE>::value / 64);
            if (rows < 6 * teams) return launch_shape<T, 64, 2, NB, 1, MODE, DYN, OWN>(a, s);
            return launch_shape<T, 64, 2, NB, 2, MODE, DYN, OWN>(a, s);
        }
            DJV_GEMV_CASE(3, 2)
        default:
            return hipErrorInvalidValue;
        }
    } else if constexpr (MODE != 2 && NB == 1) {
        // long rows at one batch row in 256-thread blocks: two rows per group, so a team
        // has four rows in flight (the short launches of a layer are one or two latency
        // rounds, not a stream)
        switch (nv) {
            DJV_GEMV_CASE(1, 2)
            DJV_GEMV_CASE(2, 2)
            DJV_GEMV_CASE(3, 2)
            DJV_GEMV_CASE(4, 2)
            DJV_GEMV_CASE(5, 2)
            DJV_GEMV_CASE(6, 2)
            DJV_GEMV_CASE(7, 2)
            DJV_GEMV_CASE(8, 2)
        default:
            return hipErrorInvalidValue;
        }
    } else {
        switch (nv) {
            DJV_GEMV_CASE(1, 2)
            DJV_GEMV_CASE(2, 2)
            DJV_GEMV_CASE(3, 1)
            DJV_GEMV_CASE(4, 1)
            DJV_GEMV_CASE(5, 1)
            DJV_GEMV_CASE(6, 1)
            DJV_GEMV_CASE(7, 1)
            DJV_GEMV_CASE(8, 1)
        default:
            return hipErrorInvalidValue;
        }
    }
#undef DJV_GEMV_CASE
}

// Chooses the team size, vectors per thread and rows per team, and launches.  OWN: every
// segment reads LN(x) with own_stats (checked by the caller).
template <typename T, int MODE, bool DYN = false, bool OWN = false>
hipError_t dispatch(const GemvArgs& a, hipStream_t s) {
    constexpr int E = WTraits<T>::kPerVec;
    if (a.nseg < 1 || a.nseg > kMaxSeg || a.nside < 0 || a.nside > kMaxSide) return hipErrorInvalidValue;
    const int nvec = a.cols / E;
    const bool small = nvec <= 3 * 64;
    const int TS = small ? 64 : 256;
    const int nv = (nvec + TS - 1) / TS;
    const int nb = a.B <= 1 ? 1 : (a.B <= 2 ? 2 : 4);
    if constexpr (MODE == 2) {
        // long-row side selections are compiled for one batch row only (the launcher runs
        // them separately otherwise)
        if (nb != 1) return hipErrorInvalidValue;
        return small ? dispatch_nv<T, 64, 1, MODE, DYN, OWN>(a, nv, s) : dispatch_nv<T, 256, 1, MODE, DYN, OWN>(a, nv, s);
    } else {
        if (small) {
            if (nb == 1) return dispatch_nv<T, 64, 1, MODE, DYN, OWN>(a, nv, s);
            if (nb == 2) return dispatch_nv<T, 64, 2, MODE, DYN, OWN>(a, nv, s);
            return dispatch_nv<T, 64, 4, MODE, DYN, OWN>(a, nv, s);
        }
        if (nb == 1) return dispatch_nv<T, 256, 1, MODE, DYN, OWN>(a, nv, s);
        if (nb == 2) return dispatch_nv<T, 256, 2, MODE, DYN, OWN>(a, nv, s);
        return dispatch_nv<T, 256, 4, MODE, DYN, OWN>(a, nv, s);
    }
}

}  // namespace gemv_detail
}  // namespace djv
