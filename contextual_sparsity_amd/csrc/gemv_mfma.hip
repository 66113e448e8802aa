// Row-gather GEMV on the matrix cores: batches of more than kMaxBatch rows, and smaller
// fp16 batches when the caller asks for this form.
//
// The same product as gemv.hpp, out[b, r] = W[row(r)] . y_b for the visited rows r, but
// with up to 32 batch rows the vector ALU can no longer keep pace with HBM (about two
// multiply-adds per weight byte per batch row), so the dot products run as
// v_mfma_f32_16x16x32_f16: a wave multiplies a tile of 16 weight rows by the batch (16 or
// 32 rows, zero-padded).  In that instruction a lane holds 8 consecutive k of one row of
// each operand, so one 16-byte load of a weight row is one A fragment.
//
// The activations stay put and the weights stream past them.  A block of 16 waves owns
// one k-slice of up to kSliceHalfs / Bpad columns and a contiguous share of the 16-row
// tiles of all segments, split by the device counts: it normalises the slice of every
// batch row (LN from slice statistics, or the given rows) into LDS as fp16 (again only
// where a segment reads another input), and its waves walk the tiles, loading 8 weight
// fragments per chunk and multiplying them with activation fragments from LDS; 16 waves
// per compute unit keep the loads in flight.  One block fills a compute unit's LDS, so
// the grid is one block per compute unit.  Each tile writes one fp32 partial per (slice, row, batch
// row), four tiles' partials at a time; a finalize sums the slices in order and applies the segment's epilogue (store,
// ReLU, bias + ReLU, Q/K/V with the cache append).
#include "gemv.hpp"

namespace djv {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) h8_t gh8_t;  // global: loads count on vmcnt only

__device__ __forceinline__ gh8_t* as_global(const void* p) {
    return reinterpret_cast<gh8_t*>(reinterpret_cast<uint64_t>(p));
}

constexpr int kMK = 32;              // k per MFMA
constexpr int kTile = 16;            // weight rows per wave tile
constexpr int kBlock = 1024;         // threads per block (16 waves)
constexpr int kWaves = kBlock / kWave;
constexpr int kSliceHalfs = 65536;   // LDS activation slice: Bpad x columns (128 KiB)
constexpr int kPad = 8;              // halfs of padding per LDS row

__host__ __device__ constexpr int bpad_of(int B) { return B <= 16 ? 16 : 32; }

struct MfmaPlan {
    int S;                   // k-slices (all segments share the row length)
    int kc;                  // columns per slice (multiple of kMK; the last may be shorter)
    int bpad;                // 16 or 32
    int G;                   // row groups: block = (group, slice), S * G blocks
    long long off[kMaxSeg];  // partial offset (floats) per segment
    float* P;                // partials [S][rows_cap][bpad] per segment
};

// Normalises the activation slice [k0, k0 + kn) of input `in` for every batch row into
// LDS as fp16 (LayerNorm from the slice statistics, or the given rows); zero rows past B.
template <int BP>
__device__ __forceinline__ void fill_slice(_Float16* ys, float (*mom)[2], const RowInput& in,
                                           const GemvArgs& a, int k0, int kn, int pitch, int wv) {
    const int tid = threadIdx.x, l = tid % kWave;
    if (!in.y) {
        for (int b = wv; b < BP; b += kWaves) {
            float mean = 0.f, rstd = 1.f;
            if (b < a.B) gemv_detail::row_moments(in, a.cols, b, mean, rstd);
            if (l == 0) {
                mom[b][0] = mean;
                mom[b][1] = rstd;
            }
        }
        __syncthreads();
    }
    const float* src = in.y ? in.y : in.x;
    const int q4 = kn / 4;
    for (int i = tid; i < BP * q4; i += kBlock) {
        const int b = i / q4, c = 4 * (i - b * q4);
        h4_t h = {0, 0, 0, 0};
        if (b < a.B) {
            const float4 v = *reinterpret_cast<const float4*>(src + (size_t)b * a.cols + k0 + c);
            const float m = in.y ? 0.f : mom[b][0], r = in.y ? 1.f : mom[b][1];
            h = h4_t{(_Float16)((v.x - m) * r), (_Float16)((v.y - m) * r), (_Float16)((v.z - m) * r),
                     (_Float16)((v.w - m) * r)};
        }
        *reinterpret_cast<h4_t*>(&ys[b * pitch + c]) = h;
    }
    __syncthreads();
}

__device__ __forceinline__ bool same_input(const RowInput& p, const RowInput& q) {
    return same_row_input(p, q);
}

template <int BT>
__global__ __launch_bounds__(kBlock) void gemv_mfma_kernel(GemvArgs a, MfmaPlan p) {
    constexpr int BP = BT * 16;
    constexpr int kU = 8;                // weight fragments per chunk
    constexpr int kChunk = kMK * kU;     // columns per chunk
    constexpr int kGroup = 4;            // tiles whose partials are stored together
    extern __shared__ __align__(16) _Float16 ys[];  // [BP][kc + kPad]
    __shared__ float mom[BP][2];
    const int tid = threadIdx.x, l = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int slice = blockIdx.x % p.S, grp = blockIdx.x / p.S;
    const int k0 = slice * p.kc;
    const int kn = min(p.kc, a.cols - k0);
    const int pitch = p.kc + kPad;
    const int nck = (kn + kChunk - 1) / kChunk;
    const int kl = 8 * (l / kTile);  // this lane's k offset inside a step
    gh8_t* zero_base = as_global(gemv_detail::g_zero_row) + kl / 8;
    const h8_t* yrow[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
        yrow[t] = reinterpret_cast<const h8_t*>(ys + (16 * t + l % kTile) * pitch + kl);

    // the block's share of the 16-row tiles of all segments (from the device counts)
    int T[kMaxSeg] = {0, 0, 0}, T_all = 0;
#pragma unroll
    for (int i = 0; i < kMaxSeg; ++i)
        if (i < a.nseg) {
            T[i] = (read_count_uniform(a.seg[i].list, a.flags) * a.seg[i].rpu + kTile - 1) / kTile;
            T_all += T[i];
        }
    const int g_begin = (int)((long long)grp * T_all / p.G), g_end = (int)((long long)(grp + 1) * T_all / p.G);

    int loaded = -1;  // segment whose input is in LDS
    int seg_start = 0;
    for (int sg = 0; sg < a.nseg; seg_start += T[sg], ++sg) {
        const int lo = max(g_begin, seg_start) - seg_start, hi = min(g_end, seg_start + T[sg]) - seg_start;
        if (lo >= hi) continue;  // block-uniform
        const GemvSeg& S = a.seg[sg];
        if (loaded < 0 || !same_input(a.seg[loaded].in, S.in)) {
            if (loaded >= 0) __syncthreads();
            fill_slice<BP>(ys, mom, S.in, a, k0, kn, pitch, wv);
        }
        loaded = sg;

        const int rows = read_count_uniform(S.list, a.flags) * S.rpu;
        const int rows_cap = S.list.cap * S.rpu;
        float* P = p.P + p.off[sg] + (size_t)slice * rows_cap * p.bpad;
        const int first = __builtin_amdgcn_readfirstlane(lo + wv);  // this wave's tiles: first + 16 i
        const int ntw = __builtin_amdgcn_readfirstlane(first < hi ? (hi - first + kWaves - 1) / kWaves : 0);
        // fragment base of this lane's row in tile i (the zero row for absent rows)
        auto tile_ptr = [&](int i) -> gh8_t* {
            const int r = (first + i * kWaves) * kTile + l % kTile;
            int unit = -1;
            if (i < ntw && r < rows) unit = unit_of(S.list, r / S.rpu, a.flags);
            if (unit < 0) return zero_base;
            const int sub = r - (r / S.rpu) * S.rpu;
            return as_global(reinterpret_cast<const _Float16*>(S.W) + ((size_t)unit * S.rpu + sub) * a.cols + k0 + kl);
        };
        // straight-line chunks: steps past the slice end reload its last step (in bounds) and
        // multiply zeros
        auto load = [&](h8_t (&w)[kU], gh8_t* ptr, int ck) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int k = min(ck * kChunk + kMK * u, kn - kMK);
                w[u] = __builtin_nontemporal_load(ptr + k / 8);
            }
        };
        const h8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        auto compute = [&](f4_t (&acc)[BT], const h8_t (&w)[kU], int ck) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const bool in = ck * kChunk + kMK * u < kn;
                const int k = min(ck * kChunk + kMK * u, kn - kMK);
                const h8_t wu = in ? w[u] : zero8;
#pragma unroll
                for (int t = 0; t < BT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wu, yrow[t][k / 8], acc[t], 0, 0, 0);
            }
        };
        // per tile: all chunks of the slice, 8 weight fragments in flight per chunk (other
        // waves cover the latency); the next tile's row is looked up a tile ahead.  The
        // partials of kGroup tiles are kept in registers and stored together: a wave's stores
        // share the in-order memory counter with its loads, so a load wait after a store also
        // waits for the store's acknowledgement, slow while the reads saturate HBM.
        gh8_t* P1 = tile_ptr(0);
        for (int i0 = 0; i0 < ntw; i0 += kGroup) {
            f4_t acc[kGroup][BT];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
#pragma unroll
                for (int t = 0; t < BT; ++t) acc[j][t] = f4_t{0.f, 0.f, 0.f, 0.f};
                if (i0 + j < ntw) {  // uniform
                    gh8_t* P0 = P1;
                    P1 = tile_ptr(i0 + j + 1);
                    for (int ck = 0; ck < nck; ++ck) {
                        h8_t w[kU];
                        load(w, P0, ck);
                        compute(acc[j], w, ck);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kGroup; ++j)
#pragma unroll
                for (int t = 0; t < BT; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int rr = (first + (i0 + j) * kWaves) * kTile + 4 * (l / kTile) + q;
                        if (i0 + j < ntw && rr < rows) P[(size_t)rr * p.bpad + 16 * t + l % kTile] = acc[j][t][q];
                    }
        }
    }
}

// Sums the k-slices in order and applies the segment's epilogue; one thread per (row, b).
template <typename T>
__global__ __launch_bounds__(256) void gemv_mfma_finalize_kernel(GemvArgs a, MfmaPlan p) {
    long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    int sg = 0;
    for (; sg < a.nseg; ++sg) {
        const long long n = (long long)a.seg[sg].list.cap * a.seg[sg].rpu * a.B;
        if (id < n) break;
        id -= n;
    }
    if (sg >= a.nseg) return;
    const GemvSeg& S = a.seg[sg];
    const int r = (int)(id / a.B), b = (int)(id - (long long)r * a.B);
    const int rows = read_count(S.list, a.flags) * S.rpu;
    if (r >= rows) return;
    const int rows_cap = S.list.cap * S.rpu;
    const float* P = p.P + p.off[sg] + (size_t)r * p.bpad + b;
    float acc = 0.f;
    for (int s = 0; s < p.S; ++s) acc += P[(size_t)s * rows_cap * p.bpad];
    const int unit = unit_of(S.list, r / S.rpu, a.flags);
    float bias = 0.f;
    if (S.epi == kEpiBiasRelu && unit >= 0) bias = to_f32<T>(reinterpret_cast<const T*>(S.bias)[unit]);
    gemv_detail::epilogue<T>(a, gemv_detail::seg_out(S), r, b, acc, unit, bias);
}

// Slices of a row of `cols` columns for batch padding bpad: as few as the LDS allows, of
// equal width rounded up to kMK.
void slice_shape(int cols, int bpad, int* S, int* kc) {
    const int kcm = (kSliceHalfs / bpad - kPad) / kMK * kMK;  // columns one block can hold
    int s = (cols + kcm - 1) / kcm;
    if (s < 1) s = 1;
    int w = (cols + s - 1) / s;
    w = (w + kMK - 1) / kMK * kMK;
    *S = s;
    *kc = w;
}

}  // namespace

long long mfma_partial_floats(int B, long long max_rows, int max_cols) {
    const int bpad = bpad_of(B);
    int S = 1, kc = 0;
    slice_shape(max_cols, bpad, &S, &kc);
    return (long long)S * max_rows * bpad;
}

hipError_t launch_gemv_mfma(const GemvArgs& a, float* partial, hipStream_t s) {
    if (a.B < 1 || a.B > kMaxBatchMfma || a.cols % kMK != 0 || !partial) return hipErrorInvalidValue;
    for (int i = 0; i < a.nseg; ++i)
        if (!a.seg[i].in.y && (!a.seg[i].in.x || !a.seg[i].in.stats || a.seg[i].in.own_stats))
            return hipErrorInvalidValue;
    MfmaPlan p{};
    p.bpad = bpad_of(a.B);
    slice_shape(a.cols, p.bpad, &p.S, &p.kc);
    p.P = partial;
    // one block per compute unit: G row groups per slice, each a contiguous share of the
    // tiles of all segments (split on the device by the actual counts)
    const int cus = device_cus();
    long long off = 0, tiles_cap = 0;
    for (int i = 0; i < a.nseg; ++i) {
        p.off[i] = off;
        off += (long long)p.S * a.seg[i].list.cap * a.seg[i].rpu * p.bpad;
        tiles_cap += ((long long)a.seg[i].list.cap * a.seg[i].rpu + kTile - 1) / kTile;
    }
    long long G = cus / p.S;
    if (G > tiles_cap) G = tiles_cap;
    if (G < 1) G = 1;
    p.G = (int)G;
    const int blocks = p.G * p.S;
    const size_t lds = (size_t)p.bpad * (p.kc + kPad) * sizeof(_Float16);
    static const hipError_t opt_in = [] {
        const int most = (kSliceHalfs + 32 * kPad) * (int)sizeof(_Float16);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_mfma_kernel<1>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, most);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_mfma_kernel<2>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, most);
        return e;
    }();
    if (opt_in != hipSuccess) return opt_in;
    prof_begin(a.prof, s);
    if (p.bpad == 16) hipLaunchKernelGGL(gemv_mfma_kernel<1>, dim3(blocks), dim3(kBlock), lds, s, a, p);
    else hipLaunchKernelGGL(gemv_mfma_kernel<2>, dim3(blocks), dim3(kBlock), lds, s, a, p);
    prof_end(a.prof, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    long long outs = 0;
    for (int i = 0; i < a.nseg; ++i) outs += (long long)a.seg[i].list.cap * a.seg[i].rpu * a.B;
    if (outs == 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_mfma_finalize_kernel<__half>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, a, p);
    return hipGetLastError();
}

}  // namespace djv
