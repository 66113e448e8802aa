// Row-gather GEMV for batches of more than kMaxBatch rows, on the matrix cores.
//
// The same product as gemv.hpp, out[b, r] = W[row(r)] . y_b for the visited rows r, but
// with up to 32 batch rows the vector ALU can no longer keep pace with HBM (about two
// multiply-adds per weight byte per batch row), so the dot products run as
// v_mfma_f32_16x16x32_f16: a wave multiplies a tile of 16 weight rows by the batch (16 or
// 32 rows, zero-padded) over a slice of the row length.  In that instruction a lane holds 8
// consecutive k of one row of each operand, so one 16-byte load of a weight row is one A
// fragment and one 16-byte load of an activation row is one B fragment.
//
// Three launches: each segment's activations are normalised (LN from slice statistics, or
// the given rows) into an fp16 copy Yh [seg][Bpad, cols] that stays in L2; the MFMA kernel
// writes one fp32 partial per (k-slice, row, batch row); a finalize sums the slices in order
// and applies the segment's epilogue (store, ReLU, bias + ReLU, Q/K/V with the cache append).
#include "gemv.hpp"

namespace djv {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kMK = 32;        // k per MFMA
constexpr int kTile = 16;      // weight rows per wave
constexpr int kU = 4;          // MFMA steps with loads in flight together

// Yh[sg][b, :] = fp16 of segment sg's input row b (zero for b >= B).  One block of 256 per
// (row b, segment sg).
__global__ __launch_bounds__(256) void normalize_f16_kernel(GemvArgs a, int bpad, __half* Yh) {
    const int b = blockIdx.x, sg = blockIdx.y;
    const RowInput& in = a.seg[sg].in;
    const int cols = a.cols, B = a.B;
    __half* dst = Yh + ((size_t)sg * bpad + b) * cols;
    if (b >= B) {
        for (int c = threadIdx.x; c < cols; c += 256) dst[c] = __float2half_rn(0.f);
        return;
    }
    float mean = 0.f, rstd = 1.f;
    if (!in.y) gemv_detail::row_moments(in, cols, b, mean, rstd);  // every wave, same values
    const float* src = (in.y ? in.y : in.x) + (size_t)b * cols;
    for (int c = threadIdx.x; c < cols; c += 256) dst[c] = __float2half_rn((src[c] - mean) * rstd);
}

// Item i of a segment: tile i / S of 16 visited rows, k-slice i % S.
__device__ __forceinline__ int seg_of(const GemvArgs& a, const int* items, int& item) {
    int sg = 0;
#pragma unroll
    for (int i = 0; i + 1 < kMaxSeg; ++i)
        if (sg == i && i + 1 < a.nseg && item >= items[i]) {
            item -= items[i];
            sg = i + 1;
        }
    return sg;
}

struct MfmaPlan {
    int S;                 // k-slices
    int ks;                // columns per slice (multiple of kMK)
    int bpad;              // 16 or 32
    int items[kMaxSeg];    // tiles * S per segment
    long long off[kMaxSeg];  // partial offset (floats) per segment
    const __half* Yh;
    float* P;              // partials [S][rows_cap][bpad] per segment
};

template <int BT>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(GemvArgs a, MfmaPlan p) {
    const int l = threadIdx.x % kWave;
    int item = blockIdx.x * (256 / kWave) + (int)(threadIdx.x / kWave);
    item = __builtin_amdgcn_readfirstlane(item);
    int total = 0;
    for (int i = 0; i < a.nseg; ++i) total += p.items[i];
    if (item >= total) return;  // whole wave
    const int sg = seg_of(a, p.items, item);
    const GemvSeg& S = a.seg[sg];
    const int tile = item / p.S, slice = item - tile * p.S;
    const int rows = read_count_uniform(S.list, a.flags) * S.rpu;
    if (tile * kTile >= rows) return;  // whole wave
    // this lane's weight row (A fragment rows) and k offset
    const int r = tile * kTile + l % kTile;
    int unit = -1;
    if (r < rows) unit = unit_of(S.list, r / S.rpu, a.flags);
    const int ub = unit < 0 ? 0 : unit;
    const size_t wrow = (size_t)ub * S.rpu + (r - (r / S.rpu) * S.rpu);
    const int kofs = slice * p.ks + 8 * (l / kTile);
    const _Float16* wp = reinterpret_cast<const _Float16*>(S.W) + wrow * a.cols + kofs;
    const h8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const _Float16* yp[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
        yp[t] = reinterpret_cast<const _Float16*>(p.Yh) + ((size_t)sg * p.bpad + 16 * t + l % kTile) * a.cols + kofs;
    f4_t acc[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + kMK * kU <= p.ks; k += kMK * kU) {
        h8_t w[kU], y[kU][BT];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            w[u] = __builtin_nontemporal_load(reinterpret_cast<const h8_t*>(wp + k + kMK * u));
#pragma unroll
            for (int t = 0; t < BT; ++t) y[u][t] = *reinterpret_cast<const h8_t*>(yp[t] + k + kMK * u);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const h8_t wu = unit < 0 ? zero8 : w[u];
#pragma unroll
            for (int t = 0; t < BT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wu, y[u][t], acc[t], 0, 0, 0);
        }
    }
    for (; k < p.ks; k += kMK) {
        const h8_t w = __builtin_nontemporal_load(reinterpret_cast<const h8_t*>(wp + k));
        const h8_t wu = unit < 0 ? zero8 : w;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const h8_t y = *reinterpret_cast<const h8_t*>(yp[t] + k);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wu, y, acc[t], 0, 0, 0);
        }
    }
    // lane l holds D[row 4 (l / 16) + q][batch l % 16] for q = 0..3
    const int rows_cap = S.list.cap * S.rpu;
    float* P = p.P + p.off[sg] + (size_t)slice * rows_cap * p.bpad;
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = tile * kTile + 4 * (l / kTile) + q;
            if (rr < rows) P[(size_t)rr * p.bpad + 16 * t + l % kTile] = acc[t][q];
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
    gemv_detail::epilogue<T>(a, S, r, b, acc, unit, bias);
}

}  // namespace

// Slices per segment and partial sizes for a launch (the same function sizes the
// workspace, so a plan never exceeds it).
void mfma_shape(const GemvArgs& a, int* S, long long* floats) {
    long long tiles = 0, rows_cap = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const long long rc = (long long)a.seg[i].list.cap * a.seg[i].rpu;
        rows_cap += rc;
        tiles += (rc + kTile - 1) / kTile;
    }
    const int kblocks = a.cols / kMK;
    int s = 1;
    // enough waves to fill the device (about 2048), with slices that divide the row
    while (tiles * s < 2048 && s < 16 && kblocks % (2 * s) == 0) s *= 2;
    *S = s;
    *floats = (long long)s * rows_cap * (a.B <= 16 ? 16 : 32);
}

hipError_t launch_gemv_mfma(const GemvArgs& a, __half* Yh, float* partial, hipStream_t s) {
    if (a.B <= kMaxBatch || a.B > 32 || a.cols % kMK != 0) return hipErrorInvalidValue;
    MfmaPlan p{};
    long long floats = 0;
    mfma_shape(a, &p.S, &floats);
    p.ks = a.cols / p.S;
    p.bpad = a.B <= 16 ? 16 : 32;
    p.Yh = Yh;
    p.P = partial;
    long long off = 0, items = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const long long rc = (long long)a.seg[i].list.cap * a.seg[i].rpu;
        p.items[i] = (int)(((rc + kTile - 1) / kTile) * p.S);
        p.off[i] = off;
        off += (long long)p.S * rc * p.bpad;
        items += p.items[i];
    }
    hipLaunchKernelGGL(normalize_f16_kernel, dim3(p.bpad, a.nseg), dim3(256), 0, s, a, p.bpad, Yh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int blocks = (int)((items + 3) / 4);
    prof_begin(a.prof, s);
    if (p.bpad == 16) hipLaunchKernelGGL(gemv_mfma_kernel<1>, dim3(blocks), dim3(256), 0, s, a, p);
    else hipLaunchKernelGGL(gemv_mfma_kernel<2>, dim3(blocks), dim3(256), 0, s, a, p);
    prof_end(a.prof, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    long long outs = 0;
    for (int i = 0; i < a.nseg; ++i) outs += (long long)a.seg[i].list.cap * a.seg[i].rpu * a.B;
    hipLaunchKernelGGL(gemv_mfma_finalize_kernel<__half>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, a, p);
    return hipGetLastError();
}

}  // namespace djv
