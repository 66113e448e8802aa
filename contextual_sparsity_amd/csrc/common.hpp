// Shared device helpers and the internal launch interface of libdejavu.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

#include "dejavu.h"

namespace djv {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxBatch = DJV_MAX_VALU_BATCH;  // batch rows held in registers by the vector-ALU kernels
constexpr int kMaxBatchMfma = DJV_MAX_BATCH;   // batch rows of the matrix-core kernels (fp16 weights)
constexpr unsigned kFlagBadIndex = 1u;
constexpr unsigned kFlagBadCount = 2u;

// ------------------------------------------------------------------------------------
// 16-byte vector of weights and its conversion to fp32
// ------------------------------------------------------------------------------------
struct alignas(16) Vec16 {
    uint32_t w[4];
};

template <typename T> struct WTraits;
template <> struct WTraits<float> {
    static constexpr int kPerVec = 4;   // elements per 16-byte vector
};
template <> struct WTraits<__half> {
    static constexpr int kPerVec = 8;
};

__device__ __forceinline__ Vec16 ldg16(const void* p) {
    // Plain global 128-bit load; weights are streamed once per call.
    return *reinterpret_cast<const Vec16*>(p);
}

__device__ __forceinline__ Vec16 ldg16_nt(const void* p) {
    // Non-temporal 128-bit load for streamed weights that are not reused.
    Vec16 v;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    v.w[0] = t[0]; v.w[1] = t[1]; v.w[2] = t[2]; v.w[3] = t[3];
    return v;
}

// A global-memory pointer known to be the same in every lane of the wave, moved to
// scalar registers: a 16-byte load through it at a 32-bit per-lane offset takes the
// scalar-base form (one vector register per offset, no 64-bit address arithmetic).
typedef const __attribute__((address_space(1))) char gchar;
__device__ __forceinline__ gchar* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ Vec16 ldg16_nt_at(gchar* base, uint32_t off) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4 gu32x4;
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<gu32x4*>(base + off));
    Vec16 v;
    v.w[0] = t[0]; v.w[1] = t[1]; v.w[2] = t[2]; v.w[3] = t[3];
    return v;
}

__device__ __forceinline__ float lo_h(uint32_t u) {
    return __half2float(__ushort_as_half((unsigned short)(u & 0xffffu)));
}
__device__ __forceinline__ float hi_h(uint32_t u) {
    return __half2float(__ushort_as_half((unsigned short)(u >> 16)));
}

// Expand a vector into fp32 elements.
template <typename T>
__device__ __forceinline__ void unpack(const Vec16& v, float (&f)[WTraits<T>::kPerVec]);
template <>
__device__ __forceinline__ void unpack<float>(const Vec16& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v.w[i]);
}
template <>
__device__ __forceinline__ void unpack<__half>(const Vec16& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_h(v.w[i]);
        f[2 * i + 1] = hi_h(v.w[i]);
    }
}

// Round an fp32 value to the storage type (round-to-nearest-even).
template <typename T> __device__ __forceinline__ T to_store(float x);
template <> __device__ __forceinline__ float to_store<float>(float x) { return x; }
template <> __device__ __forceinline__ __half to_store<__half>(float x) { return __float2half_rn(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__half>(__half x) { return __half2float(x); }

// ------------------------------------------------------------------------------------
// Reductions
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Sum over a block of NT threads (NT a multiple of 64); red holds NT/64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NT / kWave; ++q) s += red[q];
    __syncthreads();
    return s;
}

// LayerNorm statistics travel as (mean, M2) of each kLnTile-column slice of a row.
constexpr int kLnTile = 64;
constexpr int kMaxRowVecs = 256 * 8;  // 16-byte vectors of the longest weight row (32 KiB)

// Order-preserving key of an fp32 score: larger score, larger key; -0 = +0; NaN ranks as
// -inf.
__device__ __forceinline__ uint32_t score_key(float z) {
    uint32_t u = __float_as_uint(z);
    if (z != z) u = 0xFF800000u;
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void set_flag(unsigned* flags, unsigned bit) {
    if (flags) atomicOr(flags, bit);
}

// ------------------------------------------------------------------------------------
// Row maps: which weight rows a launch visits.
//   A unit (a neuron, a head, a predictor output) owns `rpu` consecutive rows.
//   Unit slot u in [0, count) names unit idx[u] (or u when idx == nullptr).
// ------------------------------------------------------------------------------------
struct UnitList {
    const int32_t* idx;    // ascending unit indices (nullptr: identity)
    const int32_t* count;  // device count (nullptr: cap)
    int cap;               // list capacity
    int units;             // number of units in the weight tensor
};

__device__ __forceinline__ int read_count(const UnitList& L, unsigned* flags) {
    if (!L.count) return L.cap;
    int c = *L.count;
    if (c < 0 || c > L.cap) {
        set_flag(flags, kFlagBadCount);
        c = c < 0 ? 0 : L.cap;
    }
    return c;
}

// Scalar (wave-uniform) load of an int through the constant address space: the value
// lands in a scalar register and the wait for it does not also wait for the vector loads
// in flight.  Only for addresses uniform over the wave, in memory the running kernel does
// not write.
typedef const __attribute__((address_space(4))) int32_t cint32_k;
typedef const __attribute__((address_space(4))) uint32_t cuint32_k;
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) { return *(cint32_k*)p; }
__device__ __forceinline__ uint32_t sload_u32(const void* p) { return *(cuint32_k*)p; }

__device__ __forceinline__ int read_count_uniform(const UnitList& L, unsigned* flags) {
    if (!L.count) return L.cap;
    int c = sload_i32(L.count);
    if (c < 0 || c > L.cap) {
        set_flag(flags, kFlagBadCount);
        c = c < 0 ? 0 : L.cap;
    }
    return c;
}

__device__ __forceinline__ int unit_of_uniform(const UnitList& L, int u, unsigned* flags) {
    if (!L.idx) return u;
    const int j = sload_i32(L.idx + u);
    if (j < 0 || j >= L.units) {
        set_flag(flags, kFlagBadIndex);
        return -1;
    }
    return j;
}

// Returns the unit of slot u or -1 (and flags it) when the index is out of range.
__device__ __forceinline__ int unit_of(const UnitList& L, int u, unsigned* flags) {
    if (!L.idx) return u;
    int j = L.idx[u];
    if (j < 0 || j >= L.units) {
        set_flag(flags, kFlagBadIndex);
        return -1;
    }
    return j;
}

}  // namespace djv

// ------------------------------------------------------------------------------------
// Internal launchers (defined in the kernel translation units)
// ------------------------------------------------------------------------------------
namespace djv {

enum GemvEpi : int {
    kEpiStore = 0,      // out[b*ld + r] = acc
    kEpiRelu = 1,       // out[b*ld + r] = max(acc, 0)
    kEpiBiasRelu = 2,   // out[b*ld + u] = max(acc + bias[unit], 0)
    kEpiQkv = 3,        // q -> out, k/v -> cache position n (rounded to the cache dtype)
};

// Activation rows fed to a GEMV: either ready rows y, or LayerNorm(x) applied on the fly,
// with the moments of x either combined from per-tile statistics written by the kernel
// that produced x (see LnTiles), or (own_stats: x accumulated in place by the row-axpys,
// which write no statistics) summed by the consumer itself from the values it loads.
struct RowInput {
    const float* y;       // [B, cols] ready input; when nullptr, LN(x) is used
    const float* x;       // [B, cols] residual stream
    const float2* stats;  // [B, ntiles] (mean, M2) of each kLnTile-column slice of x
    int ntiles;
    float eps;
    bool own_stats;       // moments of x from x itself (stats unused)
};

__host__ __device__ inline bool same_row_input(const RowInput& p, const RowInput& q) {
    return p.y == q.y && p.x == q.x && p.stats == q.stats && p.ntiles == q.ntiles && p.eps == q.eps &&
           p.own_stats == q.own_stats;
}

constexpr int kAttnMaxChunks = 1024;   // chunks per head the merge kernel accepts
constexpr int kFuseMaxChunks = 128;    // chunks per head the O-projection merges itself

struct AttnArgs {
    const void* Kc;       // [B, h, n_cap, dh]
    const void* Vc;
    UnitList list;        // heads
    int h, dh, n, n_cap, B;
    const float* q;       // [B, cap, dh]
    float scale;
    float* part;          // [B, cap, nchunk, dh + 2]
    int chunk;            // positions per chunk
    int nchunk;
    float* H;             // [B, cap, dh] (when merged by the merge kernel)
    unsigned* flags;
    int prof;
};

struct SelectJob {
    const float* z;       // [B, n_out]
    int n_out;
    int mode;             // 0 top-k, 1 threshold
    int k;
    uint32_t tau_key;     // threshold in the order-preserving key space
    uint32_t* bits;       // [B, words] per-row selection bitmaps (workspace; parallel rows only)
    int32_t* idx;         // [n_out]
    int32_t* count;       // [1]
    int lo, hi;           // units listed: those in [lo, hi), as j - lo (0, n_out: all)
};

// One weight matrix served by a GEMV launch (a launch serves up to three, all with rows
// of the same length and the same kind of input).
struct GemvSeg {
    const void* W;        // rows of `cols` elements
    UnitList list;        // which units
    int rpu;              // rows per unit
    RowInput in;
    float* out;           // fp32 output
    int ld;               // leading dimension of out per batch row
    int epi;              // GemvEpi of this segment
    const void* bias;     // kEpiBiasRelu: per-unit bias (weight dtype)
    int blocks;           // blocks of the launch serving this segment (set by the launcher)
};

constexpr int kMaxSeg = 3;
constexpr int kMaxSide = 2;
constexpr int kShortRows = 256;  // selections of rows up to this long fit any block size

struct GemvArgs {
    GemvSeg seg[kMaxSeg];
    int nseg;
    int cols;             // row length in elements (d or r), shared by all segments
    int B;
    // kEpiQkv: cache [B, h, n_cap, dh]
    void* Kc;
    void* Vc;
    int h, dh, n, n_cap;
    // selections run by the first nside blocks of the launch, each over all B rows of its
    // scores (union in the block), independent of the GEMV segments
    SelectJob side[kMaxSide];
    int nside;
    // attention chunks run by the first nattn blocks (256-thread launches), before the side
    // selections and the GEMV segments; independent of both
    AttnArgs attn;
    int nattn;
    // matrix-core form (fp16 weights, cols % 32 == 0; required above kMaxBatch rows) and
    // its k-slice partials (workspace, mfma_partial_floats)
    bool mfma;
    float* mfma_part;
    // set by the launcher: the dynamic segment split of the vector-ALU GEMV (segments that
    // read the same input, with device counts)
    bool dyn;
    unsigned* flags;
    int prof;             // profiling family of this launch (0: none)
};

hipError_t launch_gemv(bool f16, const GemvArgs& a, hipStream_t s);
// Matrix-core form (fp16 weights, cols % 32 == 0, any B up to kMaxBatchMfma).  Partial
// floats of any launch with rows_cap summed over its segments <= max_rows and
// cols <= max_cols.
long long mfma_partial_floats(int B, long long max_rows, int max_cols);
hipError_t launch_gemv_mfma(const GemvArgs& a, float* partial, hipStream_t s);

struct AxpyArgs {
    const void* W;        // [units*rpu, cols] weights
    int cols;
    UnitList list;
    int rpu;
    const float* coef;    // [B, ldc] fp32: coefficient of visited row r of batch b at b*ldc + r
    int ldc;
    int B;
    float* partial;       // [nchunk, B, cols] workspace
    int rows_per_chunk;   // chunk size for the full capacity (LDS is sized for it); with
                          // fewer rows kept the chunks shrink so every chunk has rows
    const float* resid;   // may be nullptr
    float* out;           // [B, cols]
    float2* stats;        // [B, ceil(cols / kLnTile)] (mean, M2) of each slice of out, or nullptr
    // when set, out += the product: each block adds its tile with fp32 atomics (vector-ALU
    // form only): no partial tiles, no finalize launch, no statistics; resid, partial and
    // stats are unused, and the order of the additions (so the last bits of out) depends
    // on scheduling
    bool accumulate;
    // when set, the coefficients are the attention outputs merged here from the
    // split-position partials [B, cap, nchunk, rpu + 2] (rows of a unit = its rpu dims;
    // needs rows_per_chunk <= rpu and nchunk <= kFuseMaxChunks); coef is then unused
    const float* attn_part;
    int attn_nchunk;
    bool mfma;            // matrix-core form (fp16 weights; required above kMaxBatch rows)
    int chunk_step;       // set by the launcher: chunks are multiples of this many rows
    unsigned* flags;
    int prof;
};

hipError_t launch_axpy(bool f16, const AxpyArgs& a, hipStream_t s);
// Chunks of rows for a row-axpy over rows_cap rows (max_rows_per_chunk: 0 = no limit).
int axpy_chunks(int rows_cap, int cols, bool f16, int max_rows_per_chunk, int* rows_per_chunk);
// The same for the matrix-core form (fp16; chunks are multiples of 64 rows).
int axpy_chunks_mfma(int rows_cap, int cols, int* rows_per_chunk);
constexpr int kAxpyMaxChunkRows = 1024;

// Partial (split-position) attention; with merge, also the merge kernel that writes H.
hipError_t launch_attention(bool f16, const AttnArgs& a, bool merge, hipStream_t s);
int attn_chunk_for(bool f16, int dh);  // positions per attention chunk

hipError_t launch_select(const SelectJob* jobs, int njobs, int B, hipStream_t s, int prof);

// Lazy K/V of the heads a step does not select (lazykv.hip): saves the step's attention
// input and recomputes the selected heads' missing K/V from the saved inputs.
struct LazyKvArgs {
    RowInput in;             // the layer's attention input (y ready, x with tile stats, or x whose
                             // moments the save sums itself: own_stats)
    float* Y;                // [B, n_cap, d] saved inputs
    const int32_t* kv_prev;  // [h] positions with valid K/V before this step
    int32_t* kv_next;        // [h] after it
    UnitList heads;          // the selected heads
    const void* Wqkv;        // [h, 3, dh, d]
    void* Kc;                // [B, h, n_cap, dh]
    void* Vc;
    int B, d, h, dh, n, n_cap;
    unsigned* flags;
};
hipError_t launch_lazy_kv(bool f16, const LazyKvArgs& a, hipStream_t s);

hipError_t launch_layernorm(int B, int d, const float* x, float* y, float eps, hipStream_t s);
// (mean, M2) of each kLnTile-column slice of x [B, d].
hipError_t launch_ln_stats(int B, int d, const float* x, float2* stats, hipStream_t s);

unsigned* device_flags();  // this device's flag word (device address), nullptr on error
int device_cus();          // compute units of the current device

// Benchmark hook: events recorded around the launches of one kernel family.
struct ProfHook {
    int family = 0;
    void* const* ev = nullptr;  // 2 * cap hipEvent_t
    int cap = 0;
    int used = 0;
    bool open = false;
};
ProfHook& prof_hook();

inline void prof_begin(int family, hipStream_t s) {
    ProfHook& h = prof_hook();
    if (family != 0 && h.family == family && h.used < h.cap) {
        (void)hipEventRecord(static_cast<hipEvent_t>(h.ev[2 * h.used]), s);
        h.open = true;
    }
}
inline void prof_end(int family, hipStream_t s) {
    ProfHook& h = prof_hook();
    if (h.open && h.family == family) {
        (void)hipEventRecord(static_cast<hipEvent_t>(h.ev[2 * h.used + 1]), s);
        ++h.used;
        h.open = false;
    }
}

}  // namespace djv
