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
// result does not depend on scheduling (no atomics); 16-byte loads, all of a thread's
// chunks in flight together.  It also writes (mean, M2) of every 64-column slice of out, from
// which the next GEMV applies LayerNorm while loading.  The kernel boundary between the
// two is what makes the partial tiles of all XCDs visible; no device-wide fence is used.
// Accumulating form (the lookahead stack's residual stream): each block adds its tile to
// out with fp32 atomics instead, so no partial tiles and no finalize launch; the order of
// the additions, and with it the last bits of out, depends on scheduling, and the consumer
// computes the LayerNorm moments itself.
#include "common.hpp"

namespace djv {
namespace {

// A 16-byte zero vector: loads of absent rows read it, so every weight load is issued
// unconditionally.
static __device__ const Vec16 g_zero16 = {};

constexpr int kUnroll = 8;      // rows in flight per wave
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 256;

// Rows per chunk for the rows actually kept: the launch has one chunk per rows_per_chunk
// rows of the capacity; when the device count is lower (a threshold list, a batch union)
// the rows are spread over all of them in multiples of chunk_step, so every block has work.
__device__ __forceinline__ int chunk_rows(const AxpyArgs& a, int rows) {
    const int rows_cap = a.list.cap * a.rpu;
    const int nch_cap = (rows_cap + a.rows_per_chunk - 1) / a.rows_per_chunk;
    if (nch_cap == 0) return a.rows_per_chunk;  // an empty list (top-k with k = 0): no chunk
    int r = (rows + nch_cap - 1) / nch_cap;
    r = (r + a.chunk_step - 1) / a.chunk_step * a.chunk_step;
    return min(max(r, a.chunk_step), a.rows_per_chunk);
}

// Coefficients of this chunk's rows merged from split-position attention partials: row
// r = u * dh + c (unit slot u, dim c) of batch row b gets
//   sum_ch e^{m_ch - M} acc_ch[c] / sum_ch e^{m_ch - M} l_ch,   M = max_ch m_ch,
// the sums taken in chunk order ([NOTES "Sparsified Attention"]: H_i = D_i^{-1} exp(.) X
// W_i^V, the chunks' maxima cancelling between numerator and D_i).  A chunk of at most dh
// rows touches at most two unit slots; their (m, l) go through LDS first.
//
// The staging of a chunk (row numbers and coefficients, plain or merged) is in two parts:
// stage_load issues the loads of each thread's first row and (m, l) entry, before the
// chunk's first weight requests, and stage_finish, after them, waits for those loads only
// (the vector load counter completes in issue order, so loads issued after the weights
// would also wait for the weights), merges, and fills LDS.
template <int NB>
struct StageRegs {
    static constexpr int kPre = 32 / NB;  // attention chunks whose accumulators are preloaded
    int unit;                             // index entry of this thread's first row (unchecked)
    float cf[NB];                         // its coefficients (plain rows)
    float m, l;                           // entry tid of [b][h][ch] (attention)
    float av[NB][kPre];                   // its row's chunk accumulators (attention)
};

template <int NB>
__device__ __forceinline__ void stage_load(const AxpyArgs& a, int r0, int nr, StageRegs<NB>& R) {
    constexpr int kPre = StageRegs<NB>::kPre;
    const int tid = threadIdx.x;
    // only threads with a row (or an (m, l) entry) load, at clamped (in-range) addresses,
    // and no memory operation with a side effect sits in these branches; stage_finish
    // masks what does not belong to the chunk
    const int r = r0 + min(tid, nr - 1);  // this thread's first row (nr >= 1)
    const int u = r / a.rpu;               // < count <= cap
    const int bmax = a.B - 1;
    if (tid < nr) R.unit = a.list.idx ? a.list.idx[u] : u;
    if (a.attn_part) {
        const int dh = a.rpu, nck = a.attn_nchunk, cap = a.list.cap;
        const int u0 = r0 / dh;
        const size_t stride = (size_t)dh + 2;
        if (tid < NB * 2 * nck) {  // entry [b][h][ch]
            const int ch = tid % nck, h = (tid / nck) % 2, b = min(tid / (2 * nck), bmax);
            const float* pm = a.attn_part + (((size_t)b * cap + min(u0 + h, cap - 1)) * nck + ch) * stride;
            R.m = pm[0];
            R.l = pm[1];
        }
        if (nck <= kPre && tid < nr) {
            const int c = r - u * dh;
#pragma unroll
            for (int b2 = 0; b2 < NB; ++b2) {
                const float* pp = a.attn_part + ((size_t)min(b2, bmax) * cap + u) * nck * stride + 2 + c;
#pragma unroll
                for (int k = 0; k < kPre; ++k) R.av[b2][k] = pp[(size_t)min(k, nck - 1) * stride];
            }
        }
    } else if (tid < nr) {
#pragma unroll
        for (int b = 0; b < NB; ++b) R.cf[b] = a.coef[(size_t)min(b, bmax) * a.ldc + r];
    }
}

template <int NB>
__device__ __forceinline__ void stage_finish(const AxpyArgs& a, int r0, int nr, const StageRegs<NB>& R,
                                             float* cf_s, int* row_s, float* dyn_attn) {
    constexpr int kPre = StageRegs<NB>::kPre;
    const int tid = threadIdx.x;
    // the first row's unit, checked as unit_of checks it
    int unit = tid < nr ? R.unit : -1;
    if (tid < nr && a.list.idx && (unit < 0 || unit >= a.list.units)) {
        set_flag(a.flags, kFlagBadIndex);
        unit = -1;
    }
    if (!a.attn_part) {
        if (tid < nr) {
            const int r = r0 + tid;
            row_s[tid] = unit < 0 ? -1 : unit * a.rpu + (r - (r / a.rpu) * a.rpu);
#pragma unroll
            for (int b = 0; b < NB; ++b) cf_s[b * a.rows_per_chunk + tid] = (unit >= 0 && b < a.B) ? R.cf[b] : 0.f;
        }
        for (int i = tid + kThreads; i < nr; i += kThreads) {
            const int r = r0 + i;
            const int u = r / a.rpu, sub = r - u * a.rpu;
            const int unit = unit_of(a.list, u, a.flags);
            row_s[i] = unit < 0 ? -1 : unit * a.rpu + sub;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                cf_s[b * a.rows_per_chunk + i] = (unit >= 0 && b < a.B) ? a.coef[(size_t)b * a.ldc + r] : 0.f;
        }
        return;
    }
    const int dh = a.rpu, nck = a.attn_nchunk, cap = a.list.cap;
    const int u0 = r0 / dh;
    const int nh = (r0 + nr - 1) / dh - u0 + 1;  // 1 or 2
    const size_t stride = (size_t)dh + 2;
    float* wm = dyn_attn;
    float* wl = wm + NB * 2 * nck;
    float* inv = wl + NB * 2 * nck;
    if (tid < NB * 2 * nck) {
        const int h = (tid / nck) % 2, b = tid / (2 * nck);
        const bool ok = b < a.B && h < nh;
        wm[tid] = ok ? R.m : -INFINITY;
        wl[tid] = ok ? R.l : 0.f;
    }
    for (int i = tid + kThreads; i < NB * 2 * nck; i += kThreads) {
        const int ch = i % nck, h = (i / nck) % 2, b = i / (2 * nck);
        float m = -INFINITY, l = 0.f;
        if (b < a.B && h < nh) {
            const float* pp = a.attn_part + (((size_t)b * cap + u0 + h) * nck + ch) * stride;
            m = pp[0];
            l = pp[1];
        }
        wm[i] = m;
        wl[i] = l;
    }
    __syncthreads();
    if (tid < NB * 2) {
        // one thread per (b, h): chunk weights in place and the denominator, in chunk order
        float* m = wm + tid * nck;
        const float* l = wl + tid * nck;
        float M = -INFINITY;
        for (int ch = 0; ch < nck; ++ch) M = fmaxf(M, m[ch]);
        float L = 0.f;
        for (int ch = 0; ch < nck; ++ch) {
            m[ch] = __expf(m[ch] - M);
            L = fmaf(l[ch], m[ch], L);
        }
        inv[tid] = L;
    }
    __syncthreads();
    if (nck <= kPre) {
        // the preloaded accumulators of this thread's row
        if (tid < nr) {
            const int r = r0 + tid;
            const int u = r / dh, c = r - u * dh, h = u - u0;
            row_s[tid] = unit < 0 ? -1 : unit * dh + c;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float v = 0.f;
                if (unit >= 0 && b < a.B) {
                    const float* w = wm + (b * 2 + h) * nck;
                    float acc = 0.f;
#pragma unroll
                    for (int k = 0; k < kPre; ++k)
                        if (k < nck) acc = fmaf(R.av[b][k], w[k], acc);
                    v = acc / inv[b * 2 + h];
                }
                cf_s[b * a.rows_per_chunk + tid] = v;
            }
        }
        return;
    }
    for (int i = tid; i < nr; i += kThreads) {
        const int r = r0 + i;
        const int u = r / dh, c = r - u * dh, h = u - u0;
        const int unit = unit_of(a.list, u, a.flags);
        row_s[i] = unit < 0 ? -1 : unit * dh + c;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float v = 0.f;
            if (unit >= 0 && b < a.B) {
                const float* pp = a.attn_part + ((size_t)b * cap + u) * nck * stride + 2 + c;
                const float* w = wm + (b * 2 + h) * nck;
                float acc = 0.f;
                int ch = 0;
                for (; ch + 8 <= nck; ch += 8) {
                    float av[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) av[k] = pp[(size_t)(ch + k) * stride];
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc = fmaf(av[k], w[ch + k], acc);
                }
                for (; ch < nck; ++ch) acc = fmaf(pp[(size_t)ch * stride], w[ch], acc);
                v = acc / inv[b * 2 + h];
            }
            cf_s[b * a.rows_per_chunk + i] = v;
        }
    }
}

template <typename T, int NB, bool ACC>
__global__ __launch_bounds__(kThreads) void axpy_partial_kernel(AxpyArgs a) {
    constexpr int E = WTraits<T>::kPerVec;
    constexpr int TC = kWave * E;                       // columns per tile
    // dynamic LDS: [NB][rpc] coefficients, [rpc] rows, then (merged attention) the
    // [NB][2][nchunk] chunk maxima / weights and sums, and [NB][2] denominators
    extern __shared__ float dyn[];
    // the waves' tile sums: waves 1..3 (wave 0 adds them to its own), or (ACC) all four
    __shared__ float red[ACC ? kWavesPerBlock : kWavesPerBlock - 1][NB][TC];

    const int tid = threadIdx.x, wv = tid / kWave, ln = tid % kWave;
    const int chunk = blockIdx.y;
    const int nvec = a.cols / E;
    const int v = blockIdx.x * kWave + ln;              // this lane's column vector
    const bool col_ok = v < nvec;
    const int count = read_count_uniform(a.list, a.flags);
    const int rows = count * a.rpu;
    const int rpc = chunk_rows(a, rows);
    const int r0 = chunk * rpc;
    if (r0 >= rows) return;
    const int nr = min(rows, r0 + rpc) - r0;
    float* cf_s = dyn;
    int* row_s = reinterpret_cast<int*>(dyn + NB * a.rows_per_chunk);
    const char* Wb = reinterpret_cast<const char*>(a.W);
    const size_t row_bytes = (size_t)a.cols * sizeof(T);

    // the staging loads first, then the wave's first kUnroll rows (uniform over the wave:
    // scalar index loads), whose latency overlaps the rest of the staging (and the
    // attention merge)
    StageRegs<NB> sr;
    stage_load<NB>(a, r0, nr, sr);
    // (unconditional: an absent row reads a static zero vector, and a bad index is flagged
    // by the staging's check of the same rows, so no branch with a memory operation sits
    // between the staging loads and their use, which would make the compiler wait for all
    // loads in flight there)
    Vec16 w0[kUnroll];
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    gchar* zero = reinterpret_cast<gchar*>(reinterpret_cast<uint64_t>(&g_zero16));
    gchar* Wg = reinterpret_cast<gchar*>(reinterpret_cast<uint64_t>(Wb));
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
        const int i = wvu + q * kWavesPerBlock;
        int row = -1;
        if (i < nr) {
            const int r = r0 + i;
            const int u = r / a.rpu, sub = r - u * a.rpu;
            const int unit = a.list.idx ? sload_i32(a.list.idx + u) : u;
            row = (unit < 0 || unit >= a.list.units) ? -1 : unit * a.rpu + sub;
        }
        const bool have = row >= 0 && col_ok;
        w0[q] = ldg16_nt_at(have ? Wg + (size_t)row * row_bytes + (size_t)v * 16 : zero, 0u);
    }

    stage_finish<NB>(a, r0, nr, sr, cf_s, row_s, dyn + (NB + 1) * a.rows_per_chunk);
    __syncthreads();

    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;
    auto consume = [&](const Vec16 (&w)[kUnroll], int i0) {
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
    };
    consume(w0, wv);
    for (int i0 = wv + kWavesPerBlock * kUnroll; i0 < nr; i0 += kWavesPerBlock * kUnroll) {
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
        consume(w, i0);
    }

    if constexpr (ACC) {
        // out += the tile: the four waves' sums through LDS, then each thread adds columns
        // tid, tid + 256, ... (one atomic instruction per 64 consecutive columns)
        if (col_ok) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) red[wv][b][ln * E + e] = acc[b][e];
        }
        __syncthreads();
        const int c0 = blockIdx.x * TC;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b >= a.B) break;
            float* dst = a.out + (size_t)b * a.cols + c0;
#pragma unroll
            for (int c = tid; c < TC; c += kThreads) {
                if (c0 + c < a.cols) {
                    float t = red[0][b][c];
#pragma unroll
                    for (int q = 1; q < kWavesPerBlock; ++q) t += red[q][b][c];
                    unsafeAtomicAdd(dst + c, t);
                }
            }
        }
        return;
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
// the slice's (mean, M2).  Block (slice, b) of 256 threads: thread (g, q) loads float4 q
// of the slice from chunks g, g+16, g+32, ... (all its loads in one round), the 16 group
// sums are added in order through LDS, and one wave finishes the slice.
constexpr int kFinGroups = 16;
constexpr int kFinQuads = kLnTile / 4;   // float4 per 64-column slice
constexpr int kFinBatch = 4;             // loads per thread in flight (chunks <= 64 in one round)

__global__ __launch_bounds__(kFinGroups * kFinQuads) void axpy_finalize_kernel(AxpyArgs a) {
    __shared__ float red[kFinGroups][kLnTile + 4];
    const int slice = blockIdx.x, b = blockIdx.y;
    const int g = threadIdx.x / kFinQuads, q = threadIdx.x % kFinQuads;
    const int c0 = slice * kLnTile;
    const int ncols = min(kLnTile, a.cols - c0);
    const int count = read_count(a.list, nullptr);
    const int rows = count * a.rpu;
    const int rpc = chunk_rows(a, rows);
    const int nch = (rows + rpc - 1) / rpc;
    const size_t plane = (size_t)a.B * a.cols;
    // a whole float4 inside the row, or (ragged last slice) a clamped one whose sum is unused
    const bool q_ok = 4 * q + 4 <= ncols;
    const float* p = a.partial + (size_t)b * a.cols + c0 + (q_ok ? 4 * q : 0);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ch0 = g; ch0 < nch; ch0 += kFinGroups * kFinBatch) {
        float4 t[kFinBatch];
#pragma unroll
        for (int k = 0; k < kFinBatch; ++k) {
            const int cc = min(ch0 + k * kFinGroups, nch - 1);
            t[k] = *reinterpret_cast<const float4*>(p + (size_t)cc * plane);
        }
#pragma unroll
        for (int k = 0; k < kFinBatch; ++k) {
            if (ch0 + k * kFinGroups < nch) {
                s.x += t[k].x; s.y += t[k].y; s.z += t[k].z; s.w += t[k].w;
            }
        }
    }
    red[g][4 * q + 0] = s.x;
    red[g][4 * q + 1] = s.y;
    red[g][4 * q + 2] = s.z;
    red[g][4 * q + 3] = s.w;
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    const int c = threadIdx.x;
    const bool ok = c < ncols;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kFinGroups; ++k) v += red[k][c];
    const size_t o = (size_t)b * a.cols + c0 + c;
    if (ok && a.resid) v += a.resid[o];
    if (ok) a.out[o] = v;
    if (a.stats) {
        const float mean = wave_sum(ok ? v : 0.f) / (float)ncols;
        const float dv = ok ? v - mean : 0.f;
        const float M2 = wave_sum(dv * dv);
        if (c == 0) a.stats[(size_t)b * gridDim.x + slice] = make_float2(mean, M2);
    }
}

// ---------------------------------------------------------------------------------
// Matrix-core form (fp16 weights; batches of more than kMaxBatch rows, or smaller ones on
// request): the same partial tiles, computed on the matrix cores.  D[b, c] = sum_r
// coef[b, r] W[r, c] over the block's rows is v_mfma_f32_16x16x32_f16 with A =
// coefficients (rounded to fp16) and B = weights.  The instruction wants 8 consecutive k
// (here: rows) per lane for one column, while a weight row is contiguous in columns, so
// the weights go through LDS: coalesced 16-byte row loads in, 16-bit column reads out.
//
// A block (4 waves) owns kAxCols = 512 columns, 128 per wave (8 column tiles of 16), and a
// chunk of rows taken kAxGroup = 32 at a time: the group's weight tile (32 KiB) and its
// coefficients sit in LDS while the next group's loads are already in registers.  One
// coefficient fragment feeds the wave's eight column tiles; one weight fragment feeds the
// BT batch tiles.  Each load instruction reads a 1 KiB run of one row: with 256-column
// tiles (512-byte runs, the other pieces of each gathered row read by other blocks at other
// times) the launch ran about 11% slower at batches 16 and 32.
// ---------------------------------------------------------------------------------
typedef _Float16 h8m_t __attribute__((ext_vector_type(8)));
typedef float f4m_t __attribute__((ext_vector_type(4)));
constexpr int kAxCols = 512;                  // columns per block
constexpr int kAxK = 32;                      // rows per MFMA
constexpr int kAxTiles = kAxCols / 4 / 16;    // 16-column tiles per wave
constexpr int kAxGroup = kAxK;                // rows staged per round
constexpr int kAxPitch = kAxCols + 4;         // halfs per LDS weight row (8-byte aligned rows)
constexpr int kAxCfPitch = kAxGroup + 8;      // halfs per LDS coefficient row
constexpr int kAxLoads = kAxGroup * kAxCols * 2 / 16 / kThreads;  // 16-byte loads per thread per round
constexpr int kAxTargetBlocks = 768;          // about three per compute unit (a constant, so that
                                              // workspace sizes do not depend on the device)


template <int BT>
__global__ __launch_bounds__(kThreads) void axpy_mfma_kernel(AxpyArgs a) {
    constexpr int BP = BT * 16;
    __shared__ _Float16 wt[kAxGroup][kAxPitch];
    __shared__ _Float16 cf[BP][kAxCfPitch];
    extern __shared__ int row_s[];  // [rows_per_chunk] weight row of each chunk row (-1: none)
    const int tid = threadIdx.x, wv = tid / kWave, l = tid % kWave;
    const int chunk = blockIdx.y;
    const int c0 = blockIdx.x * kAxCols;
    const int count = read_count(a.list, a.flags);
    const int rows = count * a.rpu;
    const int rpc = chunk_rows(a, rows);
    const int r0 = chunk * rpc;
    if (r0 >= rows) return;
    const int nr = min(rows, r0 + rpc) - r0;
    for (int i = tid; i < a.rows_per_chunk; i += kThreads) {
        int row = -1;
        if (i < nr) {
            const int r = r0 + i;
            const int u = r / a.rpu, sub = r - u * a.rpu;
            const int unit = unit_of(a.list, u, a.flags);
            row = unit < 0 ? -1 : unit * a.rpu + sub;
        }
        row_s[i] = row;
    }
    __syncthreads();

    // weight loads: thread t moves columns 8 (t % 64) .. + 8 of rows t / 64 + 4 q (one 1 KiB
    // run of a row per load instruction)
    const int lc = 8 * (tid % 64), lr = tid / 64;
    const bool col_ok = c0 + lc + 8 <= a.cols;
    const char* Wb = reinterpret_cast<const char*>(a.W);
    const size_t row_bytes = (size_t)a.cols * 2;
    // coefficient loads: thread t moves batch row t / 4, group rows 8 (t % 4) .. + 8
    const int cb = tid / 4, cr = 8 * (tid % 4);
    const int ngroups = (nr + kAxGroup - 1) / kAxGroup;

    Vec16 wreg[kAxLoads];
    float creg[8];
    auto load_group = [&](int g) {
#pragma unroll
        for (int q = 0; q < kAxLoads; ++q) {
            const int i = g * kAxGroup + lr + 4 * q;
            const int row = i < nr ? row_s[i] : -1;
            const char* p = (row >= 0 && col_ok) ? Wb + (size_t)row * row_bytes + (size_t)(c0 + lc) * 2
                                                 : reinterpret_cast<const char*>(&g_zero16);
            // a global (not flat) load: flat loads also count on lgkmcnt, so every LDS wait
            // below would wait for them too
            wreg[q] = ldg16_nt_at(reinterpret_cast<gchar*>(reinterpret_cast<uint64_t>(p)), 0);
        }
        if (cb < BP) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = g * kAxGroup + cr + e;
                creg[e] = (cb < a.B && i < nr && row_s[i] >= 0) ? a.coef[(size_t)cb * a.ldc + r0 + i] : 0.f;
            }
        }
    };

    f4m_t acc[kAxTiles][BT];
#pragma unroll
    for (int j = 0; j < kAxTiles; ++j)
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[j][t] = f4m_t{0.f, 0.f, 0.f, 0.f};
    const int kb = 8 * (l / 16), cl = wv * (16 * kAxTiles) + l % 16;

    load_group(0);
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
        for (int q = 0; q < kAxLoads; ++q) {
            // two 8-byte stores: rows are 8-byte aligned in LDS
            uint2* dst = reinterpret_cast<uint2*>(&wt[lr + 4 * q][lc]);
            dst[0] = make_uint2(wreg[q].w[0], wreg[q].w[1]);
            dst[1] = make_uint2(wreg[q].w[2], wreg[q].w[3]);
        }
        if (cb < BP) {
            h8m_t hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = (_Float16)creg[e];
            *reinterpret_cast<h8m_t*>(&cf[cb][cr]) = hv;
        }
        __syncthreads();
        if (g + 1 < ngroups) load_group(g + 1);
#pragma unroll
        for (int s = 0; s < kAxGroup / kAxK; ++s) {
            h8m_t av[BT];
#pragma unroll
            for (int t = 0; t < BT; ++t) av[t] = *reinterpret_cast<const h8m_t*>(&cf[16 * t + l % 16][s * kAxK + kb]);
#pragma unroll
            for (int j = 0; j < kAxTiles; ++j) {
                h8m_t bw;
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[e] = wt[s * kAxK + kb + e][cl + 16 * j];
#pragma unroll
                for (int t = 0; t < BT; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t], bw, acc[j][t], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // lane l holds D[b = 16 t + 4 (l / 16) + q][column c0 + cl + 16 j]
#pragma unroll
    for (int j = 0; j < kAxTiles; ++j) {
        const int c = c0 + cl + 16 * j;
        if (c >= a.cols) continue;
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int b = 16 * t + 4 * (l / 16) + q;
                if (b < a.B) a.partial[((size_t)chunk * a.B + b) * a.cols + c] = acc[j][t][q];
            }
    }
}

template <typename T>
hipError_t dispatch_mfma(const AxpyArgs& args, hipStream_t s) {
    AxpyArgs a = args;
    a.chunk_step = kAxGroup;
    if (a.B < 1 || a.B > kMaxBatchMfma || a.attn_part || a.rows_per_chunk % kAxGroup != 0)
        return hipErrorInvalidValue;
    const int rows_cap = a.list.cap * a.rpu;
    const int nch = rows_cap > 0 ? (rows_cap + a.rows_per_chunk - 1) / a.rows_per_chunk : 0;
    if (nch > 0) {
        const size_t dyn = (size_t)a.rows_per_chunk * sizeof(int);
        dim3 grid((a.cols + kAxCols - 1) / kAxCols, nch);
        prof_begin(a.prof, s);
        if (a.B <= 16) hipLaunchKernelGGL(axpy_mfma_kernel<1>, grid, dim3(kThreads), dyn, s, a);
        else hipLaunchKernelGGL(axpy_mfma_kernel<2>, grid, dim3(kThreads), dyn, s, a);
        prof_end(a.prof, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 fgrid((a.cols + kLnTile - 1) / kLnTile, a.B);
    hipLaunchKernelGGL(axpy_finalize_kernel, fgrid, dim3(kFinGroups * kFinQuads), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const AxpyArgs& args, hipStream_t s) {
    if (args.mfma) {
        if constexpr (sizeof(T) == 2) {
            if (args.accumulate) return hipErrorInvalidValue;
            return dispatch_mfma<T>(args, s);
        } else {
            return hipErrorInvalidValue;
        }
    }
    AxpyArgs a = args;
    a.chunk_step = kWavesPerBlock * kUnroll;
    if (a.B > kMaxBatch) return hipErrorInvalidValue;
    constexpr int E = WTraits<T>::kPerVec;
    const int tiles = (a.cols / E + kWave - 1) / kWave;
    const int rows_cap = a.list.cap * a.rpu;
    const int nch = rows_cap > 0 ? (rows_cap + a.rows_per_chunk - 1) / a.rows_per_chunk : 0;
    if (nch > 0) {
        const int nb = a.B <= 1 ? 1 : (a.B <= 2 ? 2 : 4);
        size_t dyn = (size_t)a.rows_per_chunk * (nb * sizeof(float) + sizeof(int));
        if (a.attn_part) {
            if (a.attn_nchunk < 1 || a.attn_nchunk > kFuseMaxChunks || a.rows_per_chunk > a.rpu)
                return hipErrorInvalidValue;
            dyn += ((size_t)nb * 2 * a.attn_nchunk * 2 + (size_t)nb * 2) * sizeof(float);
        }
        dim3 grid(tiles, nch);
        prof_begin(a.prof, s);
        if (a.accumulate) {
            if (nb == 1) hipLaunchKernelGGL((axpy_partial_kernel<T, 1, true>), grid, dim3(kThreads), dyn, s, a);
            else if (nb == 2) hipLaunchKernelGGL((axpy_partial_kernel<T, 2, true>), grid, dim3(kThreads), dyn, s, a);
            else hipLaunchKernelGGL((axpy_partial_kernel<T, 4, true>), grid, dim3(kThreads), dyn, s, a);
        } else {
            if (nb == 1) hipLaunchKernelGGL((axpy_partial_kernel<T, 1, false>), grid, dim3(kThreads), dyn, s, a);
            else if (nb == 2) hipLaunchKernelGGL((axpy_partial_kernel<T, 2, false>), grid, dim3(kThreads), dyn, s, a);
            else hipLaunchKernelGGL((axpy_partial_kernel<T, 4, false>), grid, dim3(kThreads), dyn, s, a);
        }
        prof_end(a.prof, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.accumulate) return hipSuccess;
    dim3 fgrid((a.cols + kLnTile - 1) / kLnTile, a.B);
    hipLaunchKernelGGL(axpy_finalize_kernel, fgrid, dim3(kFinGroups * kFinQuads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int axpy_chunks_mfma(int rows_cap, int cols, int* rows_per_chunk) {
    // about kAxTargetBlocks blocks over the column tiles and row chunks; chunks are whole
    // staging rounds of kAxGroup rows, at most kAxpyMaxChunkRows
    const int tiles = (cols + kAxCols - 1) / kAxCols;
    const int step = kAxGroup;
    if (rows_cap <= 0) {
        *rows_per_chunk = step;
        return 0;
    }
    int chunks = (kAxTargetBlocks + tiles - 1) / tiles;
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

int axpy_chunks(int rows_cap, int cols, bool f16, int max_rows_per_chunk, int* rows_per_chunk) {
    const int E = f16 ? 8 : 4;
    const int tiles = (cols / E + kWave - 1) / kWave;  // 512-column tiles
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
    if (max_rows_per_chunk > 0 && rpc > max_rows_per_chunk) rpc = max_rows_per_chunk;
    *rows_per_chunk = rpc;
    return (rows_cap + rpc - 1) / rpc;
}

hipError_t launch_axpy(bool f16, const AxpyArgs& a, hipStream_t s) {
    return f16 ? dispatch<__half>(a, s) : dispatch<float>(a, s);
}

}  // namespace djv
