// C ABI of libdejavu: argument validation, workspace layout and kernel sequencing.
//
// Every entry point validates all of its arguments before the first HIP call, so each
// error path can be exercised on a machine without a GPU.  Kernels are enqueued on the
// caller's stream; nothing here allocates device memory or synchronises (except
// dejavu_poll_device_error).
#include "dejavu.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <initializer_list>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "common.hpp"

using namespace djv;

namespace djv {
// gather.hip: kept rows copied to a contiguous buffer (the unfused gather of the fusion
// ablation); row_bytes a multiple of 2.
hipError_t launch_gather_rows(const void* W, void* out, const UnitList& list, int rpu, size_t row_bytes,
                              unsigned* flags, hipStream_t s);
// norms.hip: scores[u] = sqrt(sum over b and c of v[b, u, c]^2), v [B, units, w] fp32.
hipError_t launch_unit_norms(const float* v, int B, int units, int w, float* scores, hipStream_t s);
// misc.hip: plain streaming read of `bytes` (a multiple of 16) from buf.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);
}  // namespace djv

namespace {

thread_local std::string g_err;

djv_status fail(djv_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define DJV_REQUIRE(cond, status, ...)                 \
    do {                                               \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define DJV_TRY(expr)                                  \
    do {                                               \
        djv_status s_ = (expr);                        \
        if (s_ != DJV_OK) return s_;                   \
    } while (0)

#define DJV_HIP(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return fail(DJV_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// ------------------------------------------------------------------------------------
// Static scratch of dejavu_sparse_mlp_no_alloc, for callers that cannot allocate.  Each
// GPU the library runs on holds its own copy of `scratch` until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device (with that device current) and only that address is ever passed
// to kernels.  Calls share their GPU's copy and leave its contents to the next call, so
// calls that overlap on one GPU race.
// ------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = DJV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`.
djv_status static_scratch(void** out) {
    int dev = -1;
    DJV_HIP(hipGetDevice(&dev));
    DJV_REQUIRE(dev >= 0 && dev < kMaxDevices, DJV_EUNSUPPORTED, "device %d: at most %d devices", dev,
                kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        DJV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        DJV_REQUIRE(p != nullptr, DJV_EHIP, "hipGetSymbolAddress(scratch) gave no address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DJV_OK;
}

constexpr int kMaxSelect = 65536;
constexpr int kMaxRowBytes = kMaxRowVecs * 16;  // one row: 256 threads x 8 vectors of 16 bytes

size_t esize(int wt) { return wt == DJV_F16 ? 2 : 4; }
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
int words_of(int n) { return (n + 31) / 32; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

djv_status check_dtype(int wt) {
    DJV_REQUIRE(wt == DJV_F32 || wt == DJV_F16, DJV_EINVAL, "dtype must be DJV_F32 or DJV_F16 (got %d)", wt);
    return DJV_OK;
}
djv_status check_batch(int B) {
    DJV_REQUIRE(B >= 1, DJV_EINVAL, "B must be >= 1 (got %d)", B);
    DJV_REQUIRE(B <= DJV_MAX_BATCH, DJV_EUNSUPPORTED, "B = %d exceeds the library's limit %d", B, DJV_MAX_BATCH);
    return DJV_OK;
}
// Batches above kMaxBatch run on the matrix cores: fp16 weights, and every GEMV row length
// a multiple of the instruction's k (32).
djv_status check_wide_batch(int B, int wt, std::initializer_list<int> cols) {
    if (B <= kMaxBatch) return DJV_OK;
    DJV_REQUIRE(wt == DJV_F16, DJV_EUNSUPPORTED, "B = %d > %d needs fp16 weights", B, kMaxBatch);
    for (int c : cols)
        DJV_REQUIRE(c % 32 == 0, DJV_EUNSUPPORTED, "B = %d > %d needs row lengths that are multiples of 32 (got %d)",
                    B, kMaxBatch, c);
    return DJV_OK;
}
djv_status check_rowlen(int cols, int wt, const char* name) {
    DJV_REQUIRE(cols > 0, DJV_EINVAL, "%s must be > 0 (got %d)", name, cols);
    DJV_REQUIRE(cols % 8 == 0, DJV_EINVAL, "%s must be a multiple of 8 (got %d)", name, cols);
    DJV_REQUIRE((size_t)cols * esize(wt) <= (size_t)kMaxRowBytes, DJV_EUNSUPPORTED,
                "%s = %d: rows above %d bytes are not supported", name, cols, kMaxRowBytes);
    return DJV_OK;
}
djv_status check_ptr(const void* p, const char* name) {
    DJV_REQUIRE(p != nullptr, DJV_EINVAL, "%s is NULL", name);
    DJV_REQUIRE(aligned(p, 16), DJV_EALIGN, "%s is not 16-byte aligned", name);
    return DJV_OK;
}
djv_status check_opt_ptr(const void* p, const char* name) {
    if (!p) return DJV_OK;
    DJV_REQUIRE(aligned(p, 16), DJV_EALIGN, "%s is not 16-byte aligned", name);
    return DJV_OK;
}
djv_status check_idx_ptr(const void* p, const char* name) {
    DJV_REQUIRE(p != nullptr, DJV_EINVAL, "%s is NULL", name);
    DJV_REQUIRE(aligned(p, 4), DJV_EALIGN, "%s is not 4-byte aligned", name);
    return DJV_OK;
}
djv_status check_select(int n_out, int mode, int k, float t, const char* what) {
    DJV_REQUIRE(n_out >= 1, DJV_EINVAL, "%s: n_out must be >= 1 (got %d)", what, n_out);
    DJV_REQUIRE(n_out <= kMaxSelect, DJV_EUNSUPPORTED, "%s: n_out = %d exceeds %d", what, n_out, kMaxSelect);
    DJV_REQUIRE(mode == DJV_TOPK || mode == DJV_THRESHOLD, DJV_EINVAL, "%s: unknown mode %d", what, mode);
    if (mode == DJV_TOPK)
        DJV_REQUIRE(k >= 0 && k <= n_out, DJV_EINVAL, "%s: k = %d outside [0, %d]", what, k, n_out);
    else
        DJV_REQUIRE(t > 0.f && t < 1.f, DJV_EINVAL, "%s: t must lie in (0, 1)", what);
    return DJV_OK;
}
djv_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return DJV_OK;
    DJV_REQUIRE(ws != nullptr, DJV_EINVAL, "workspace is NULL (%zu bytes needed)", need);
    DJV_REQUIRE(aligned(ws, 256), DJV_EALIGN, "workspace is not 256-byte aligned");
    DJV_REQUIRE(ws_bytes >= need, DJV_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return DJV_OK;
}

// Order-preserving key of an fp32 score (same map as the selection kernel).
uint32_t score_key_host(float z) {
    uint32_t u;
    std::memcpy(&u, &z, 4);
    if (z != z) u = 0xFF800000u;
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
uint32_t tau_key(float t) {
    const double td = (double)t;
    const float tau = (float)std::log(td / (1.0 - td));
    return score_key_host(tau);
}

// Batches of at least this many rows use the matrix-core kernels where they can (fp16
// weights, row lengths divisible by 32); batches above kMaxBatch always do.
std::atomic<int> g_mfma_min_batch{kMaxBatch + 1};
// When set, the lookahead stack keeps its finalize launches (bitwise reproducible).
std::atomic<int> g_deterministic{0};

bool wide_possible(int wt, std::initializer_list<int> cols) {
    if (wt != DJV_F16) return false;
    for (int c : cols)
        if (c % 32 != 0) return false;
    return true;
}
bool layer_wide(const djv_model& m) { return wide_possible(m.wt, {m.d, m.r}); }

// ------------------------------------------------------------------------------------
// Workspace plans.  The same functions size the workspace (base == nullptr) and carve
// it, so a size query and a call always agree.
// ------------------------------------------------------------------------------------
struct Arena {
    char* base;
    size_t off = 0;
    explicit Arena(void* b) : base(static_cast<char*>(b)) {}
    template <typename T> T* take(size_t n) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += al256(n * sizeof(T));
        return p;
    }
};

// Scratch of the matrix-core GEMV: its k-slice partials, sized for the largest launch a
// plan makes (rows summed over the launch's segments, longest row).  `on` selects the
// matrix-core form for every launch of a call; the scratch is reserved whenever the form
// is possible (fp16 weights, row lengths divisible by 32), so a workspace size never
// depends on the batch threshold in force.
struct MfmaWs { float* part; bool on; bool reserved; };
MfmaWs plan_mfma(Arena& A, bool possible, int B, long long max_rows, int max_cols) {
    MfmaWs w{nullptr, false, false};
    if (!possible) return w;
    w.reserved = true;
    w.part = A.take<float>((size_t)mfma_partial_floats(B, max_rows, max_cols));
    w.on = B > kMaxBatch || B >= g_mfma_min_batch.load(std::memory_order_relaxed);
    return w;
}

struct PredWs { float* u; float* z; uint32_t* bits; MfmaWs mf; };
PredWs plan_predict(Arena& A, int B, int d, int r, int n_out, bool need_z, bool wide,
                    const MfmaWs* shared = nullptr) {
    PredWs w;
    w.u = A.take<float>((size_t)B * r);
    w.z = need_z ? A.take<float>((size_t)B * n_out) : nullptr;
    w.bits = A.take<uint32_t>((size_t)B * words_of(n_out));
    w.mf = shared ? *shared : plan_mfma(A, wide, B, std::max(r, n_out), std::max(d, r));
    return w;
}

struct MlpWs { float* a; float* partial; int rpc; MfmaWs mf; };
MlpWs plan_mlp(Arena& A, int B, int d, int cap, bool f16, bool wide, const MfmaWs* shared = nullptr) {
    MlpWs w;
    w.a = A.take<float>((size_t)B * (cap > 0 ? cap : 1));
    int nch = axpy_chunks(cap, d, f16, 0, &w.rpc);
    w.mf = shared ? *shared : plan_mfma(A, wide, B, cap, d);
    if (w.mf.reserved) {
        // room for either form's chunks; the rows per chunk of the form in use
        int rpc_m = 0;
        nch = std::max(nch, axpy_chunks_mfma(cap, d, &rpc_m));
        if (w.mf.on) w.rpc = rpc_m;
    }
    w.partial = A.take<float>((size_t)nch * B * d);
    return w;
}

// fused: the O-projection merges the attention chunks itself (no merge kernel, no H);
// possible when a head has at most kFuseMaxChunks chunks, with chunks of at most dh rows.
struct MhaWs { float* q; float* part; float* H; float* partial; int rpc, chunk, nchunk_max; bool fused; MfmaWs mf; };
MhaWs plan_mha(Arena& A, int B, int d, int dh, int cap, int n_cap, bool f16, bool wide,
              const MfmaWs* shared = nullptr) {
    MhaWs w;
    const int c = cap > 0 ? cap : 1;
    w.mf = shared ? *shared : plan_mfma(A, wide, B, (long long)cap * 3 * dh, d);
    w.chunk = attn_chunk_for(f16, dh);
    w.nchunk_max = (n_cap + w.chunk - 1) / w.chunk;
    w.fused = w.nchunk_max <= kFuseMaxChunks && !w.mf.on;
    w.q = A.take<float>((size_t)B * c * dh);
    w.part = A.take<float>((size_t)B * c * w.nchunk_max * (dh + 2));
    w.H = A.take<float>((size_t)B * c * dh);
    // room for the chunks of every form the threshold may pick (vector ALU fused or not,
    // matrix cores); the rows per chunk of the form in use
    const bool can_fuse = w.nchunk_max <= kFuseMaxChunks;
    int nch = axpy_chunks(cap * dh, d, f16, w.fused ? dh : 0, &w.rpc);
    if (w.mf.reserved) {
        int rpc_v = 0, rpc_m = 0;
        nch = std::max(nch, axpy_chunks(cap * dh, d, f16, can_fuse ? dh : 0, &rpc_v));
        nch = std::max(nch, axpy_chunks_mfma(cap * dh, d, &rpc_m));
        if (w.mf.on) w.rpc = rpc_m;
    }
    w.partial = A.take<float>((size_t)nch * B * d);
    return w;
}

// Capacity of a selected list: top-k keeps k per token, so a batch's union holds at most
// min(n, B*k) units; a threshold can keep all n.
int cap_of(int mode, int k, int n, int B) {
    if (mode != DJV_TOPK) return n;
    const long long c = (long long)k * B;
    return c < n ? (int)c : n;
}

// A tensor-parallel shard of a model: its predictors score all heads / neurons and select
// among them; its weights, caches and lists cover its own range (h heads from h_offset,
// N neurons from N_offset).  Unsharded: the range is everything.
int heads_total(const djv_model& m) { return m.h_total > 0 ? m.h_total : m.h; }
int neurons_total(const djv_model& m) { return m.N_total > 0 ? m.N_total : m.N; }
bool sharded(const djv_model& m) { return m.h_total > 0 || m.N_total > 0; }
int capA_of(const djv_model& m) { return std::min(cap_of(m.mode, m.k_A, heads_total(m), m.B), m.h); }
int capM_of(const djv_model& m) { return std::min(cap_of(m.mode, m.k_M, neurons_total(m), m.B), m.N); }

// Activation state and scratch of a layer or a stack of layers.
struct LayerWs {
    float* xs[2];                     // residual-stream ring: inputs of layers 1..L-1
    float2* sx[2];                    // LayerNorm tile statistics of xs[i]
    float2* s_in;                     // statistics of the caller's x (layer 0 input)
    float* xm;                        // x' = x + attention
    float2* sm;                       // statistics of x'
    int32_t* idxA[2]; int32_t* cntA[2];
    int32_t* idxM[2]; int32_t* cntM[2];
    MhaWs mha; MlpWs mlp;             // attention and MLP scratch
    PredWs predA, predM;              // predictor scratch
    MfmaWs mf;                        // matrix-core scratch of every launch of the layer
    int tiles;                        // LayerNorm statistic slices per row
};
LayerWs plan_layer(Arena& A, const djv_model& m, bool dense) {
    const bool f16 = m.wt == DJV_F16;
    LayerWs w;
    w.tiles = (m.d + kLnTile - 1) / kLnTile;
    for (int i = 0; i < 2; ++i) {
        w.xs[i] = A.take<float>((size_t)m.B * m.d);
        w.sx[i] = A.take<float2>((size_t)m.B * w.tiles);
    }
    w.s_in = A.take<float2>((size_t)m.B * w.tiles);
    w.xm = A.take<float>((size_t)m.B * m.d);
    w.sm = A.take<float2>((size_t)m.B * w.tiles);
    const int capA = dense ? m.h : capA_of(m);
    const int capM = dense ? m.N : capM_of(m);
    for (int i = 0; i < 2; ++i) {
        w.idxA[i] = A.take<int32_t>(m.h);
        w.cntA[i] = A.take<int32_t>(1);
        w.idxM[i] = A.take<int32_t>(m.N);
        w.cntM[i] = A.take<int32_t>(1);
    }
    // one matrix-core scratch for every launch of the layer; its largest launches: Q/K/V
    // with both P1, both P2, MLP up
    const long long rows = std::max({(long long)capA * 3 * m.dh + 2LL * m.r,
                                     (long long)heads_total(m) + neurons_total(m), (long long)capM});
    w.mf = plan_mfma(A, layer_wide(m), m.B, rows, std::max(m.d, m.r));
    w.mha = plan_mha(A, m.B, m.d, m.dh, capA, m.n_cap, f16, true, &w.mf);
    w.mlp = plan_mlp(A, m.B, m.d, capM, f16, true, &w.mf);
    if (!dense) {
        w.predA = plan_predict(A, m.B, m.d, m.r, heads_total(m), true, true, &w.mf);
        w.predM = plan_predict(A, m.B, m.d, m.r, neurons_total(m), true, true, &w.mf);
    } else {
        w.predA = w.predM = PredWs{nullptr, nullptr, nullptr, w.mf};
    }
    return w;
}

RowInput plain_input(const float* y) {
    RowInput in{};
    in.y = y;
    return in;
}
RowInput ln_input(const float* x, const float2* stats, const LayerWs& w, float eps) {
    RowInput in{};
    in.x = x;
    in.stats = stats;
    in.ntiles = w.tiles;
    in.eps = eps;
    return in;
}
// LN(x) with the moments computed by the consuming GEMV (x accumulated in place).
RowInput own_ln_input(const float* x, float eps) {
    RowInput in{};
    in.x = x;
    in.eps = eps;
    in.own_stats = true;
    return in;
}

// ------------------------------------------------------------------------------------
// Kernel sequences shared by the entry points (arguments already validated)
// ------------------------------------------------------------------------------------
struct PredJob {
    const void* P1; const void* P2; int n_out;
    int mode, k; float t;
    int32_t* idx; int32_t* count; float* z;
    const PredWs* w;
    int lo, hi;  // the units listed: [lo, hi) of the n_out scored, rebased to lo
};

// GEMV segments of the layer's weight streams.
GemvSeg seg_first(const PredJob& j, int r, const RowInput& in) {
    GemvSeg S{};
    S.W = j.P1; S.list = UnitList{nullptr, nullptr, r, r}; S.rpu = 1; S.in = in;
    S.out = j.w->u; S.ld = r; S.epi = kEpiRelu;
    return S;
}
GemvSeg seg_second(const PredJob& j) {
    GemvSeg S{};
    S.W = j.P2; S.list = UnitList{nullptr, nullptr, j.n_out, j.n_out}; S.rpu = 1;
    S.in = plain_input(j.w->u); S.out = j.z; S.ld = j.n_out; S.epi = kEpiStore;
    return S;
}
SelectJob select_job(const PredJob& j) {
    return SelectJob{j.z, j.n_out, j.mode, j.k, j.mode == DJV_THRESHOLD ? tau_key(j.t) : 0u,
                     j.w->bits, j.idx, j.count, j.lo, j.hi};
}
GemvSeg seg_qkv(const void* Wqkv, const UnitList& heads, int dh, const RowInput& in, float* q) {
    GemvSeg S{};
    S.W = Wqkv; S.list = heads; S.rpu = 3 * dh; S.in = in; S.out = q; S.ld = heads.cap * dh;
    S.epi = kEpiQkv;
    return S;
}
GemvSeg seg_up(const void* W1, const void* b1, const UnitList& neurons, const RowInput& in, float* a) {
    GemvSeg S{};
    S.W = W1; S.list = neurons; S.rpu = 1; S.in = in; S.out = a; S.ld = neurons.cap;
    S.epi = kEpiBiasRelu; S.bias = b1;
    return S;
}

GemvArgs gemv_args(int cols, int B, int prof, const MfmaWs& mf) {
    GemvArgs g{};
    g.cols = cols; g.B = B; g.flags = device_flags(); g.prof = prof;
    g.mfma = mf.on; g.mfma_part = mf.part;
    return g;
}
void add_seg(GemvArgs& g, const GemvSeg& S) { g.seg[g.nseg++] = S; }
void add_side(GemvArgs& g, const SelectJob& J) { g.side[g.nside++] = J; }

// One or two predictors reading the same input, in three launches: both first layers
// (one GEMV launch), both second layers (one launch), both selections (one launch).
djv_status run_predict(bool f16, int B, int d, int r, const RowInput& in, const PredJob* jobs,
                       int njobs, const MfmaWs& mf, hipStream_t s) {
    GemvArgs g = gemv_args(d, B, DJV_PROF_PRED_1, mf);
    for (int i = 0; i < njobs; ++i) add_seg(g, seg_first(jobs[i], r, in));
    DJV_HIP(launch_gemv(f16, g, s));
    g = gemv_args(r, B, DJV_PROF_PRED_2, mf);
    for (int i = 0; i < njobs; ++i) add_seg(g, seg_second(jobs[i]));
    DJV_HIP(launch_gemv(f16, g, s));
    SelectJob sj[2];
    for (int i = 0; i < njobs; ++i) sj[i] = select_job(jobs[i]);
    DJV_HIP(launch_select(sj, njobs, B, s, DJV_PROF_SELECT));
    return DJV_OK;
}

// Row-axpy over the kept W2 rows: out = resid + W2_S^T a.  stats (optional) receives the
// tile statistics of out.
djv_status run_down(bool f16, int B, int d, const void* W2, const UnitList& neurons,
                    const float* resid, float* out, float2* stats, const MlpWs& w, hipStream_t s,
                    bool accumulate = false) {
    AxpyArgs x{};
    x.W = W2; x.cols = d; x.list = neurons; x.rpu = 1; x.coef = w.a; x.ldc = neurons.cap; x.B = B;
    x.partial = w.partial; x.rows_per_chunk = w.rpc; x.resid = resid;
    x.out = out; x.stats = stats; x.mfma = w.mf.on; x.flags = device_flags(); x.prof = DJV_PROF_MLP_DOWN;
    x.accumulate = accumulate;
    DJV_HIP(launch_axpy(f16, x, s));
    return DJV_OK;
}

// out = resid + MLP_S(in): gather-GEMV over the kept W1 rows, then row-axpy over the kept
// W2 rows.
djv_status run_mlp(bool f16, int B, int d, int N, const RowInput& in, const void* W1,
                   const void* b1, const void* W2, const int32_t* idx, const int32_t* count,
                   int cap, const float* resid, float* out, float2* stats, const MlpWs& w,
                   hipStream_t s) {
    const UnitList list{idx, count, cap, N};
    GemvArgs g = gemv_args(d, B, DJV_PROF_MLP_UP, w.mf);
    add_seg(g, seg_up(W1, b1, list, in, w.a));
    DJV_HIP(launch_gemv(f16, g, s));
    return run_down(f16, B, d, W2, list, resid, out, stats, w, s);
}

// Split-position attention over the kept heads (q from the QKV step).
AttnArgs attend_args(int B, int h, int dh, int n, int n_cap, void* Kc, void* Vc,
                     const UnitList& heads, float scale, const MhaWs& w) {
    AttnArgs at{};
    at.Kc = Kc; at.Vc = Vc; at.list = heads; at.h = h; at.dh = dh; at.n = n; at.n_cap = n_cap;
    at.B = B; at.q = w.q; at.scale = scale; at.part = w.part; at.chunk = w.chunk;
    at.nchunk = (n + 1 + w.chunk - 1) / w.chunk; at.H = w.H; at.flags = device_flags();
    at.prof = DJV_PROF_ATTN;
    return at;
}

// The attention's own launches: the chunks, and the merge kernel unless the O-projection
// merges them.
djv_status run_attend(bool f16, int B, int h, int dh, int n, int n_cap, void* Kc, void* Vc,
                      const UnitList& heads, float scale, const MhaWs& w, hipStream_t s) {
    DJV_HIP(launch_attention(f16, attend_args(B, h, dh, n, n_cap, Kc, Vc, heads, scale, w), !w.fused, s));
    return DJV_OK;
}

// Row-axpy over the kept heads' W_O rows: out = resid + sum_i H_i W_i^O (H merged from
// the attention chunks here when fused).
djv_status run_oproj(bool f16, int B, int d, int dh, int n, const void* Wo, const UnitList& heads,
                     const float* resid, float* out, float2* stats, const MhaWs& w, hipStream_t s,
                     bool accumulate = false) {
    AxpyArgs x{};
    x.W = Wo; x.cols = d; x.list = heads; x.rpu = dh; x.coef = w.H; x.ldc = heads.cap * dh; x.B = B;
    x.partial = w.partial; x.rows_per_chunk = w.rpc; x.resid = resid; x.out = out; x.stats = stats;
    x.mfma = w.mf.on; x.flags = device_flags(); x.prof = DJV_PROF_O_PROJ;
    x.accumulate = accumulate;
    if (w.fused) {
        x.attn_part = w.part;
        x.attn_nchunk = (n + 1 + w.chunk - 1) / w.chunk;
    }
    DJV_HIP(launch_axpy(f16, x, s));
    return DJV_OK;
}

// out = resid + MHA_S(in), appending the kept heads' K/V at position n: head-sparse QKV
// GEMV, split-position attention and its merge, row-axpy over the kept heads' W_O rows.
djv_status run_mha(bool f16, int B, int d, int h, int dh, int n, int n_cap, const RowInput& in,
                   const void* Wqkv, const void* Wo, void* Kc, void* Vc, const int32_t* idx,
                   const int32_t* count, int cap, float scale, const float* resid, float* out,
                   float2* stats, const MhaWs& w, hipStream_t s) {
    const UnitList heads{idx, count, cap, h};
    GemvArgs g = gemv_args(d, B, DJV_PROF_QKV, w.mf);
    g.Kc = Kc; g.Vc = Vc; g.h = h; g.dh = dh; g.n = n; g.n_cap = n_cap;
    add_seg(g, seg_qkv(Wqkv, heads, dh, in, w.q));
    DJV_HIP(launch_gemv(f16, g, s));
    DJV_TRY(run_attend(f16, B, h, dh, n, n_cap, Kc, Vc, heads, scale, w, s));
    return run_oproj(f16, B, d, dh, n, Wo, heads, resid, out, stats, w, s);
}

djv_status check_model(const djv_model* m) {
    DJV_REQUIRE(m != nullptr, DJV_EINVAL, "model is NULL");
    DJV_TRY(check_dtype(m->wt));
    DJV_TRY(check_batch(m->B));
    DJV_TRY(check_rowlen(m->d, m->wt, "d"));
    DJV_TRY(check_rowlen(m->r, m->wt, "r"));
    DJV_TRY(check_wide_batch(m->B, m->wt, {m->d, m->r}));
    DJV_REQUIRE(m->N >= 1 && m->h >= 1, DJV_EINVAL, "N and h must be >= 1");
    DJV_REQUIRE(m->dh == 64 || m->dh == 128, DJV_EUNSUPPORTED, "dh must be 64 or 128 (got %d)", m->dh);
    DJV_REQUIRE(m->n >= 0 && m->n < m->n_cap, DJV_EINVAL, "need 0 <= n < n_cap (n = %d, n_cap = %d)", m->n, m->n_cap);
    DJV_REQUIRE((m->n_cap + attn_chunk_for(m->wt == DJV_F16, m->dh) - 1) / attn_chunk_for(m->wt == DJV_F16, m->dh)
                    <= kAttnMaxChunks, DJV_EUNSUPPORTED, "n_cap = %d is too long", m->n_cap);
    DJV_REQUIRE(std::isfinite(m->scale), DJV_EINVAL, "scale must be finite");
    DJV_REQUIRE(m->eps > 0.f && std::isfinite(m->eps), DJV_EINVAL, "eps must be > 0");
    DJV_REQUIRE(m->h_total > 0 ? (m->h_offset >= 0 && m->h_offset + (long long)m->h <= m->h_total)
                               : (m->h_total == 0 && m->h_offset == 0),
                DJV_EINVAL, "head shard: need 0 <= h_offset and h_offset + h <= h_total (or all 0)");
    DJV_REQUIRE(m->N_total > 0 ? (m->N_offset >= 0 && m->N_offset + (long long)m->N <= m->N_total)
                               : (m->N_total == 0 && m->N_offset == 0),
                DJV_EINVAL, "neuron shard: need 0 <= N_offset and N_offset + N <= N_total (or all 0)");
    DJV_TRY(check_select(heads_total(*m), m->mode, m->k_A, m->t_A, "head selection"));
    DJV_TRY(check_select(neurons_total(*m), m->mode, m->k_M, m->t_M, "neuron selection"));
    return DJV_OK;
}

djv_status check_layer(const djv_layer* L, bool dense) {
    DJV_REQUIRE(L != nullptr, DJV_EINVAL, "layer descriptor is NULL");
    DJV_TRY(check_ptr(L->Wqkv, "Wqkv"));
    DJV_TRY(check_ptr(L->Wo, "Wo"));
    DJV_TRY(check_ptr(L->W1, "W1"));
    DJV_REQUIRE(L->b1 != nullptr, DJV_EINVAL, "b1 is NULL");
    DJV_TRY(check_ptr(L->W2, "W2"));
    DJV_TRY(check_ptr(L->Kc, "Kc"));
    DJV_TRY(check_ptr(L->Vc, "Vc"));
    if (!dense) {
        DJV_TRY(check_ptr(L->P1_A, "P1_A"));
        DJV_TRY(check_ptr(L->P2_A, "P2_A"));
        DJV_TRY(check_ptr(L->P1_M, "P1_M"));
        DJV_TRY(check_ptr(L->P2_M, "P2_M"));
    }
    DJV_REQUIRE((L->Y == nullptr) == (L->kv_len == nullptr), DJV_EINVAL,
                "lazy K/V needs both Y and kv_len (or neither)");
    if (L->Y) {
        DJV_TRY(check_ptr(L->Y, "Y"));
        DJV_TRY(check_idx_ptr(L->kv_len, "kv_len"));
    }
    return DJV_OK;
}

// Lazy K/V of a layer with the step's head list (nothing when the layer has no Y).
djv_status run_lazy_kv(bool f16, const djv_model& m, const djv_layer& L, const RowInput& in,
                       const UnitList& heads, hipStream_t s) {
    if (!L.Y) return DJV_OK;
    LazyKvArgs a{};
    a.in = in; a.Y = L.Y;
    a.kv_prev = L.kv_len + (size_t)(m.n & 1) * m.h;
    a.kv_next = L.kv_len + (size_t)((m.n + 1) & 1) * m.h;
    a.heads = heads; a.Wqkv = L.Wqkv; a.Kc = L.Kc; a.Vc = L.Vc;
    a.B = m.B; a.d = m.d; a.h = m.h; a.dh = m.dh; a.n = m.n; a.n_cap = m.n_cap;
    a.flags = device_flags();
    DJV_HIP(launch_lazy_kv(f16, a, s));
    return DJV_OK;
}

size_t layer_ws_bytes(const djv_model& m) {
    Arena A(nullptr);
    plan_layer(A, m, false);
    Arena D(nullptr);
    plan_layer(D, m, true);
    return A.off > D.off ? A.off : D.off;
}

djv_status copy_async(void* dst, const void* src, size_t bytes, hipStream_t s) {
    if (!dst || bytes == 0) return DJV_OK;
    DJV_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
    return DJV_OK;
}

// Copies a layer's sets into the optional trace.
djv_status trace_sets(const djv_trace* tr, const djv_model& m, int l, const LayerWs& w, int buf,
                      hipStream_t s) {
    if (!tr) return DJV_OK;
    const int capA = capA_of(m), capM = capM_of(m);
    if (tr->sets_A) DJV_TRY(copy_async(tr->sets_A + (size_t)l * m.h, w.idxA[buf], capA * 4, s));
    if (tr->sets_M) DJV_TRY(copy_async(tr->sets_M + (size_t)l * m.N, w.idxM[buf], capM * 4, s));
    if (tr->counts) {
        DJV_TRY(copy_async(tr->counts + 2 * l, w.cntA[buf], 4, s));
        DJV_TRY(copy_async(tr->counts + 2 * l + 1, w.cntM[buf], 4, s));
    }
    return DJV_OK;
}

djv_status trace_x(const djv_trace* tr, const djv_model& m, int l, const float* x, hipStream_t s) {
    if (!tr || !tr->x_in) return DJV_OK;
    return copy_async(tr->x_in + (size_t)l * m.B * m.d, x, (size_t)m.B * m.d * 4, s);
}

// Score buffers of layer l: the trace's when it asks for them, else the workspace's.
float* zA_of(const djv_trace* tr, const djv_model& m, int l, const LayerWs& w) {
    return (tr && tr->z_A) ? tr->z_A + (size_t)l * m.B * heads_total(m) : w.predA.z;
}
float* zM_of(const djv_trace* tr, const djv_model& m, int l, const LayerWs& w) {
    return (tr && tr->z_M) ? tr->z_M + (size_t)l * m.B * neurons_total(m) : w.predM.z;
}

PredJob job_A(const djv_model& m, const djv_layer& L, const LayerWs& w, int buf,
              const djv_trace* tr, int l) {
    return PredJob{L.P1_A, L.P2_A, heads_total(m), m.mode, m.k_A, m.t_A, w.idxA[buf], w.cntA[buf],
                   zA_of(tr, m, l, w), &w.predA, m.h_offset, m.h_offset + m.h};
}
PredJob job_M(const djv_model& m, const djv_layer& L, const LayerWs& w, int buf,
              const djv_trace* tr, int l) {
    return PredJob{L.P1_M, L.P2_M, neurons_total(m), m.mode, m.k_M, m.t_M, w.idxM[buf], w.cntM[buf],
                   zM_of(tr, m, l, w), &w.predM, m.N_offset, m.N_offset + m.N};
}

// Input and output of layer l in a stack of L: layer 0 reads the caller's x, the last
// layer writes it, the others use the two-entry ring.
struct LayerIO {
    const float* x_in; const float2* s_in;
    float* x_out; float2* s_out;
};
LayerIO layer_io(float* x, const LayerWs& w, int l, int L) {
    LayerIO io;
    io.x_in = l == 0 ? x : w.xs[l & 1];
    io.s_in = l == 0 ? w.s_in : w.sx[l & 1];
    io.x_out = l == L - 1 ? x : w.xs[(l + 1) & 1];
    io.s_out = l == L - 1 ? nullptr : w.sx[(l + 1) & 1];
    return io;
}

// Device count of a selected list, or nullptr when it is known on the host to equal the
// capacity (top-k with one sequence keeps exactly k, unless a shard keeps only its part of
// them), which saves kernels a dependent read.
const int32_t* count_of(const djv_model& m, const int32_t* count) {
    return (m.mode == DJV_TOPK && m.B == 1 && !sharded(m)) ? nullptr : count;
}

// Attention then MLP of layer l with the sets in buffer `buf`.  With serial set, the
// neuron set is predicted from LN(x') in between (the order of the naive block).
djv_status layer_body(const djv_model& m, const djv_layer& L, const LayerIO& io, const LayerWs& w,
                      int buf, bool serial, const djv_trace* tr, int l, hipStream_t s) {
    const bool f16 = m.wt == DJV_F16;
    DJV_TRY(run_lazy_kv(f16, m, L, ln_input(io.x_in, io.s_in, w, m.eps),
                        UnitList{w.idxA[buf], count_of(m, w.cntA[buf]), capA_of(m), m.h}, s));
    DJV_TRY(run_mha(f16, m.B, m.d, m.h, m.dh, m.n, m.n_cap, ln_input(io.x_in, io.s_in, w, m.eps),
                    L.Wqkv, L.Wo, L.Kc, L.Vc, w.idxA[buf], count_of(m, w.cntA[buf]),
                    capA_of(m), m.scale, io.x_in, w.xm, w.sm, w.mha, s));
    if (tr && tr->x_mid)
        DJV_TRY(copy_async(tr->x_mid + (size_t)l * m.B * m.d, w.xm, (size_t)m.B * m.d * 4, s));
    const RowInput in_m = ln_input(w.xm, w.sm, w, m.eps);
    if (serial) {
        const PredJob jm = job_M(m, L, w, buf, tr, l);
        DJV_TRY(run_predict(f16, m.B, m.d, m.r, in_m, &jm, 1, w.mf, s));
    }
    DJV_TRY(run_mlp(f16, m.B, m.d, m.N, in_m, L.W1, L.b1, L.W2, w.idxM[buf], count_of(m, w.cntM[buf]),
                    capM_of(m), w.xm, io.x_out, io.s_out, w.mlp, s));
    return DJV_OK;
}

// One serial layer (head set from LN(x), neuron set from LN(x')).
djv_status serial_layer(const djv_model& m, const djv_layer& L, const LayerIO& io,
                        const LayerWs& w, const djv_trace* tr, int l, hipStream_t s) {
    DJV_TRY(trace_x(tr, m, l, io.x_in, s));
    const PredJob ja = job_A(m, L, w, 0, tr, l);
    DJV_TRY(run_predict(m.wt == DJV_F16, m.B, m.d, m.r, ln_input(io.x_in, io.s_in, w, m.eps), &ja, 1, w.mf, s));
    DJV_TRY(layer_body(m, L, io, w, 0, true, tr, l, s));
    return trace_sets(tr, m, l, w, 0, s);
}

}  // namespace

// ======================================================================================
// Entry points
// ======================================================================================
extern "C" {

const char* dejavu_last_error(void) { return g_err.c_str(); }

const char* dejavu_version(void) { return "dejavu-mi355x 0.2 (gfx950)"; }

djv_status dejavu_workspace_bytes(int B, int d, int N, int h, int dh, int r, int n_cap,
                                  size_t* bytes) {
    DJV_REQUIRE(bytes != nullptr, DJV_EINVAL, "bytes is NULL");
    DJV_REQUIRE(B >= 0 && d >= 0 && N >= 0 && h >= 0 && dh >= 0 && r >= 0 && n_cap >= 0,
                DJV_EINVAL, "sizes must be >= 0");
    const int Bq = B > 0 ? B : 1;
    size_t need = 0;
    auto upd = [&](size_t v) { if (v > need) need = v; };
    for (int f = 0; f < 2; ++f) {
        const bool f16 = f == 1;
        const int n_out = N > h ? N : h;
        if (n_out > 0) {
            Arena a(nullptr);
            plan_predict(a, Bq, d, r, n_out, true, f16 && d % 32 == 0 && r % 32 == 0);
            upd(a.off);
        }
        if (N > 0 && d > 0) {
            Arena a(nullptr);
            plan_mlp(a, Bq, d, N, f16, f16 && d % 32 == 0);
            upd(a.off);
        }
        if (h > 0 && d > 0 && dh > 0) {
            Arena a(nullptr);
            plan_mha(a, Bq, d, dh, h, n_cap > 0 ? n_cap : 1, f16, f16 && d % 32 == 0);
            upd(a.off);
        }
        if (N > 0 && h > 0 && d > 0 && dh > 0) {
            djv_model m{};
            m.wt = f16 ? DJV_F16 : DJV_F32; m.B = Bq; m.d = d; m.N = N; m.h = h; m.dh = dh;
            m.r = r; m.n_cap = n_cap > 0 ? n_cap : 1; m.mode = DJV_THRESHOLD;
            upd(layer_ws_bytes(m));
        }
    }
    *bytes = need;
    return DJV_OK;
}

djv_status dejavu_workspace_bytes_model(const djv_model* m, size_t* bytes) {
    DJV_REQUIRE(bytes != nullptr, DJV_EINVAL, "bytes is NULL");
    DJV_TRY(check_model(m));
    *bytes = layer_ws_bytes(*m);
    return DJV_OK;
}

djv_status dejavu_layernorm(int B, int d, const float* x, float* y, float eps, void* stream) {
    DJV_REQUIRE(B >= 1 && d >= 1, DJV_EINVAL, "B and d must be >= 1");
    DJV_REQUIRE(d <= 16384, DJV_EUNSUPPORTED, "d = %d exceeds 16384", d);
    DJV_REQUIRE(eps > 0.f && std::isfinite(eps), DJV_EINVAL, "eps must be > 0");
    DJV_TRY(check_ptr(x, "x"));
    DJV_TRY(check_ptr(y, "y"));
    DJV_HIP(launch_layernorm(B, d, x, y, eps, (hipStream_t)stream));
    return DJV_OK;
}

djv_status dejavu_gather_rows(djv_dtype wt, int rpu, int cols, int units, const void* W,
                              const int32_t* idx, const int32_t* count, int cap, void* out,
                              void* stream) {
    DJV_TRY(check_dtype(wt));
    DJV_REQUIRE(rpu >= 1 && cols >= 1 && units >= 1, DJV_EINVAL, "rpu, cols and units must be >= 1");
    DJV_REQUIRE(cap >= 1 && cap <= units, DJV_EINVAL, "cap = %d outside [1, units = %d]", cap, units);
    DJV_REQUIRE((long long)cap * rpu <= 0x7fffffffLL && (long long)units * rpu <= 0x7fffffffLL, DJV_EUNSUPPORTED,
                "too many rows");
    const size_t row_bytes = (size_t)cols * esize(wt);
    const size_t al = row_bytes % 16 == 0 ? 16 : (row_bytes % 4 == 0 ? 4 : 2);
    DJV_REQUIRE(W != nullptr && out != nullptr, DJV_EINVAL, "W and out must not be NULL");
    DJV_REQUIRE(aligned(W, al) && aligned(out, al), DJV_EALIGN, "W and out must be %zu-byte aligned", al);
    DJV_TRY(check_idx_ptr(idx, "idx"));
    if (count) DJV_TRY(check_idx_ptr(count, "count"));
    const UnitList list{idx, count, cap, units};
    DJV_HIP(launch_gather_rows(W, out, list, rpu, row_bytes, device_flags(), (hipStream_t)stream));
    return DJV_OK;
}

djv_status dejavu_select(int B, int n_out, const float* z, djv_mode mode, int k, float t,
                         int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
    return dejavu_select_range(B, n_out, z, mode, k, t, 0, n_out, idx, count, ws, ws_bytes, stream);
}

djv_status dejavu_select_range(int B, int n_out, const float* z, djv_mode mode, int k, float t,
                               int lo, int hi, int32_t* idx, int32_t* count, void* ws,
                               size_t ws_bytes, void* stream) {
    DJV_REQUIRE(B >= 1 && B <= 65535, DJV_EINVAL, "B must lie in [1, 65535] (got %d)", B);
    DJV_TRY(check_select(n_out, mode, k, t, "select"));
    DJV_REQUIRE(0 <= lo && lo <= hi && hi <= n_out, DJV_EINVAL,
                "need 0 <= lo <= hi <= n_out (lo = %d, hi = %d, n_out = %d)", lo, hi, n_out);
    DJV_TRY(check_ptr(z, "z"));
    DJV_TRY(check_idx_ptr(idx, "idx"));
    DJV_TRY(check_idx_ptr(count, "count"));
    Arena sz(nullptr);
    sz.take<uint32_t>((size_t)B * words_of(n_out));
    DJV_TRY(check_ws(ws, ws_bytes, sz.off));
    Arena A(ws);
    uint32_t* bits = A.take<uint32_t>((size_t)B * words_of(n_out));
    SelectJob j{z, n_out, (int)mode, k, mode == DJV_THRESHOLD ? tau_key(t) : 0u, bits, idx, count, lo, hi};
    DJV_HIP(launch_select(&j, 1, B, (hipStream_t)stream, DJV_PROF_SELECT));
    return DJV_OK;
}

djv_status dejavu_predict(djv_dtype wt, int B, int d, int r, int n_out, const float* y,
                          const void* P1, const void* P2, djv_mode mode, int k, float t,
                          int32_t* idx, int32_t* count, float* logits,
                          void* ws, size_t ws_bytes, void* stream) {
    DJV_TRY(check_dtype(wt));
    DJV_TRY(check_batch(B));
    DJV_TRY(check_rowlen(d, wt, "d"));
    DJV_TRY(check_rowlen(r, wt, "r"));
    DJV_TRY(check_wide_batch(B, wt, {d, r}));
    DJV_TRY(check_select(n_out, mode, k, t, "predict"));
    DJV_TRY(check_ptr(y, "y"));
    DJV_TRY(check_ptr(P1, "P1"));
    DJV_TRY(check_ptr(P2, "P2"));
    DJV_TRY(check_idx_ptr(idx, "idx"));
    DJV_TRY(check_idx_ptr(count, "count"));
    DJV_TRY(check_opt_ptr(logits, "logits"));
    Arena sz(nullptr);
    const bool wide = wide_possible(wt, {d, r});
    plan_predict(sz, B, d, r, n_out, logits == nullptr, wide);
    DJV_TRY(check_ws(ws, ws_bytes, sz.off));
    Arena A(ws);
    const PredWs w = plan_predict(A, B, d, r, n_out, logits == nullptr, wide);
    const PredJob j{P1, P2, n_out, (int)mode, k, t, idx, count, logits ? logits : w.z, &w, 0, n_out};
    return run_predict(wt == DJV_F16, B, d, r, plain_input(y), &j, 1, w.mf, (hipStream_t)stream);
}

static djv_status check_mlp_args(djv_dtype wt, int B, int d, int N, const float* y, const void* W1,
                                 const void* b1, const void* W2, int cap, const float* resid,
                                 float* out) {
    DJV_TRY(check_dtype(wt));
    DJV_TRY(check_batch(B));
    DJV_TRY(check_rowlen(d, wt, "d"));
    DJV_TRY(check_wide_batch(B, wt, {d}));
    DJV_REQUIRE(N >= 1, DJV_EINVAL, "N must be >= 1");
    DJV_REQUIRE(cap >= 1 && cap <= N, DJV_EINVAL, "cap = %d outside [1, N = %d]", cap, N);
    DJV_TRY(check_ptr(y, "y"));
    DJV_TRY(check_ptr(W1, "W1"));
    DJV_REQUIRE(b1 != nullptr, DJV_EINVAL, "b1 is NULL");
    DJV_TRY(check_ptr(W2, "W2"));
    DJV_TRY(check_opt_ptr(resid, "resid"));
    DJV_TRY(check_ptr(out, "out"));
    return DJV_OK;
}

// Scratch bytes of an MLP call (valid arguments).
static size_t mlp_ws_need(djv_dtype wt, int B, int d, int cap) {
    Arena sz(nullptr);
    plan_mlp(sz, B, d, cap, wt == DJV_F16, wide_possible(wt, {d}));
    return sz.off;
}

static djv_status mlp_common(djv_dtype wt, int B, int d, int N, const float* y, const void* W1,
                             const void* b1, const void* W2, const int32_t* idx,
                             const int32_t* count, int cap, const float* resid, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
    DJV_TRY(check_mlp_args(wt, B, d, N, y, W1, b1, W2, cap, resid, out));
    const bool f16 = wt == DJV_F16;
    const bool wide = wide_possible(wt, {d});
    DJV_TRY(check_ws(ws, ws_bytes, mlp_ws_need(wt, B, d, cap)));
    Arena A(ws);
    const MlpWs w = plan_mlp(A, B, d, cap, f16, wide);
    return run_mlp(f16, B, d, N, plain_input(y), W1, b1, W2, idx, count, cap, resid, out, nullptr,
                   w, (hipStream_t)stream);
}

djv_status dejavu_sparse_mlp(djv_dtype wt, int B, int d, int N, const float* y, const void* W1,
                             const void* b1, const void* W2, const int32_t* idx,
                             const int32_t* count, int cap, const float* resid, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
    DJV_TRY(check_idx_ptr(idx, "idx"));
    DJV_TRY(check_idx_ptr(count, "count"));
    return mlp_common(wt, B, d, N, y, W1, b1, W2, idx, count, cap, resid, out, ws, ws_bytes, stream);
}

djv_status dejavu_sparse_mlp_no_alloc(djv_dtype wt, int B, int d, int N, const float* y,
                                      const void* W1, const void* b1, const void* W2,
                                      const int32_t* idx, const int32_t* count, int cap,
                                      const float* resid, float* out, void* stream) {
    DJV_TRY(check_idx_ptr(idx, "idx"));
    DJV_TRY(check_idx_ptr(count, "count"));
    DJV_TRY(check_mlp_args(wt, B, d, N, y, W1, b1, W2, cap, resid, out));
    const size_t need = mlp_ws_need(wt, B, d, cap);
    DJV_REQUIRE(need <= kStaticScratchBytes, DJV_EUNSUPPORTED,
                "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
                "dejavu_sparse_mlp with a workspace)", need, kStaticScratchBytes);
    void* ptr = nullptr;
    DJV_TRY(static_scratch(&ptr));
    return mlp_common(wt, B, d, N, y, W1, b1, W2, idx, count, cap, resid, out, ptr,
                      kStaticScratchBytes, stream);
}

djv_status dejavu_dense_mlp(djv_dtype wt, int B, int d, int N, const float* y, const void* W1,
                            const void* b1, const void* W2, const float* resid, float* out,
                            void* ws, size_t ws_bytes, void* stream) {
    return mlp_common(wt, B, d, N, y, W1, b1, W2, nullptr, nullptr, N, resid, out, ws, ws_bytes,
                      stream);
}

static djv_status mha_common(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                             const float* y, const void* Wqkv, const void* Wo, void* Kc, void* Vc,
                             const int32_t* idx, const int32_t* count, int cap, float scale,
                             const float* resid, float* out, void* ws, size_t ws_bytes,
                             void* stream) {
    DJV_TRY(check_dtype(wt));
    DJV_TRY(check_batch(B));
    DJV_TRY(check_rowlen(d, wt, "d"));
    DJV_TRY(check_wide_batch(B, wt, {d}));
    DJV_REQUIRE(h >= 1, DJV_EINVAL, "h must be >= 1");
    DJV_REQUIRE(dh == 64 || dh == 128, DJV_EUNSUPPORTED, "dh must be 64 or 128 (got %d)", dh);
    DJV_REQUIRE(n >= 0 && n < n_cap, DJV_EINVAL, "need 0 <= n < n_cap (n = %d, n_cap = %d)", n, n_cap);
    DJV_REQUIRE((n_cap + attn_chunk_for(wt == DJV_F16, dh) - 1) / attn_chunk_for(wt == DJV_F16, dh)
                    <= kAttnMaxChunks, DJV_EUNSUPPORTED, "n_cap = %d is too long", n_cap);
    DJV_REQUIRE(cap >= 1 && cap <= h, DJV_EINVAL, "cap = %d outside [1, h = %d]", cap, h);
    DJV_REQUIRE(std::isfinite(scale), DJV_EINVAL, "scale must be finite");
    DJV_TRY(check_ptr(y, "y"));
    DJV_TRY(check_ptr(Wqkv, "Wqkv"));
    DJV_TRY(check_ptr(Wo, "Wo"));
    DJV_TRY(check_ptr(Kc, "Kc"));
    DJV_TRY(check_ptr(Vc, "Vc"));
    DJV_TRY(check_opt_ptr(resid, "resid"));
    DJV_TRY(check_ptr(out, "out"));
    const bool f16 = wt == DJV_F16;
    Arena sz(nullptr);
    const bool wide = wide_possible(wt, {d});
    plan_mha(sz, B, d, dh, cap, n_cap, f16, wide);
    DJV_TRY(check_ws(ws, ws_bytes, sz.off));
    Arena A(ws);
    const MhaWs w = plan_mha(A, B, d, dh, cap, n_cap, f16, wide);
    return run_mha(f16, B, d, h, dh, n, n_cap, plain_input(y), Wqkv, Wo, Kc, Vc, idx, count, cap,
                   scale, resid, out, nullptr, w, (hipStream_t)stream);
}

djv_status dejavu_sparse_mha(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                             const float* y, const void* Wqkv, const void* Wo, void* Kc, void* Vc,
                             const int32_t* head_idx, const int32_t* head_count, int cap,
                             float scale, const float* resid, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
    DJV_TRY(check_idx_ptr(head_idx, "head_idx"));
    DJV_TRY(check_idx_ptr(head_count, "head_count"));
    return mha_common(wt, B, d, h, dh, n, n_cap, y, Wqkv, Wo, Kc, Vc, head_idx, head_count, cap,
                      scale, resid, out, ws, ws_bytes, stream);
}

djv_status dejavu_dense_mha(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                            const float* y, const void* Wqkv, const void* Wo, void* Kc, void* Vc,
                            float scale, const float* resid, float* out, void* ws,
                            size_t ws_bytes, void* stream) {
    return mha_common(wt, B, d, h, dh, n, n_cap, y, Wqkv, Wo, Kc, Vc, nullptr, nullptr, h, scale,
                      resid, out, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------------------
// Output norms: the scores of the "true" selection
// ------------------------------------------------------------------------------------
djv_status dejavu_neuron_norms(djv_dtype wt, int B, int d, int N, const float* y, const void* W1,
                               const void* b1, float* scores, void* ws, size_t ws_bytes,
                               void* stream) {
    DJV_TRY(check_dtype(wt));
    DJV_TRY(check_batch(B));
    DJV_TRY(check_rowlen(d, wt, "d"));
    DJV_TRY(check_wide_batch(B, wt, {d}));
    DJV_REQUIRE(N >= 1, DJV_EINVAL, "N must be >= 1");
    DJV_TRY(check_ptr(y, "y"));
    DJV_TRY(check_ptr(W1, "W1"));
    DJV_REQUIRE(b1 != nullptr, DJV_EINVAL, "b1 is NULL");
    DJV_TRY(check_ptr(scores, "scores"));
    const bool f16 = wt == DJV_F16;
    Arena sz(nullptr);
    const bool wide = wide_possible(wt, {d});
    plan_mlp(sz, B, d, N, f16, wide);
    DJV_TRY(check_ws(ws, ws_bytes, sz.off));
    Arena A(ws);
    const MlpWs w = plan_mlp(A, B, d, N, f16, wide);
    const hipStream_t s = (hipStream_t)stream;
    // the dense up-projection's activations a [B, N], then their norms across the batch
    GemvArgs g = gemv_args(d, B, DJV_PROF_MLP_UP, w.mf);
    add_seg(g, seg_up(W1, b1, UnitList{nullptr, nullptr, N, N}, plain_input(y), w.a));
    DJV_HIP(launch_gemv(f16, g, s));
    DJV_HIP(launch_unit_norms(w.a, B, N, 1, scores, s));
    return DJV_OK;
}

djv_status dejavu_head_norms(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                             const float* y, const void* Wqkv, void* Kc, void* Vc, float scale,
                             float* scores, void* ws, size_t ws_bytes, void* stream) {
    DJV_TRY(check_dtype(wt));
    DJV_TRY(check_batch(B));
    DJV_TRY(check_rowlen(d, wt, "d"));
    DJV_TRY(check_wide_batch(B, wt, {d}));
    DJV_REQUIRE(h >= 1, DJV_EINVAL, "h must be >= 1");
    DJV_REQUIRE(dh == 64 || dh == 128, DJV_EUNSUPPORTED, "dh must be 64 or 128 (got %d)", dh);
    DJV_REQUIRE(n >= 0 && n < n_cap, DJV_EINVAL, "need 0 <= n < n_cap (n = %d, n_cap = %d)", n, n_cap);
    DJV_REQUIRE((n_cap + attn_chunk_for(wt == DJV_F16, dh) - 1) / attn_chunk_for(wt == DJV_F16, dh)
                    <= kAttnMaxChunks, DJV_EUNSUPPORTED, "n_cap = %d is too long", n_cap);
    DJV_REQUIRE(std::isfinite(scale), DJV_EINVAL, "scale must be finite");
    DJV_TRY(check_ptr(y, "y"));
    DJV_TRY(check_ptr(Wqkv, "Wqkv"));
    DJV_TRY(check_ptr(Kc, "Kc"));
    DJV_TRY(check_ptr(Vc, "Vc"));
    DJV_TRY(check_ptr(scores, "scores"));
    const bool f16 = wt == DJV_F16;
    Arena sz(nullptr);
    const bool wide = wide_possible(wt, {d});
    plan_mha(sz, B, d, dh, h, n_cap, f16, wide);
    DJV_TRY(check_ws(ws, ws_bytes, sz.off));
    Arena A(ws);
    const MhaWs w = plan_mha(A, B, d, dh, h, n_cap, f16, wide);
    const hipStream_t s = (hipStream_t)stream;
    // Q/K/V of every head (K/V appended at n), attention merged into H [B, h, dh], norms
    const UnitList heads{nullptr, nullptr, h, h};
    GemvArgs g = gemv_args(d, B, DJV_PROF_QKV, w.mf);
    g.Kc = Kc; g.Vc = Vc; g.h = h; g.dh = dh; g.n = n; g.n_cap = n_cap;
    add_seg(g, seg_qkv(Wqkv, heads, dh, plain_input(y), w.q));
    DJV_HIP(launch_gemv(f16, g, s));
    DJV_HIP(launch_attention(f16, attend_args(B, h, dh, n, n_cap, Kc, Vc, heads, scale, w), true, s));
    DJV_HIP(launch_unit_norms(w.H, B, h, dh, scores, s));
    return DJV_OK;
}

djv_status dejavu_sparse_layer(const djv_model* m, const djv_layer* layer, float* x,
                               const djv_trace* trace, void* ws, size_t ws_bytes, void* stream) {
    DJV_TRY(check_model(m));
    DJV_TRY(check_layer(layer, false));
    DJV_TRY(check_ptr(x, "x"));
    DJV_TRY(check_ws(ws, ws_bytes, layer_ws_bytes(*m)));
    hipStream_t s = (hipStream_t)stream;
    Arena A(ws);
    const LayerWs w = plan_layer(A, *m, false);
    DJV_HIP(launch_ln_stats(m->B, m->d, x, w.s_in, s));
    return serial_layer(*m, *layer, layer_io(x, w, 0, 1), w, trace, 0, s);
}

djv_status dejavu_stack_decode(const djv_model* m, const djv_layer* layers, int L, float* x,
                               int lookahead, int dense, const djv_trace* trace, void* ws,
                               size_t ws_bytes, void* stream) {
    DJV_TRY(check_model(m));
    DJV_REQUIRE(L >= 1, DJV_EINVAL, "L must be >= 1");
    DJV_REQUIRE(layers != nullptr, DJV_EINVAL, "layers is NULL");
    for (int l = 0; l < L; ++l) DJV_TRY(check_layer(&layers[l], dense != 0));
    DJV_TRY(check_ptr(x, "x"));
    DJV_TRY(check_ws(ws, ws_bytes, layer_ws_bytes(*m)));
    hipStream_t sm = (hipStream_t)stream;
    const bool f16 = m->wt == DJV_F16;
    Arena A(ws);
    const LayerWs w = plan_layer(A, *m, dense != 0);
    // Unless the caller asks for bitwise-reproducible results, the lookahead stack in the
    // vector-ALU form keeps the residual stream in x itself: the O-projection and MLP-down
    // row-axpys add their products to it with fp32 atomics and the GEMVs that read LN(x)
    // (and lazy K/V's save of the attention input) sum its moments themselves, so no
    // finalize launch follows either projection.  The matrix-core form uses the finalize.
    const bool in_place = lookahead && !dense && !w.mf.on &&
                          !g_deterministic.load(std::memory_order_relaxed);
    if (!in_place) DJV_HIP(launch_ln_stats(m->B, m->d, x, w.s_in, sm));

    if (dense) {
        for (int l = 0; l < L; ++l) {
            const djv_layer& Ly = layers[l];
            const LayerIO io = layer_io(x, w, l, L);
            DJV_TRY(trace_x(trace, *m, l, io.x_in, sm));
            DJV_TRY(run_lazy_kv(f16, *m, Ly, ln_input(io.x_in, io.s_in, w, m->eps),
                                UnitList{nullptr, nullptr, m->h, m->h}, sm));
            DJV_TRY(run_mha(f16, m->B, m->d, m->h, m->dh, m->n, m->n_cap,
                            ln_input(io.x_in, io.s_in, w, m->eps), Ly.Wqkv, Ly.Wo, Ly.Kc, Ly.Vc,
                            nullptr, nullptr, m->h, m->scale, io.x_in, w.xm, w.sm, w.mha, sm));
            if (trace && trace->x_mid)
                DJV_TRY(copy_async(trace->x_mid + (size_t)l * m->B * m->d, w.xm,
                                   (size_t)m->B * m->d * 4, sm));
            DJV_TRY(run_mlp(f16, m->B, m->d, m->N, ln_input(w.xm, w.sm, w, m->eps), Ly.W1, Ly.b1,
                            Ly.W2, nullptr, nullptr, m->N, w.xm, io.x_out, io.s_out, w.mlp, sm));
        }
        return DJV_OK;
    }

    if (!lookahead) {
        for (int l = 0; l < L; ++l)
            DJV_TRY(serial_layer(*m, layers[l], layer_io(x, w, l, L), w, trace, l, sm));
        return DJV_OK;
    }

    // Lookahead schedule on one stream: the sets of layer l+1 are predicted from LN(x_l)
    // inside layer l's launches.  Both first predictor layers share the Q/K/V launch (same
    // input), the second layers run after the attention, and each selection runs in a side
    // block of a later weight stream: S_A^{l+1} beside the MLP up-projection of layer l,
    // S_M^l beside the Q/K/V launch of layer l.
    const int capA = capA_of(*m), capM = capM_of(*m);
    {
        // layer 0's scores from LN(x_0); S_A^0 alone, S_M^0 in layer 0's Q/K/V launch
        const LayerIO io0 = layer_io(x, w, 0, L);
        const RowInput in0 = in_place ? own_ln_input(x, m->eps) : ln_input(io0.x_in, io0.s_in, w, m->eps);
        const PredJob ja = job_A(*m, layers[0], w, 0, trace, 0), jm = job_M(*m, layers[0], w, 0, trace, 0);
        GemvArgs g = gemv_args(m->d, m->B, DJV_PROF_PRED_1, w.mf);
        add_seg(g, seg_first(ja, m->r, in0));
        add_seg(g, seg_first(jm, m->r, in0));
        DJV_HIP(launch_gemv(f16, g, sm));
        g = gemv_args(m->r, m->B, DJV_PROF_PRED_2, w.mf);
        add_seg(g, seg_second(ja));
        add_seg(g, seg_second(jm));
        DJV_HIP(launch_gemv(f16, g, sm));
        const SelectJob sa = select_job(ja);
        DJV_HIP(launch_select(&sa, 1, m->B, sm, DJV_PROF_SELECT));
    }
    for (int l = 0; l < L; ++l) {
        const int cur = l & 1, nxt = (l + 1) & 1;
        const bool ahead = l + 1 < L;
        const djv_layer& Ly = layers[l];
        const LayerIO io = in_place ? LayerIO{x, nullptr, x, nullptr} : layer_io(x, w, l, L);
        const RowInput in_a = in_place ? own_ln_input(x, m->eps) : ln_input(io.x_in, io.s_in, w, m->eps);
        const UnitList heads{w.idxA[cur], count_of(*m, w.cntA[cur]), capA, m->h};
        const UnitList neurons{w.idxM[cur], count_of(*m, w.cntM[cur]), capM, m->N};
        PredJob na{}, nm{};
        if (ahead) {
            na = job_A(*m, layers[l + 1], w, nxt, trace, l + 1);
            nm = job_M(*m, layers[l + 1], w, nxt, trace, l + 1);
        }
        DJV_TRY(trace_x(trace, *m, l, io.x_in, sm));
        DJV_TRY(run_lazy_kv(f16, *m, Ly, in_a, heads, sm));

        // Q/K/V of the kept heads (+ K/V append), P1 of both predictors for l+1, S_M^l
        GemvArgs g = gemv_args(m->d, m->B, DJV_PROF_QKV, w.mf);
        g.Kc = Ly.Kc; g.Vc = Ly.Vc; g.h = m->h; g.dh = m->dh; g.n = m->n; g.n_cap = m->n_cap;
        add_seg(g, seg_qkv(Ly.Wqkv, heads, m->dh, in_a, w.mha.q));
        if (ahead) {
            add_seg(g, seg_first(na, m->r, in_a));
            add_seg(g, seg_first(nm, m->r, in_a));
        }
        add_side(g, select_job(job_M(*m, Ly, w, cur, trace, l)));
        DJV_HIP(launch_gemv(f16, g, sm));
        DJV_TRY(trace_sets(trace, *m, l, w, cur, sm));

        if (ahead && w.mha.fused) {
            // P2 of both predictors for l+1, with the attention chunks in its first blocks
            g = gemv_args(m->r, m->B, DJV_PROF_PRED_2, w.mf);
            add_seg(g, seg_second(na));
            add_seg(g, seg_second(nm));
            g.attn = attend_args(m->B, m->h, m->dh, m->n, m->n_cap, Ly.Kc, Ly.Vc, heads, m->scale, w.mha);
            g.nattn = m->B * capA * g.attn.nchunk;
            DJV_HIP(launch_gemv(f16, g, sm));
        } else {
            DJV_TRY(run_attend(f16, m->B, m->h, m->dh, m->n, m->n_cap, Ly.Kc, Ly.Vc, heads, m->scale,
                               w.mha, sm));
            if (ahead) {
                g = gemv_args(m->r, m->B, DJV_PROF_PRED_2, w.mf);
                add_seg(g, seg_second(na));
                add_seg(g, seg_second(nm));
                DJV_HIP(launch_gemv(f16, g, sm));
            }
        }
        // x' = x + attention: added to x itself (in place), else written to xm with its
        // tile statistics
        float* xm = in_place ? x : w.xm;
        if (in_place)
            DJV_TRY(run_oproj(f16, m->B, m->d, m->dh, m->n, Ly.Wo, heads, nullptr, x, nullptr, w.mha, sm, true));
        else
            DJV_TRY(run_oproj(f16, m->B, m->d, m->dh, m->n, Ly.Wo, heads, io.x_in, w.xm, w.sm, w.mha, sm));
        if (trace && trace->x_mid)
            DJV_TRY(copy_async(trace->x_mid + (size_t)l * m->B * m->d, xm, (size_t)m->B * m->d * 4, sm));

        // MLP up-projection of the kept neurons, S_A^{l+1}
        g = gemv_args(m->d, m->B, DJV_PROF_MLP_UP, w.mf);
        add_seg(g, seg_up(Ly.W1, Ly.b1, neurons,
                          in_place ? own_ln_input(x, m->eps) : ln_input(w.xm, w.sm, w, m->eps), w.mlp.a));
        if (ahead) add_side(g, select_job(na));
        DJV_HIP(launch_gemv(f16, g, sm));
        if (in_place)
            DJV_TRY(run_down(f16, m->B, m->d, Ly.W2, neurons, nullptr, x, nullptr, w.mlp, sm, true));
        else
            DJV_TRY(run_down(f16, m->B, m->d, Ly.W2, neurons, w.xm, io.x_out, io.s_out, w.mlp, sm));
    }
    return DJV_OK;
}

djv_status dejavu_set_mfma_min_batch(int b, int* previous) {
    DJV_REQUIRE(b >= 1 && b <= kMaxBatch + 1, DJV_EINVAL, "b = %d outside [1, %d]", b, kMaxBatch + 1);
    const int old = g_mfma_min_batch.exchange(b);
    if (previous) *previous = old;
    return DJV_OK;
}

djv_status dejavu_set_deterministic(int on, int* previous) {
    DJV_REQUIRE(on == 0 || on == 1, DJV_EINVAL, "on = %d is not 0 or 1", on);
    const int old = g_deterministic.exchange(on);
    if (previous) *previous = old;
    return DJV_OK;
}

djv_status dejavu_profile_kernel(int family, void* const* events, int capacity) {
    DJV_REQUIRE(family >= DJV_PROF_OFF && family <= DJV_PROF_SELECT, DJV_EINVAL,
                "unknown kernel family %d", family);
    ProfHook& h = prof_hook();
    if (family == DJV_PROF_OFF) {
        h = ProfHook{};
        return DJV_OK;
    }
    DJV_REQUIRE(events != nullptr && capacity >= 1, DJV_EINVAL, "events and capacity >= 1 are required");
    h.family = family;
    h.ev = events;
    h.cap = capacity;
    h.used = 0;
    h.open = false;
    return DJV_OK;
}

djv_status dejavu_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    DJV_REQUIRE(buf != nullptr && out != nullptr, DJV_EINVAL, "buf and out must not be NULL");
    DJV_REQUIRE(bytes > 0 && bytes % 16 == 0, DJV_EINVAL, "bytes = %zu must be a positive multiple of 16", bytes);
    DJV_REQUIRE(aligned(buf, 16) && aligned(out, 4), DJV_EALIGN, "buf must be 16-byte and out 4-byte aligned");
    DJV_HIP(launch_read_probe(buf, bytes, out, (hipStream_t)stream));
    return DJV_OK;
}

djv_status dejavu_profile_count(int* count) {
    DJV_REQUIRE(count != nullptr, DJV_EINVAL, "count is NULL");
    *count = prof_hook().used;
    return DJV_OK;
}

djv_status dejavu_poll_device_error(void* stream, uint32_t* flags) {
    DJV_REQUIRE(flags != nullptr, DJV_EINVAL, "flags is NULL");
    unsigned* dflags = device_flags();
    DJV_REQUIRE(dflags != nullptr, DJV_EHIP, "device flag word unavailable");
    DJV_HIP(hipStreamSynchronize((hipStream_t)stream));
    unsigned v = 0;
    DJV_HIP(hipMemcpy(&v, dflags, sizeof v, hipMemcpyDeviceToHost));
    const unsigned zero = 0;
    DJV_HIP(hipMemcpy(dflags, &zero, sizeof zero, hipMemcpyHostToDevice));
    *flags = v;
    return DJV_OK;
}

}  // extern "C"
