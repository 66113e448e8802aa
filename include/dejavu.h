/*
 * dejavu.h -- C ABI of libdejavu.so: the contextually sparse decode-step transformer
 * layer (Deja Vu) on AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [BLOG]  "用Deja Vu来提高 LLM 的推理速度", blog explainer at m.haoling.cc
 *   [NOTES] DejaVu reading notes at pages.squarehuang.top/paper/DejaVu
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller, unless the
 *   argument says "host".  The library allocates nothing, frees nothing and keeps no
 *   state between calls apart from one device flag word per GPU (see "Device-side index
 *   trust").  Tensors are dense, row-major, and 16-byte aligned.
 * Types.  Weights and the KV cache are fp32 (DJV_F32) or fp16 (DJV_F16), the same type
 *   for all of them; activations (x, y, outputs, predictor scores) are always fp32;
 *   accumulation is always fp32.
 * Layouts.
 *   y, x, out      [B, d]
 *   Wqkv           [h, 3, dh, d]   block i, part 0/1/2 = (W_i^Q)^T, (W_i^K)^T, (W_i^V)^T
 *   Wo             [h * dh, d]     rows i*dh .. i*dh+dh-1 hold W_i^O
 *   W1, W2         [N, d]          neuron-major: W1[j] is column j of W^1 and W2[j] is
 *                                  row j of (W^2)^T, so a kept neuron is one contiguous row
 *   b1             [N]             first-layer MLP bias (weight dtype)
 *   Kc, Vc         [B, h, n_cap, dh]  per-sequence KV cache; positions 0..n-1 are valid
 *   P1             [r, d], P2 [n_out, r]  a two-layer sparsity predictor
 *   idx            [cap] int32, ascending unit indices; count [1] int32 on the device
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call validates its arguments on the host, enqueues its kernels on `stream` and
 *   returns without synchronising; results are ready when the stream reaches them.
 * Errors.  A call returns DJV_OK or a negative djv_status and sets a thread-local message
 *   (dejavu_last_error).  Argument errors are detected before any HIP call, so they can
 *   be tested on a host without a GPU.  A HIP launch failure returns DJV_EHIP.
 * Device-side index trust.  Index lists and counts produced on the device are checked
 *   by the kernels: an index outside [0, units) contributes nothing and a count above
 *   the list capacity is clamped; both set a flag readable with dejavu_poll_device_error.
 * Workspace.  `ws` is caller-owned device scratch of at least dejavu_workspace_bytes()
 *   bytes for the dimensions of the call (256-byte aligned).  It needs no initial
 *   contents.  Calls that share a workspace must be ordered on one stream.
 */
#ifndef DEJAVU_H
#define DEJAVU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DJV_OK = 0,
    DJV_EINVAL = -1,       /* bad dimension, pointer, mode, k or t */
    DJV_EALIGN = -2,       /* a tensor pointer is not 16-byte aligned (ws: 256) */
    DJV_EWORKSPACE = -3,   /* ws_bytes below dejavu_workspace_bytes() */
    DJV_EUNSUPPORTED = -4, /* valid but outside the library's limits (see each call) */
    DJV_EHIP = -5          /* a HIP runtime call or kernel launch failed */
} djv_status;

/* The two range enumerators make every int a value of the type (also in C++), so an
 * argument outside the listed values is well defined and returns DJV_EINVAL. */
typedef enum {
    DJV_F32 = 0,
    DJV_F16 = 1,
    DJV_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    DJV_DTYPE_RANGE_MAX_ = 2147483647
} djv_dtype;

typedef enum {
    DJV_TOPK = 0,       /* keep the k best-scoring units */
    DJV_THRESHOLD = 1,  /* keep the units whose sigmoid score exceeds t */
    DJV_MODE_RANGE_MIN_ = -2147483647 - 1,
    DJV_MODE_RANGE_MAX_ = 2147483647
} djv_mode;

/* Device flag bits reported by dejavu_poll_device_error. */
#define DJV_FLAG_BAD_INDEX 1u  /* an index list held a value outside [0, units) */
#define DJV_FLAG_BAD_COUNT 2u  /* a device count exceeded its list's capacity */

/* Limits of the library (DJV_EUNSUPPORTED beyond them):
 *   B <= DJV_MAX_BATCH; d and r multiples of 8 with d*esize <= 32768 bytes and
 *   r*esize <= 32768 bytes (one row fits 256 threads x 8 x 16-byte loads); dh in {64, 128};
 *   n_out <= 65536 for selection.
 *   Batches of B <= DJV_MAX_VALU_BATCH rows run on the vector ALU in either dtype.  Larger
 *   batches run their products on the matrix cores and need DJV_F16 weights and every
 *   GEMV row length (d, and r for the predictor) a multiple of 32; their fp16 rounding of
 *   the normalised activations (and of the row-axpy coefficients) is part of the result. */
#define DJV_MAX_BATCH 32
#define DJV_MAX_VALU_BATCH 4

/* --------------------------------------------------------------------------------------
 * dejavu_workspace_bytes -- workspace size for any call with these dimensions or smaller.
 *   All arguments are sizes (host ints); `bytes` is a host pointer.  Pass 0 for a size
 *   the caller will not use.  Returns DJV_EINVAL on a negative size or a NULL `bytes`.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_workspace_bytes(int B, int d, int N, int h, int dh, int r, int n_cap,
                                  size_t* bytes);

/* --------------------------------------------------------------------------------------
 * dejavu_layernorm -- y[b] = (x[b] - mean) / sqrt(var + eps), biased variance, no affine.
 *   [NOTES "LLM Contextually Sparse", third finding: residual blocks with a Norm on the
 *   block input]; pre-LN as in OPT.  x, y: [B, d] fp32 (may alias).  eps > 0.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_layernorm(int B, int d, const float* x, float* y, float eps, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_select -- selection on given scores z [B, n_out] fp32.
 *   [BLOG section 2]: a sigmoid per predictor output makes a select / skip decision;
 *   [BLOG section 1]: keep the best-scoring ~20% of heads / ~5% of neurons.
 *   DJV_TOPK: per row, the k best under (score descending, index ascending), with -0 = +0
 *   and NaN ranked as -inf (0 <= k <= n_out).  DJV_THRESHOLD: per row, {j : z[j] > tau}
 *   with tau = fp32(ln(t / (1 - t))) for 0 < t < 1 (sigmoid(z) > t).  With B > 1 the
 *   result is the union of the rows' sets.  Writes idx[0..count-1] ascending (idx has
 *   room for n_out entries) and count[0].  Bit-exact: depends only on the bits of z.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_select(int B, int n_out, const float* z, djv_mode mode, int k, float t,
                         int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_select_range -- dejavu_select over all n_out units, listing only the kept units j
 *   with lo <= j < hi, as j - lo (a tensor-parallel shard's part of the set, in its own
 *   row numbering; see djv_model's shard fields).  idx has room for hi - lo entries.
 *   0 <= lo <= hi <= n_out (DJV_EINVAL otherwise); the workspace is dejavu_select's.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_select_range(int B, int n_out, const float* z, djv_mode mode, int k, float t,
                               int lo, int hi, int32_t* idx, int32_t* count, void* ws,
                               size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_predict -- sparsity predictor and selection: z = P2 . ReLU(P1 . y[b]) for each b
 *   (fp32 accumulation, scores stored fp32), then dejavu_select(z).
 *   [BLOG section 2]: a two-layer MLP per block type whose output width is the number of
 *   heads or neurons.  P1 [r, d], P2 [n_out, r] in dtype wt.  `logits` (device, may be
 *   NULL) receives z [B, n_out] for bit-exact selection tests.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_predict(djv_dtype wt, int B, int d, int r, int n_out, const float* y,
                          const void* P1, const void* P2, djv_mode mode, int k, float t,
                          int32_t* idx, int32_t* count, float* logits,
                          void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_sparse_mlp -- out[b] = resid[b] + sum_{j in S} ReLU(W1[j] . y[b] + b1[j]) W2[j],
 *   S = idx[0 .. count-1] (count read on the device, at most cap).
 *   [NOTES "Sparsified MLP"]: MLP_{S_M}(y) = sigma(y W^1_{S_M}) (W^2_{S_M})^T; [BLOG
 *   section 3.2]: the kept rows are read in place, fused with the product (one pass over
 *   the weights, no gathered copy).  resid may be NULL (treated as 0) or alias out.
 *   1 <= cap <= N.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_sparse_mlp(djv_dtype wt, int B, int d, int N, const float* y,
                             const void* W1, const void* b1, const void* W2,
                             const int32_t* idx, const int32_t* count, int cap,
                             const float* resid, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_sparse_mlp_no_alloc -- dejavu_sparse_mlp without a workspace, for callers that
 *   cannot allocate device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc).  Same arguments, result and errors as
 *   dejavu_sparse_mlp (bit-identical output), minus ws / ws_bytes: its scratch is a
 *   static device array of DJV_STATIC_SCRATCH_BYTES that each GPU holds until the process
 *   ends, its address taken on the first call on each device.  The call allocates nothing
 *   (no hipMalloc, no library allocation).  A call whose scratch (dejavu_sparse_mlp's
 *   workspace for these B, d, cap) exceeds DJV_STATIC_SCRATCH_BYTES returns
 *   DJV_EUNSUPPORTED before any HIP call; 16 MiB holds, e.g., the OPT-175B-shaped MLP
 *   (d 12288, N 49152) at B = 1 for any cap, and at B <= 4 with 5% of neurons per token.
 *   Every call on a GPU shares that GPU's scratch and leaves its contents to the next
 *   (nothing in it needs to start at zero): calls that overlap on one GPU, on different
 *   streams or threads, race and give undefined results.
 * ------------------------------------------------------------------------------------ */
#define DJV_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
djv_status dejavu_sparse_mlp_no_alloc(djv_dtype wt, int B, int d, int N, const float* y,
                                      const void* W1, const void* b1, const void* W2,
                                      const int32_t* idx, const int32_t* count, int cap,
                                      const float* resid, float* out, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_gather_rows -- the unfused form of the gather, for the fusion ablation:
 *   out[slot * rpu + j] = W[idx[slot] * rpu + j] for slot < count and 0 <= j < rpu, and
 *   zero rows for count <= slot < cap (rows of `cols` elements of dtype wt).
 *   [BLOG section 3.2 "Kernel Fusion"]: without fusion the kept rows are read, written to a
 *   contiguous copy W' and read again by the product (three passes over the kept bytes);
 *   the library's sparse calls never do this, they read the kept rows in place.
 *   W: [units * rpu, cols], out: [cap * rpu, cols] (device; 16-byte aligned when a row is
 *   a multiple of 16 bytes, 4-byte when a multiple of 4, else 2-byte).  idx / count as in
 *   dejavu_sparse_mlp (count NULL: cap).  An index outside [0, units) gives a zero row and
 *   sets DJV_FLAG_BAD_INDEX.  cols >= 1, rpu >= 1, 1 <= cap <= units.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_gather_rows(djv_dtype wt, int rpu, int cols, int units, const void* W,
                              const int32_t* idx, const int32_t* count, int cap, void* out,
                              void* stream);

/* dejavu_dense_mlp -- the same with S = all N neurons (the dense comparison path). */
djv_status dejavu_dense_mlp(djv_dtype wt, int B, int d, int N, const float* y,
                            const void* W1, const void* b1, const void* W2,
                            const float* resid, float* out,
                            void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_sparse_mha -- out[b] = resid[b] + sum_{i in S} H_i(y[b]) W_i^O,
 *   H_i = softmax_t(scale * q_i . K[b,i,t]) V[b,i,t] over t = 0..n, with S =
 *   head_idx[0 .. head_count-1] (at most cap).
 *   [NOTES "Sparsified Attention"]: MHA_{S_A}(y) = sum_{i in S_A} H_i(y) W_i^O, each head
 *   projected by its own d_h x d block and the results summed.  [NOTES "Sparsity operator
 *   for Attention"]: the current token's K/V are computed for the selected heads only
 *   and stored: q_i, k_i, v_i = W_i^{Q,K,V} y, k_i and v_i are rounded to the cache
 *   dtype and written at position n of Kc / Vc (other heads' position n is untouched),
 *   then the token attends over positions 0..n.  0 <= n < n_cap.  resid may be NULL or
 *   alias out.  1 <= cap <= h.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_sparse_mha(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                             const float* y, const void* Wqkv, const void* Wo,
                             void* Kc, void* Vc, const int32_t* head_idx,
                             const int32_t* head_count, int cap, float scale,
                             const float* resid, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/* dejavu_dense_mha -- the same with S = all h heads (the dense comparison path). */
djv_status dejavu_dense_mha(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                            const float* y, const void* Wqkv, const void* Wo,
                            void* Kc, void* Vc, float scale, const float* resid, float* out,
                            void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_neuron_norms -- the neuron scores of the "true" selection: scores[j] =
 *   sqrt(sum_b a[b, j]^2) with a[b, j] = ReLU(W1[j] . y[b] + b1[j]), for all N neurons.
 *   [BLOG section 1 "Contextual Sparsity"]: a dense pass records each neuron's activations
 *   across the tokens and ranks the neurons by the L2 norm of that row; the tokens here
 *   are the B batch rows.  Dense: reads all of W1.  scores [N] fp32 (device).  Select on
 *   them with dejavu_select (one row) to get the true set.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_neuron_norms(djv_dtype wt, int B, int d, int N, const float* y,
                               const void* W1, const void* b1, float* scores,
                               void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_head_norms -- the head scores of the "true" selection: scores[i] =
 *   sqrt(sum_b ||H_i(y[b])||^2), H_i(y[b]) the head's attention output (d_h values, before
 *   the output projection) over positions 0..n as in dejavu_dense_mha, for all h heads.
 *   [BLOG section 1 "Contextual Sparsity"]: each head's output is a matrix (tokens x d_h)
 *   and the heads are ranked by its L2 norm.  Like dejavu_dense_mha it computes every
 *   head's K/V of y and writes them at position n of Kc / Vc.  scores [h] fp32 (device).
 *   Workspace: dejavu_workspace_bytes with these B, d, h, dh, n_cap.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_head_norms(djv_dtype wt, int B, int d, int h, int dh, int n, int n_cap,
                             const float* y, const void* Wqkv, void* Kc, void* Vc, float scale,
                             float* scores, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * Layer and stack descriptors (host structs holding device pointers).
 * ------------------------------------------------------------------------------------ */
typedef struct djv_layer {
    const void* Wqkv; const void* Wo;           /* attention weights */
    const void* W1; const void* b1; const void* W2;  /* MLP weights */
    void* Kc; void* Vc;                         /* this layer's KV cache */
    const void* P1_A; const void* P2_A;         /* head predictor [r,d], [h,r] */
    const void* P1_M; const void* P2_M;         /* neuron predictor [r,d], [N,r] */
    /* Lazy K/V (both NULL: off).  [NOTES "Sparsity operator for Attention"]: a step
     * stores K/V only for its selected heads and keeps its attention input y for the
     * others; a head selected again first gets its missing K/V computed from the kept
     * inputs.  Y [B, n_cap, d] fp32: the layer's y of every position (written at n by each
     * step).  kv_len [2, h] int32: per head, the number of positions whose K/V are valid;
     * a step at position n reads half (n & 1) and writes half ((n + 1) & 1), so set both
     * halves to the filled length (n of the first step) before it.  With lazy K/V every
     * selected head attends over the K/V that computing all heads at every step gives. */
    float* Y; int32_t* kv_len;
} djv_layer;

typedef struct djv_model {
    djv_dtype wt;
    int B, d, N, h, dh, r;
    int n, n_cap;            /* cached length before this step; cache capacity */
    float scale;             /* attention score scale (1/sqrt(dh) for OPT) */
    float eps;               /* LayerNorm epsilon */
    djv_mode mode;           /* selection rule for both predictors */
    int k_A, k_M;            /* top-k sizes (DJV_TOPK) */
    float t_A, t_M;          /* thresholds (DJV_THRESHOLD) */
    /* Tensor-parallel shard (all four 0: unsharded).  The blocks' sums run over heads and
     * neurons ([NOTES "Sparsified MLP"], [NOTES "Sparsified Attention"]), so g GPUs can each
     * hold a contiguous range of them and add their parts.  h_total > 0: the head
     * predictor scores all h_total heads (P2_A [h_total, r]) and selects among them (k_A
     * counts over all), and this model's Wqkv, Wo, Kc, Vc hold the h heads from h_offset;
     * its head list holds the kept heads of that range, as head - h_offset.  N_total,
     * N_offset: the same for the neurons (P2_M [N_total, r]; W1, b1, W2 hold the N
     * neurons from N_offset).  Each block then adds the shard's part of its sum to x; the
     * sum of the parts over shards (an all-reduce between blocks, not made here) is the
     * unsharded block.  Traces: z_A [L, B, h_total], z_M [L, B, N_total], sets local. */
    int h_total, h_offset, N_total, N_offset;
} djv_model;

/* Optional per-layer trace for tests (device pointers, each may be NULL):
 *   x_in [L, B, d]: each layer's input x; x_mid [L, B, d]: each layer's x' (after
 *   attention); z_A [L, B, h] / z_M [L, B, N] (h_total / N_total for a shard): the
 *   predictor scores the layer's sets were
 *   selected from; sets_A [L, h] / sets_M [L, N]: the selected index lists (first
 *   counts[l, 0] / counts[l, 1] entries valid); counts [L, 2]. */
typedef struct djv_trace {
    float* x_in; float* x_mid; float* z_A; float* z_M;
    int32_t* sets_A; int32_t* sets_M; int32_t* counts;
} djv_trace;

/* --------------------------------------------------------------------------------------
 * dejavu_sparse_layer -- one sparse decoder layer, serial prediction ([BLOG section 2]:
 *   predict heads, sparse attention, predict neurons, sparse MLP):
 *   S_A = select(SP_A(LN(x))); x' = x + MHA_{S_A}(LN(x));
 *   S_M = select(SP_M(LN(x'))); x <- x' + MLP_{S_M}(LN(x')).
 *   x [B, d] is updated in place.  trace may be NULL.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_sparse_layer(const djv_model* m, const djv_layer* layer, float* x,
                               const djv_trace* trace, void* ws, size_t ws_bytes,
                               void* stream);

/* --------------------------------------------------------------------------------------
 * dejavu_stack_decode -- one decode step through L layers (x [B, d] updated in place).
 *   lookahead = 1 ([BLOG section 3.1], [NOTES "Reducing Overhead with Asynchronous
 *   Execution"]): layer l+1's sets are predicted from y_l = LN(x_l) while layer l
 *   computes; layer 0's sets are predicted first from LN(x_0).  The overlap is inside
 *   launches on the one stream: the predictor weights stream in the same launches as
 *   layer l's weights and each selection runs in a side block of a later launch.
 *   With lookahead, B <= DJV_MAX_VALU_BATCH (vector ALU) and dejavu_set_deterministic
 *   off (the default), the residual stream stays in x between
 *   launches: the attention and MLP outputs are added to it with fp32 atomics, so no
 *   reduction launch follows either output projection, and the kernels that read LN(x)
 *   compute its moments themselves.  The order of those additions depends on scheduling,
 *   so two runs may differ in the last bits of x (and, through them, in the sets of later
 *   layers where two scores nearly tie); with dejavu_set_deterministic(1) the partial sums
 *   are reduced in a fixed order instead and every run gives the same bits.
 *   lookahead = 0: each layer as dejavu_sparse_layer.
 *   dense = 1: every layer dense (all heads and neurons, no predictor).
 *   layers: host array of L descriptors.  Everything is enqueued on `stream`; nothing is
 *   allocated and nothing waits on the host.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_stack_decode(const djv_model* m, const djv_layer* layers, int L, float* x,
                               int lookahead, int dense, const djv_trace* trace,
                               void* ws, size_t ws_bytes, void* stream);

/* dejavu_workspace_bytes_model -- workspace for dejavu_sparse_layer / dejavu_stack_decode. */
djv_status dejavu_workspace_bytes_model(const djv_model* m, size_t* bytes);

/* --------------------------------------------------------------------------------------
 * dejavu_poll_device_error -- synchronises `stream`, copies the current device's flag
 *   word (one per GPU, shared by every call on it; zero at load) to *flags (host) and
 *   clears it.  Returns DJV_EHIP on a HIP error, DJV_EINVAL if flags is NULL.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_poll_device_error(void* stream, uint32_t* flags);

/* --------------------------------------------------------------------------------------
 * dejavu_set_mfma_min_batch -- kernel form by batch size.  Calls whose batch has at least
 *   `b` rows run their GEMVs and row-axpys on the matrix cores where that form applies
 *   (DJV_F16 weights and every GEMV row length a multiple of 32); other calls with
 *   B <= DJV_MAX_VALU_BATCH use the vector-ALU kernels.  Batches above DJV_MAX_VALU_BATCH
 *   always use the matrix cores.  Default DJV_MAX_VALU_BATCH + 1; b must lie in
 *   [1, DJV_MAX_VALU_BATCH + 1] (DJV_EINVAL otherwise).  *previous (host, may be NULL)
 *   receives the value replaced.  Process-wide; each call reads it once when it plans its
 *   launches, so a change does not affect work already enqueued.  Workspace sizes do not
 *   depend on it.  The matrix-core form rounds the normalised activations and the
 *   row-axpy coefficients to fp16.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_set_mfma_min_batch(int b, int* previous);

/* --------------------------------------------------------------------------------------
 * dejavu_set_deterministic -- on = 1: every call gives the same bits for the same inputs
 *   (the lookahead stack reduces its output-projection partial sums in a fixed order, one
 *   extra launch after each projection).  on = 0 (default): the lookahead stack adds them
 *   to the residual stream with atomics (see dejavu_stack_decode).  Other calls are always
 *   reproducible.  *previous (host, may be NULL) receives the value replaced; DJV_EINVAL
 *   unless on is 0 or 1.  Process-wide, read once per call when it plans its launches.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_set_deterministic(int on, int* previous);

/* --------------------------------------------------------------------------------------
 * Benchmark hook.  dejavu_profile_kernel(family, events, capacity): from now on, every
 *   launch of the given kernel family records events[2i] just before and events[2i+1]
 *   just after the i-th such launch, on that launch's stream, for i < capacity (later
 *   launches are not recorded).  events: host array of 2*capacity hipEvent_t (as void*)
 *   created by the caller with timing enabled; it must stay valid until the hook is
 *   switched off with DJV_PROF_OFF.  Setting a family resets the count.  One hook per
 *   process, not thread-safe; it enqueues nothing itself.
 *   dejavu_profile_count(count): launches recorded since the family was set (host int).
 * ------------------------------------------------------------------------------------ */
#define DJV_PROF_OFF 0
#define DJV_PROF_QKV 1        /* head-sparse Q/K/V GEMV with the KV append */
#define DJV_PROF_MLP_UP 2     /* gather-GEMV over the kept W1 rows */
#define DJV_PROF_MLP_DOWN 3   /* row-axpy over the kept W2 rows (partial tiles) */
#define DJV_PROF_O_PROJ 4     /* row-axpy over the kept heads' W_O rows (partial tiles) */
#define DJV_PROF_ATTN 5       /* split-position attention (partial chunks) */
#define DJV_PROF_PRED_1 6     /* predictor first layer d -> r */
#define DJV_PROF_PRED_2 7     /* predictor second layer r -> n_out */
#define DJV_PROF_SELECT 8     /* per-row selection */
djv_status dejavu_profile_kernel(int family, void* const* events, int capacity);
djv_status dejavu_profile_count(int* count);

/* --------------------------------------------------------------------------------------
 * dejavu_read_probe -- benchmark reference: reads `bytes` of buf once with 16-byte
 *   non-temporal loads (the load form of the weight streams above), every block of a
 *   grid of 8 blocks per compute unit streaming one contiguous share, and folds the data
 *   into one word.  out (device, one
 *   uint32) is written only when that word equals an arbitrary fixed value, which keeps
 *   the loads from being removed; its contents are not a result.  The rate of this call
 *   is the plain HBM read rate that the sparse layer's rate on its touched bytes is
 *   compared with.  buf: device, 16-byte aligned, bytes a positive multiple of 16 (else
 *   DJV_EINVAL / DJV_EALIGN).  Enqueues one kernel on `stream`.
 * ------------------------------------------------------------------------------------ */
djv_status dejavu_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* dejavu_last_error -- message of this thread's last failing call ("" if none). */
const char* dejavu_last_error(void);

/* dejavu_version -- library version string. */
const char* dejavu_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DEJAVU_H */
