"""Deja Vu contextually sparse decode layer: plain, slow float64 CPU oracle.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP library
(``contextual_sparsity_amd``) and imports nothing from it; the library never
imports this module.

Arithmetic.  Every value read from an input array is converted exactly to
float64 (fp16 and fp32 are subsets of fp64) and all arithmetic is float64.  A
value is rounded to a narrower type only where the method stores it in one:
the new K/V cache rows (round-to-nearest-even to the cache dtype) and the
predictor scores (rounded once to fp32, the type selection works on).  Matrix
products, sums, ``exp`` and sorting are library primitives used as single
steps; nothing is blocked, fused or reordered beyond the formulas.

Sources (each function names the passage it follows):
  [BLOG]  "用Deja Vu来提高 LLM 的推理速度", blog explainer at m.haoling.cc
  [ABS]   "Deja Vu: Contextual Sparsity for Efficient LLMs at Inference Time",
          paper summary page at shd-paper.top (English abstract)
  [NOTES] DejaVu reading notes at pages.squarehuang.top/paper/DejaVu

Storage conventions (the pages write row vectors times d x d_h matrices; the
stored layouts below hold the same numbers, transposed where noted):
  y, x       [B, d]            activations, one row per sequence in the batch
  Wqkv       [h, 3, d_h, d]    Wqkv[i, 0] = (W_i^Q)^T, [i, 1] = (W_i^K)^T, [i, 2] = (W_i^V)^T
  Wo         [h * d_h, d]      rows i*d_h .. i*d_h+d_h-1 are W_i^O (d_h x d)
  W1         [N, d]            W1[j] = column j of W^1 (neuron-major, N = 4d)
  b1         [N]
  W2         [N, d]            W2[j] = column j of W^2, i.e. row j of (W^2)^T
  K, V       [B, h, n_cap, d_h] per-sequence cache; positions 0..n-1 hold past tokens
  P1         [r, d], P2 [n_out, r]   two-layer sparsity predictor

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
(closed forms, worked fixtures under ``tests/golden/``, brute force, invariants)
except where its docstring says "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

LN_EPS = 1e-5

TOPK = 0
THRESHOLD = 1


def _f64(a) -> np.ndarray:
    """Exact widening of fp16 / fp32 / fp64 data to float64."""
    return np.asarray(a).astype(np.float64)


# --------------------------------------------------------------------------------------
# Keep counts
# --------------------------------------------------------------------------------------
def keep_count(pct, n: int) -> int:
    """Number of units kept at a keep-percentage: k = ceil(pct * n / 100), exactly.

    [BLOG §1 "Contextual Sparsity"]: about 20% of attention heads and about 5% of MLP
    neurons are kept.  The rounding is not stated; ceiling is the reading that keeps
    3 of 12 heads at 20% (nearest would keep 2) and 154 of 3072 neurons at 5%.  The
    ceiling is taken in rational arithmetic so exact multiples do not round up
    (5% of 16000 is 800, not 801).
    """
    p = Fraction(str(pct)) if isinstance(pct, float) else Fraction(pct)
    if p < 0 or p > 100 or n < 0:
        raise ValueError("pct must lie in [0, 100] and n >= 0")
    return math.ceil(p * n / 100)


# --------------------------------------------------------------------------------------
# LayerNorm (pre-LN residual block)
# --------------------------------------------------------------------------------------
def layernorm(x, eps: float = LN_EPS) -> np.ndarray:
    """Row-wise LayerNorm without affine terms: (x - mean) / sqrt(var + eps).

    [NOTES "LLM Contextually Sparse" third finding]: blocks are residual, y = F(x) + x,
    with a Norm on the block input.  Reading: pre-LN as in OPT, biased variance,
    eps = 1e-5, gamma = 1, beta = 0.
    """
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


# --------------------------------------------------------------------------------------
# Sparsity predictor
# --------------------------------------------------------------------------------------
def predictor_logits_f64(y, P1, P2) -> np.ndarray:
    """Two-layer predictor, before rounding: z = P2 . ReLU(P1 . y) for every row of y.

    [BLOG §2 "稀疏性预测"]: each of the two predictors is a two-layer MLP whose output
    width is the number of heads (or neurons), with a sigmoid per output acting as a
    select / skip classifier.  [NOTES "Deja Vu Framework"]: one such predictor per
    block, fed the block's input embedding.  Readings: ReLU hidden activation, no
    biases; the sigmoid is monotone and is folded into the selection rule.
    """
    y = _f64(y)
    u = np.maximum(0.0, y @ _f64(P1).T)
    return u @ _f64(P2).T


def predictor_logits(y, P1, P2) -> np.ndarray:
    """Predictor scores rounded once to fp32, the type selection operates on."""
    return predictor_logits_f64(y, P1, P2).astype(np.float32)


# --------------------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------------------
def rank_order(z_row) -> np.ndarray:
    """Indices ordered best first: higher score first, lower index first among equals.

    NaN counts as -inf and -0 as +0, so the order (and therefore every top-k set) is
    unique.  This order is the reading adopted for ties, which the pages leave open.
    """
    z = _f64(np.asarray(z_row, dtype=np.float32))
    z = np.where(np.isnan(z), -np.inf, z) + 0.0
    return np.argsort(-z, kind="stable")


def topk_set(z_row, k: int) -> np.ndarray:
    """The k best-ranked indices of one score row, returned in ascending index order.

    [BLOG §1]: keep the heads / neurons with the largest scores.  [BLOG §2]: the
    predictor's per-output sigmoid scores rank them; sigmoid is monotone, so ranking
    the fp32 logits is the same order without fp32 saturation at 1.0.
    """
    n = len(z_row)
    if not (0 <= k <= n):
        raise ValueError("k must lie in [0, n_out]")
    return np.sort(rank_order(z_row)[:k]).astype(np.int32)


def logit_threshold(t) -> np.float32:
    """tau = fp32(ln(t / (1 - t))) for the fp32 probability t, computed in float64."""
    t = float(np.float32(t))
    if not (0.0 < t < 1.0):
        raise ValueError("t must lie in (0, 1)")
    return np.float32(math.log(t / (1.0 - t)))


def threshold_set(z_row, t) -> np.ndarray:
    """Indices whose predicted probability sigmoid(z) exceeds t, ascending.

    [BLOG §2]: each predictor output is a binary select / skip decision from a sigmoid,
    labelled in training by a threshold t.  sigmoid(z) > t  <=>  z > logit(t); the
    comparison is strict and made in fp32 against fp32(logit t).  NaN is never selected.
    """
    tau = logit_threshold(t)
    z = np.asarray(z_row, dtype=np.float32)
    return np.flatnonzero(z > tau).astype(np.int32)


def select(z, mode: int, k: int = 0, t: float = 0.5) -> np.ndarray:
    """Per-token selection, then the union over the batch, in ascending index order.

    z is [B, n_out] fp32.  For B > 1 the pages are silent; the reading used here is
    that every token is selected on its own and the batch computes with the union.
    """
    z = np.asarray(z, dtype=np.float32)
    if z.ndim == 1:
        z = z[None, :]
    sets = []
    for row in z:
        sets.append(topk_set(row, k) if mode == TOPK else threshold_set(row, t))
    if not sets:
        return np.zeros(0, dtype=np.int32)
    return np.unique(np.concatenate(sets)).astype(np.int32)


# --------------------------------------------------------------------------------------
# Sparsified MLP  [NOTES "Sparsified MLP"]
# --------------------------------------------------------------------------------------
def sparse_mlp(y, W1, b1, W2, S_M) -> np.ndarray:
    """MLP_{S_M}(y) = sigma(y W^1_{S_M} + b1_{S_M}) (W^2_{S_M})^T, sigma = ReLU.

    [NOTES "Sparsified MLP"]: only the neuron subset S_M of the 4d hidden units is
    computed.  W1 and W2 are neuron-major, so the subset is the rows S_M of each.
    b1 is the first-layer bias of the neurons in S_M (no second-layer bias).
    """
    y = _f64(y)
    S = np.asarray(S_M, dtype=np.int64)
    a = np.maximum(0.0, y @ _f64(W1[S]).T + _f64(b1[S])[None, :])
    return a @ _f64(W2[S])


def dense_mlp(y, W1, b1, W2) -> np.ndarray:
    """Textbook dense MLP: ReLU(y W^1 + b1) (W^2)^T over all 4d neurons, no subset."""
    y = _f64(y)
    hidden = np.maximum(0.0, y @ _f64(W1).T + _f64(b1)[None, :])
    return hidden @ _f64(W2)


# --------------------------------------------------------------------------------------
# Sparsified attention  [NOTES "Sparsified Attention"]
# --------------------------------------------------------------------------------------
def _round_to(v: np.ndarray, dtype) -> np.ndarray:
    """Round float64 values once to the storage dtype (round-to-nearest-even)."""
    return np.asarray(v, dtype=np.float64).astype(dtype)


def _attend(q, keys, values, scale) -> np.ndarray:
    """D^{-1} exp(s) V over the given keys: s_t = scale * q . k_t.

    The max is subtracted before exp; this cancels between numerator and D exactly.
    """
    s = scale * (keys @ q)
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def sparse_mha(y, Wqkv, Wo, K, V, n: int, S_A, scale: float):
    """MHA_{S_A}(y) = sum over i in S_A of H_i(y) W_i^O for each sequence in the batch.

    [NOTES "Sparsified Attention"]: H_i(y) = D_i(y)^{-1} exp(y W_i^Q (W_i^K)^T X^T) X W_i^V
    with X the past tokens; the head outputs are projected per head and summed.
    [NOTES "Sparsity operator for Attention"]: the current token's K/V are computed
    for the predicted heads and stored into the cache; heads outside S_A are not
    touched.  Readings: the new key/value are rounded to the cache dtype and appended
    at position n, then the token attends over positions 0..n; ``scale`` multiplies
    the scores (1/sqrt(d_h) in the configurations, 1 for the literal formula).

    Returns (out [B, d] float64, K_new [B, |S_A|, d_h], V_new [B, |S_A|, d_h]) where the
    new rows are in the cache dtype.
    """
    y = _f64(y)
    B, d = y.shape
    h, three, dh, d2 = Wqkv.shape
    assert three == 3 and d2 == d
    S = [int(i) for i in S_A]
    out = np.zeros((B, d))
    k_new = np.zeros((B, len(S), dh), dtype=K.dtype)
    v_new = np.zeros((B, len(S), dh), dtype=V.dtype)
    for b in range(B):
        for slot, i in enumerate(S):
            q = _f64(Wqkv[i, 0]) @ y[b]
            k = _f64(Wqkv[i, 1]) @ y[b]
            v = _f64(Wqkv[i, 2]) @ y[b]
            k_new[b, slot] = _round_to(k, K.dtype)
            v_new[b, slot] = _round_to(v, V.dtype)
            keys = np.concatenate([_f64(K[b, i, :n]), _f64(k_new[b, slot])[None, :]])
            vals = np.concatenate([_f64(V[b, i, :n]), _f64(v_new[b, slot])[None, :]])
            H = _attend(q, keys, vals, scale)
            out[b] += H @ _f64(Wo[i * dh:(i + 1) * dh])
    return out, k_new, v_new


def dense_mha(y, Wqkv, Wo, K, V, n: int, scale: float):
    """Textbook dense multi-head attention for one decode step: all heads, heads
    concatenated, then one product with the full output projection.

    Written independently of ``sparse_mha`` (concatenation instead of a per-head sum)
    so that ``sparse_mha`` with S_A = all heads can be checked against it.
    Returns (out [B, d], K_new [B, h, d_h], V_new [B, h, d_h]).
    """
    y = _f64(y)
    B, d = y.shape
    h, _, dh, _ = Wqkv.shape
    Wq = _f64(Wqkv[:, 0]).reshape(h * dh, d)
    Wk = _f64(Wqkv[:, 1]).reshape(h * dh, d)
    Wv = _f64(Wqkv[:, 2]).reshape(h * dh, d)
    Q = (y @ Wq.T).reshape(B, h, dh)
    Kn = _round_to((y @ Wk.T).reshape(B, h, dh), K.dtype)
    Vn = _round_to((y @ Wv.T).reshape(B, h, dh), V.dtype)
    Hcat = np.zeros((B, h * dh))
    for b in range(B):
        for i in range(h):
            keys = np.concatenate([_f64(K[b, i, :n]), _f64(Kn[b, i])[None, :]])
            vals = np.concatenate([_f64(V[b, i, :n]), _f64(Vn[b, i])[None, :]])
            logits = scale * (keys @ Q[b, i])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            Hcat[b, i * dh:(i + 1) * dh] = p @ vals
    return Hcat @ _f64(Wo), Kn, Vn


def cache_after_steps(Wqkv, K0, V0, n0: int, ys) -> Tuple[np.ndarray, np.ndarray]:
    """The K/V cache after decode steps at positions n0, n0+1, ... with attention inputs
    ys[t] [B, d]: positions below n0 as in K0 / V0, position n0 + t holding every head's
    round(W_i^K ys[t]) and round(W_i^V ys[t]) in the cache dtype.

    [NOTES "Sparsity operator for Attention"]: a step stores K/V only for its selected
    heads and keeps y for the others, recomputing their K/V from it when they are
    selected later; a head attending at a later step therefore sees exactly these
    entries.  This is the plain definition that lazy recomputation must reach.
    """
    K, V = np.array(K0, copy=True), np.array(V0, copy=True)
    for t, y in enumerate(ys):
        y = _f64(y)
        k = np.einsum("icd,bd->bic", _f64(Wqkv[:, 1]), y)
        v = np.einsum("icd,bd->bic", _f64(Wqkv[:, 2]), y)
        K[:, :, n0 + t] = _round_to(k, K.dtype)
        V[:, :, n0 + t] = _round_to(v, V.dtype)
    return K, V


# --------------------------------------------------------------------------------------
# "True" selection by output norm  [BLOG §1 "Contextual Sparsity"]
# --------------------------------------------------------------------------------------
def neuron_norms(y, W1, b1) -> np.ndarray:
    """Per-neuron score: the L2 norm of the neuron's activations across the tokens.

    [BLOG §1]: for the MLP the norm is not taken of a token's output vector; the MLP acts
    per position, so its hidden activations form a (neurons x tokens) matrix and each
    neuron is scored by the norm of its row.  The tokens of one decode step are the batch
    rows of y.  Returns [N] float64.
    """
    y = _f64(y)
    a = np.maximum(0.0, y @ _f64(W1).T + _f64(b1)[None, :])  # [B, N]
    return np.sqrt((a * a).sum(axis=0))


def head_norms(y, Wqkv, K, V, n: int, scale: float) -> np.ndarray:
    """Per-head score: the L2 (Frobenius) norm of the head's output matrix over the tokens.

    [BLOG §1]: each head's output is a matrix (tokens x d_h, the head's slice of the
    attention output before the output projection), scored by its L2 norm.  H_i is the
    head's attention over positions 0..n with its own K/V of y appended at position n
    (rounded to the cache dtype), as in ``sparse_mha``.  Returns [h] float64.
    """
    y = _f64(y)
    B = y.shape[0]
    h = Wqkv.shape[0]
    sq = np.zeros(h)
    for i in range(h):
        for b in range(B):
            q = _f64(Wqkv[i, 0]) @ y[b]
            k = _round_to(_f64(Wqkv[i, 1]) @ y[b], K.dtype)
            v = _round_to(_f64(Wqkv[i, 2]) @ y[b], V.dtype)
            keys = np.concatenate([_f64(K[b, i, :n]), _f64(k)[None, :]])
            vals = np.concatenate([_f64(V[b, i, :n]), _f64(v)[None, :]])
            H = _attend(q, keys, vals, scale)
            sq[i] += float(H @ H)
    return np.sqrt(sq)


def recall(S_pred, S_true) -> float:
    """Share of the true set that the predicted set holds: |S_pred & S_true| / |S_true|
    (1.0 for an empty true set)."""
    t = set(int(j) for j in S_true)
    if not t:
        return 1.0
    return len(t & set(int(j) for j in S_pred)) / len(t)


# --------------------------------------------------------------------------------------
# Layer and stack
# --------------------------------------------------------------------------------------
@dataclass
class LayerWeights:
    """One decoder layer's weights and KV cache (arrays in their stored dtypes)."""
    Wqkv: np.ndarray
    Wo: np.ndarray
    W1: np.ndarray
    b1: np.ndarray
    W2: np.ndarray
    K: np.ndarray
    V: np.ndarray


@dataclass
class PredictorWeights:
    """The attention-head predictor (P1_A, P2_A) and the neuron predictor (P1_M, P2_M)."""
    P1_A: np.ndarray
    P2_A: np.ndarray
    P1_M: np.ndarray
    P2_M: np.ndarray


def sparse_layer(x, L: LayerWeights, S_A, S_M, n: int, scale: float):
    """One pre-LN decoder layer with sparse blocks.

    x' = x + MHA_{S_A}(LN(x));  x'' = x' + MLP_{S_M}(LN(x')).
    [NOTES "Typical LLM procedure"]: generation runs attention then MLP per layer
    reading and updating the KV cache; [NOTES third finding]: residual blocks.
    Returns (x'', x', K_new, V_new).
    """
    x = _f64(x)
    att, kn, vn = sparse_mha(layernorm(x), L.Wqkv, L.Wo, L.K, L.V, n, S_A, scale)
    x1 = x + att
    x2 = x1 + sparse_mlp(layernorm(x1), L.W1, L.b1, L.W2, S_M)
    return x2, x1, kn, vn


def dense_layer(x, L: LayerWeights, n: int, scale: float):
    """The dense decoder layer (all heads, all neurons); returns (x'', x')."""
    x = _f64(x)
    att, _, _ = dense_mha(layernorm(x), L.Wqkv, L.Wo, L.K, L.V, n, scale)
    x1 = x + att
    x2 = x1 + dense_mlp(layernorm(x1), L.W1, L.b1, L.W2)
    return x2, x1


# --------------------------------------------------------------------------------------
# Tensor-parallel shards  [NOTES "Sparsified MLP"], [NOTES "Sparsified Attention"]
# --------------------------------------------------------------------------------------
def shard_set(S, lo: int, hi: int) -> np.ndarray:
    """The part of a selected set that falls in a shard's unit range [lo, hi), renumbered
    from the shard's first unit: {j - lo : j in S, lo <= j < hi}, ascending.

    Both sparse blocks are sums over the kept units (MLP_{S_M} over neurons, MHA_{S_A}
    over heads), so a shard holding a contiguous range of units computes the terms of its
    own kept units; the pages do not discuss several GPUs, this is that sum split by
    ranges.  Every shard selects from the same global scores.
    """
    S = np.asarray(S, dtype=np.int64)
    return (S[(S >= lo) & (S < hi)] - lo).astype(np.int32)


def shard_ranges(n: int, g: int) -> list:
    """g contiguous ranges covering 0..n-1, the first n % g one unit longer."""
    base, extra = divmod(n, g)
    out, lo = [], 0
    for i in range(g):
        hi = lo + base + (1 if i < extra else 0)
        out.append((lo, hi))
        lo = hi
    return out


def shard_layer_weights(L: "LayerWeights", h_lo: int, h_hi: int, n_lo: int, n_hi: int, dh: int):
    """The rows of one shard: heads h_lo..h_hi-1 (their Wqkv blocks, Wo rows and caches)
    and neurons n_lo..n_hi-1 (W1, b1, W2 rows)."""
    return LayerWeights(Wqkv=L.Wqkv[h_lo:h_hi], Wo=L.Wo[h_lo * dh:h_hi * dh], W1=L.W1[n_lo:n_hi],
                        b1=L.b1[n_lo:n_hi], W2=L.W2[n_lo:n_hi], K=L.K[:, h_lo:h_hi],
                        V=L.V[:, h_lo:h_hi])


@dataclass
class Selection:
    """Selection rule shared by both predictors of a layer."""
    mode: int = TOPK
    k_A: int = 0
    k_M: int = 0
    t_A: float = 0.5
    t_M: float = 0.5


def predict_sets(y, P: PredictorWeights, sel: Selection) -> Tuple[np.ndarray, np.ndarray]:
    """(S_A, S_M) predicted from one input embedding y by both predictors."""
    zA = predictor_logits(y, P.P1_A, P.P2_A)
    zM = predictor_logits(y, P.P1_M, P.P2_M)
    return (select(zA, sel.mode, sel.k_A, sel.t_A), select(zM, sel.mode, sel.k_M, sel.t_M))


def serial_layer(x, L: LayerWeights, P: PredictorWeights, sel: Selection, n: int, scale: float):
    """The naive serial block of [BLOG §2]: predict heads, sparse MHA, predict neurons,
    sparse MLP, in that order.  The head predictor reads LN(x) (the attention input),
    the neuron predictor reads LN(x') (the MLP input).

    Returns (x'', x', S_A, S_M, K_new, V_new).
    """
    x = _f64(x)
    y = layernorm(x)
    S_A = select(predictor_logits(y, P.P1_A, P.P2_A), sel.mode, sel.k_A, sel.t_A)
    att, kn, vn = sparse_mha(y, L.Wqkv, L.Wo, L.K, L.V, n, S_A, scale)
    x1 = x + att
    y1 = layernorm(x1)
    S_M = select(predictor_logits(y1, P.P1_M, P.P2_M), sel.mode, sel.k_M, sel.t_M)
    x2 = x1 + sparse_mlp(y1, L.W1, L.b1, L.W2, S_M)
    return x2, x1, S_A, S_M, kn, vn


def lookahead_stack(x0, layers: Sequence[LayerWeights], preds: Sequence[PredictorWeights],
                    sel: Selection, n: int, scale: float):
    """A stack of sparse layers with the asynchronous lookahead predictor.

    [BLOG §3.1 "并行化稀疏性预测"] and [NOTES "Reducing Overhead with Asynchronous
    Execution"]: the sets of layer l+1 are predicted from layer l's input while layer
    l computes, since embeddings change slowly across layers.  Readings: the
    predictor of layer l+1 reads y_l = LN(x_l), the embedding layer l's attention
    reads; layer 0's sets are predicted serially from LN(x_0).

    Returns (x_L, xs, sets) with xs[l] the input of layer l (xs[L] = x_L) and
    sets[l] = (S_A^l, S_M^l).  parity unpinned beyond its parts and the schedule pin:
    no worked multi-layer example exists on the pages.
    """
    x = _f64(x0)
    nl = len(layers)
    xs = [x]
    sets: List[Optional[Tuple[np.ndarray, np.ndarray]]] = [None] * nl
    if nl == 0:
        return x, xs, []
    sets[0] = predict_sets(layernorm(x), preds[0], sel)
    for l in range(nl):
        y = layernorm(x)
        if l + 1 < nl:
            sets[l + 1] = predict_sets(y, preds[l + 1], sel)
        S_A, S_M = sets[l]
        x, _, _, _ = sparse_layer(x, layers[l], S_A, S_M, n, scale)
        xs.append(x)
    return x, xs, sets
