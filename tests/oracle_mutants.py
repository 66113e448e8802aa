"""Plausible mistakes planted in the float64 oracle, on the CPU, for the mutation test.

Loaded as a pytest plugin (``-p oracle_mutants``) with DJV_ORACLE_MUTANT naming one
entry of MUTANTS: it replaces that oracle function, in the oracle module and in the
package namespace the tests use, with a version carrying one slip (a dropped term, a
wrong sign or index, a wrong tie rule, a wrong rounding).  tests/test_oracle_mutations.py
runs the oracle's pin tests under each mutant and requires them to fail."""
import math
import os

import numpy as np

import oracle
import oracle.dejavu_oracle as D

_f64 = D._f64


def _ln_unbiased(x, eps=D.LN_EPS):
    x = _f64(x)
    return (x - x.mean(axis=-1, keepdims=True)) / np.sqrt(x.var(axis=-1, ddof=1, keepdims=True) + eps)


def _ln_no_eps(x, eps=D.LN_EPS):
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True))


def _pred_no_relu(y, P1, P2):
    return (_f64(y) @ _f64(P1).T) @ _f64(P2).T


def _pred_relu_after(y, P1, P2):
    return np.maximum(0.0, (_f64(y) @ _f64(P1).T) @ _f64(P2).T)


def _rank_high_index_first(z_row):
    z = _f64(np.asarray(z_row, dtype=np.float32))
    z = np.where(np.isnan(z), -np.inf, z) + 0.0
    n = len(z)
    return np.array(sorted(range(n), key=lambda j: (-z[j], -j)), dtype=np.int64)


def _rank_nan_first(z_row):
    z = _f64(np.asarray(z_row, dtype=np.float32))
    z = np.where(np.isnan(z), np.inf, z) + 0.0
    return np.argsort(-z, kind="stable")


def _topk_one_short(z_row, k):
    return np.sort(D.rank_order(z_row)[:max(k - 1, 0)]).astype(np.int32)


def _topk_unsorted(z_row, k):
    return D.rank_order(z_row)[:k].astype(np.int32)


def _threshold_ge(z_row, t):
    tau = D.logit_threshold(t)
    return np.flatnonzero(np.asarray(z_row, dtype=np.float32) >= tau).astype(np.int32)


def _logit_inverted(t):
    t = float(np.float32(t))
    return np.float32(math.log((1.0 - t) / t))


def _keep_round(pct, n):
    return int(round(float(pct) * n / 100))


def _select_intersection(z, mode, k=0, t=0.5):
    z = np.asarray(z, dtype=np.float32)
    if z.ndim == 1:
        z = z[None, :]
    sets = [set(D.topk_set(r, k) if mode == D.TOPK else D.threshold_set(r, t)) for r in z]
    return np.array(sorted(set.intersection(*sets)), dtype=np.int32)


def _mlp_no_bias(y, W1, b1, W2, S_M):
    S = np.asarray(S_M, dtype=np.int64)
    return np.maximum(0.0, _f64(y) @ _f64(W1[S]).T) @ _f64(W2[S])


def _mlp_no_relu(y, W1, b1, W2, S_M):
    S = np.asarray(S_M, dtype=np.int64)
    return (_f64(y) @ _f64(W1[S]).T + _f64(b1[S])[None, :]) @ _f64(W2[S])


def _attend_unnormalised(q, keys, values, scale):
    s = scale * (keys @ q)
    return np.exp(s - s.max()) @ values


def _attend_scale_twice(q, keys, values, scale):
    s = scale * scale * (keys @ q)
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def _mha_variant(slot_rows=False, no_append=False, no_round=False):
    def f(y, Wqkv, Wo, K, V, n, S_A, scale):
        y = _f64(y)
        B, d = y.shape
        dh = Wqkv.shape[2]
        S = [int(i) for i in S_A]
        out = np.zeros((B, d))
        k_new = np.zeros((B, len(S), dh), dtype=K.dtype)
        v_new = np.zeros((B, len(S), dh), dtype=V.dtype)
        for b in range(B):
            for slot, i in enumerate(S):
                q = _f64(Wqkv[i, 0]) @ y[b]
                k = _f64(Wqkv[i, 1]) @ y[b]
                v = _f64(Wqkv[i, 2]) @ y[b]
                k_new[b, slot] = D._round_to(k, K.dtype)
                v_new[b, slot] = D._round_to(v, V.dtype)
                kk, vv = (k, v) if no_round else (_f64(k_new[b, slot]), _f64(v_new[b, slot]))
                keys, vals = _f64(K[b, i, :n]), _f64(V[b, i, :n])
                if not no_append:
                    keys = np.concatenate([keys, kk[None, :]])
                    vals = np.concatenate([vals, vv[None, :]])
                H = D._attend(q, keys, vals, scale) if len(keys) else np.zeros(dh)
                r = slot if slot_rows else i
                out[b] += H @ _f64(Wo[r * dh:(r + 1) * dh])
        return out, k_new, v_new
    return f


MUTANTS = {
    "layernorm_unbiased_variance": ("layernorm", _ln_unbiased),
    "layernorm_without_eps": ("layernorm", _ln_no_eps),
    "predictor_without_relu": ("predictor_logits_f64", _pred_no_relu),
    "predictor_relu_after_second_layer": ("predictor_logits_f64", _pred_relu_after),
    "ties_higher_index_first": ("rank_order", _rank_high_index_first),
    "nan_ranked_first": ("rank_order", _rank_nan_first),
    "topk_one_short": ("topk_set", _topk_one_short),
    "topk_not_ascending": ("topk_set", _topk_unsorted),
    "threshold_not_strict": ("threshold_set", _threshold_ge),
    "logit_inverted": ("logit_threshold", _logit_inverted),
    "keep_count_rounds_to_nearest": ("keep_count", _keep_round),
    "batch_intersection_not_union": ("select", _select_intersection),
    "mlp_without_bias": ("sparse_mlp", _mlp_no_bias),
    "mlp_without_relu": ("sparse_mlp", _mlp_no_relu),
    "softmax_not_normalised": ("_attend", _attend_unnormalised),
    "softmax_scale_applied_twice": ("_attend", _attend_scale_twice),
    "output_projection_rows_of_slot_not_head": ("sparse_mha", _mha_variant(slot_rows=True)),
    "current_token_not_attended": ("sparse_mha", _mha_variant(no_append=True)),
    "new_kv_not_rounded_to_cache_type": ("sparse_mha", _mha_variant(no_round=True)),
}


def pytest_configure(config):
    name = os.environ.get("DJV_ORACLE_MUTANT", "")
    if not name:
        return
    attr, fn = MUTANTS[name]
    setattr(D, attr, fn)
    if hasattr(oracle, attr):
        setattr(oracle, attr, fn)
