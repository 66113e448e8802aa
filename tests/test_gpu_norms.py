"""The "true" selection's scores on the GPU against the oracle: per-neuron activation norms
across the batch rows, per-head attention output norms (with the K/V append of every
head), the true sets selected from them, and the recall of predicted sets."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host, rel_l2, ws_for, wt_code

pytestmark = pytest.mark.gpu

SHAPES = {
    "f32-ragged": synth.LayerShape(d=1032, N=1500, h=6, dh=64, n=300, r=136, dtype="f32"),
    "f16-ragged": synth.LayerShape(d=1056, N=1500, h=6, dh=128, n=300, r=160, dtype="f16"),
    "f16-wide": synth.LayerShape(d=4096, N=4000, h=8, dh=128, n=1024, r=1024, dtype="f16"),
}


def _setup(name, B, seed=5):
    s = SHAPES[name].with_(B=B)
    w = synth.make_layer(s, seed, 0, DEV)
    x = synth.make_input(s, seed, DEV)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    return s, w, y


def _true_set(scores, k, n):
    idx = torch.empty(n, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = dj.workspace(4 * ((n + 31) // 32) + 256, DEV)
    dj.dejavu_select(1, n, scores.view(1, n), dj.DJV_TOPK, k, 0.5, idx, cnt, ws)
    torch.cuda.synchronize()
    return host(idx)[: int(cnt.item())]


# batches above the vector-ALU limit run on the matrix cores, which need fp16 weights
CASES = [(n, B) for n in SHAPES for B in (1, 3, 5)
         if B <= dj.DJV_MAX_VALU_BATCH or SHAPES[n].dtype == "f16"]


@pytest.mark.parametrize("name,B", CASES)
def test_neuron_norms(name, B):
    print(f"neuron norms {name} B={B}", flush=True)
    s, w, y = _setup(name, B)
    scores = torch.empty(s.N, device=DEV)
    dj.dejavu_neuron_norms(wt_code(s), B, s.d, s.N, y, w["W1"], w["b1"], scores, ws_for(s))
    torch.cuda.synchronize()
    ref = O.neuron_norms(host(y), host(w["W1"]), host(w["b1"]))
    assert_close(host(scores), ref, TOL[s.dtype], rel_l2(host(scores), ref))
    # the true set: bit-exact selection on the GPU's own scores
    k = (5 * s.N + 99) // 100
    assert np.array_equal(_true_set(scores, k, s.N), O.select(host(scores)[None], O.TOPK, k=k))


@pytest.mark.parametrize("name,B", CASES)
def test_head_norms(name, B):
    print(f"head norms {name} B={B}", flush=True)
    s, w, y = _setup(name, B)
    K0, V0 = host(w["K"]).copy(), host(w["V"]).copy()
    scale = s.dh ** -0.5
    scores = torch.empty(s.h, device=DEV)
    dj.dejavu_head_norms(wt_code(s), B, s.d, s.h, s.dh, s.n, s.cap, y, w["Wqkv"], w["K"], w["V"], scale,
                         scores, ws_for(s))
    torch.cuda.synchronize()
    ref = O.head_norms(host(y), host(w["Wqkv"]), K0, V0, s.n, scale)
    assert_close(host(scores), ref, TOL[s.dtype], rel_l2(host(scores), ref))
    # every head's K/V of y is written at position n, nothing else changes
    _, kn, vn = O.dense_mha(host(y), host(w["Wqkv"]), host(w["Wo"]), K0, V0, s.n, scale)
    assert_close(host(w["K"])[:, :, s.n], kn, TOL[s.dtype])
    assert_close(host(w["V"])[:, :, s.n], vn, TOL[s.dtype])
    assert np.array_equal(host(w["K"])[:, :, : s.n], K0[:, :, : s.n])
    k = (20 * s.h + 99) // 100
    assert np.array_equal(_true_set(scores, k, s.h), O.select(host(scores)[None], O.TOPK, k=k))


def test_recall_of_a_predicted_set():
    # recall of the predictor's neuron set against the true set, both from the GPU
    s, w, y = _setup("f16-ragged", 1)
    p = synth.make_predictors(s, 5, 0, DEV)
    k = (5 * s.N + 99) // 100
    scores = torch.empty(s.N, device=DEV)
    ws = ws_for(s)
    dj.dejavu_neuron_norms(wt_code(s), 1, s.d, s.N, y, w["W1"], w["b1"], scores, ws)
    true = _true_set(scores, k, s.N)
    idx = torch.empty(s.N, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    dj.dejavu_predict(wt_code(s), 1, s.d, s.r, s.N, y, p["P1_M"], p["P2_M"], dj.DJV_TOPK, k, 0.5, idx, cnt,
                      None, ws)
    torch.cuda.synchronize()
    pred = host(idx)[: int(cnt.item())]
    r = O.recall(pred, true)
    assert 0.0 <= r <= 1.0 and O.recall(true, true) == 1.0
    # untrained predictor weights: about the chance level k / N, far from 1
    assert r < 0.5
