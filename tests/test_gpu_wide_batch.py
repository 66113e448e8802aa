"""The matrix-core GEMV and row-axpy against the oracle: batches of 5 to 32 tokens, and
batches of 1 to 4 with the form forced by dejavu_set_mfma_min_batch.  Predictor scores
and sets, sparse MLP, sparse attention with the KV append, a serial layer and a
lookahead stack.  fp16 weights; row lengths are multiples of 32 and include
a 64-column tile cut in half (d = 1056), ragged 16-row tiles (N = 1500, k = 37) and
k-slices shorter than one unrolled step (r = 160).

The tolerance is the fp16 one of the vector-ALU path: the matrix-core path rounds the
normalised activations to fp16 (as the vector-ALU fp16 path does) and in addition the
row-axpy coefficients, a relative error of at most 2^-11 per product, far below 1e-2."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host, idx_tensor, oracle_layer, rel_l2, ws_for, wt_code
from test_gpu_layer import Stack, check_stack

pytestmark = pytest.mark.gpu

SHAPES = {
    "w-ragged": synth.LayerShape(d=1056, N=1500, h=6, dh=128, n=300, r=160, dtype="f16"),
    "w-dh64": synth.LayerShape(d=1024, N=3000, h=8, dh=64, n=200, r=128, dtype="f16"),
    "w-wide": synth.LayerShape(d=4096, N=4000, h=8, dh=128, n=1024, r=1024, dtype="f16"),
}
BATCHES = [5, 8, 16, 32]


def _setup(name, B, seed=3):
    s = SHAPES[name].with_(B=B)
    return s, synth.make_layer(s, seed, 0, DEV), synth.make_predictors(s, seed, 0, DEV), \
        synth.make_input(s, seed, DEV)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", BATCHES)
def test_predict_wide(name, B):
    print(f"predict {name} B={B}", flush=True)
    s, w, p, x = _setup(name, B)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    ws = ws_for(s)
    for P1, P2, n_out, k in ((p["P1_M"], p["P2_M"], s.N, (5 * s.N + 99) // 100),
                             (p["P1_A"], p["P2_A"], s.h, (20 * s.h + 99) // 100)):
        idx = torch.empty(n_out, dtype=torch.int32, device=DEV)
        cnt = torch.empty(1, dtype=torch.int32, device=DEV)
        z = torch.empty(B, n_out, dtype=torch.float32, device=DEV)
        dj.dejavu_predict(wt_code(s), B, s.d, s.r, n_out, y, P1, P2, dj.DJV_TOPK, k, 0.5, idx, cnt, z, ws)
        torch.cuda.synchronize()
        z_ref = O.predictor_logits_f64(host(y), host(P1), host(P2))
        assert_close(host(z), z_ref, TOL[s.dtype], rel_l2(host(z), z_ref))
        # every batch row on its own, not only the whole
        for b in range(B):
            assert_close(host(z)[b], z_ref[b], TOL[s.dtype], b)
        got = host(idx)[: int(cnt.item())]
        assert np.array_equal(got, O.select(host(z), O.TOPK, k=k))


def _random_set(n, k, seed):
    g = np.random.default_rng(seed)
    return np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", BATCHES)
def test_sparse_mlp_wide(name, B):
    print(f"sparse_mlp {name} B={B}", flush=True)
    s, w, p, x = _setup(name, B)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    ws = ws_for(s)
    Wn = oracle_layer(w)
    for k in (1, 37, (5 * s.N + 99) // 100, s.N):
        S = _random_set(s.N, k, k)
        idx, cnt, cap = idx_tensor(S)
        out = x.clone()
        dj.dejavu_sparse_mlp(wt_code(s), B, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap,
                             out, out, ws)
        torch.cuda.synchronize()
        ref = O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S)
        got = host(out) - host(x)
        assert_close(got, ref, TOL[s.dtype], (k, rel_l2(got, ref)))
        for b in range(B):
            assert_close(got[b], ref[b], TOL[s.dtype], (k, b))


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", [5, 16, 32])
def test_sparse_mha_wide(name, B):
    print(f"sparse_mha {name} B={B}", flush=True)
    s, w, p, x = _setup(name, B)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    scale = s.dh ** -0.5
    for S in ([0], [1, s.h - 1], list(range(s.h))):
        S = np.array(S, dtype=np.int32)
        K0, V0 = host(w["K"]).copy(), host(w["V"]).copy()
        idx, cnt, cap = idx_tensor(S)
        out = torch.empty(B, s.d, device=DEV)
        dj.dejavu_sparse_mha(wt_code(s), B, s.d, s.h, s.dh, s.n, s.cap, y, w["Wqkv"], w["Wo"], w["K"],
                             w["V"], idx, cnt, cap, scale, None, out, ws_for(s))
        torch.cuda.synchronize()
        ref, kn, vn = O.sparse_mha(host(y), host(w["Wqkv"]), host(w["Wo"]), K0, V0, s.n, S, scale)
        assert_close(host(out), ref, TOL[s.dtype], (S, rel_l2(host(out), ref)))
        K1, V1 = host(w["K"]), host(w["V"])
        for slot, i in enumerate(S):
            assert_close(K1[:, i, s.n], kn[:, slot], TOL[s.dtype])
            assert_close(V1[:, i, s.n], vn[:, slot], TOL[s.dtype])
        mask = np.ones(s.h, dtype=bool)
        mask[S] = False
        assert np.array_equal(K1[:, mask], K0[:, mask]) and np.array_equal(V1[:, mask], V0[:, mask])
        assert np.array_equal(K1[:, :, : s.n], K0[:, :, : s.n])


@pytest.mark.parametrize("B", [8, 32])
def test_serial_layer_wide(B):
    print(f"serial layer B={B}", flush=True)
    st = Stack(SHAPES["w-ragged"].with_(B=B), 1, 31, k_A=2, k_M=75)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)


@pytest.mark.parametrize("B", [5, 16])
def test_stack_wide(B):
    print(f"lookahead stack B={B}", flush=True)
    st = Stack(SHAPES["w-ragged"].with_(B=B), 3, 32, k_A=2, k_M=75)
    x, tr = st.run(lookahead=True)
    check_stack(st, host(x), tr, lookahead=True)
    # the union of per-token sets
    assert (tr["counts"][:, 1] >= st.k_M).all()
    x2, _ = st.run(lookahead=True)
    assert np.array_equal(host(x), host(x2))


def test_threshold_layer_wide():
    s = SHAPES["w-ragged"].with_(B=8)
    st = Stack(s, 1, 33, k_A=0, k_M=0, mode=dj.DJV_THRESHOLD, t_A=0.6, t_M=0.7)
    x, tr = st.run(lookahead=False, single_layer=True)
    assert 0 < tr["counts"][0, 1] < s.N
    check_stack(st, host(x), tr, lookahead=False)


# ---------------------------------------------------- matrix-core form at small batches
@pytest.fixture
def mfma_from_1():
    old = dj.dejavu_set_mfma_min_batch(1)
    yield
    dj.dejavu_set_mfma_min_batch(old)


@pytest.mark.parametrize("B", [1, 2, 4])
def test_small_batch_matrix_core_blocks(B, mfma_from_1):
    print(f"matrix-core blocks B={B}", flush=True)
    test_predict_wide("w-ragged", B)
    test_sparse_mlp_wide("w-ragged", B)
    test_sparse_mha_wide("w-dh64", B)
    # the form did switch: the matrix-core row-axpy rounds its coefficients to fp16, so
    # its bits differ from the vector-ALU result (both within the tolerance above)
    s, w, p, x = _setup("w-ragged", B)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    idx, cnt, cap = idx_tensor(_random_set(s.N, 75, 75))
    outs = []
    for b_min in (1, dj.DJV_MAX_VALU_BATCH + 1):
        dj.dejavu_set_mfma_min_batch(b_min)
        out = torch.empty(B, s.d, device=DEV)
        dj.dejavu_sparse_mlp(wt_code(s), B, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap,
                             None, out, ws_for(s))
        outs.append(host(out))
    torch.cuda.synchronize()
    dj.dejavu_set_mfma_min_batch(1)
    assert not np.array_equal(outs[0], outs[1])
    assert_close(outs[0], outs[1], TOL[s.dtype])


@pytest.mark.parametrize("B", [1, 3])
def test_small_batch_matrix_core_stack(B, mfma_from_1):
    print(f"matrix-core lookahead stack B={B}", flush=True)
    test_stack_wide(B)
