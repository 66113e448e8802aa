"""GPU blocks against the oracle: LayerNorm, predictor, sparse and dense MLP, sparse and
dense attention (with the KV append), on shapes that span several tiles and ragged
tails, fp32 and fp16 weights, batch 1 to 4."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host, idx_tensor, oracle_layer, rel_l2, ws_for, wt_code

pytestmark = pytest.mark.gpu

SHAPES = {
    # several GEMV row groups, axpy column tiles with a ragged last tile, 3 attention chunks
    "f32-ragged": synth.LayerShape(d=1032, N=1500, h=6, dh=64, n=300, r=136, dtype="f32"),
    "f16-ragged": synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16"),
    "opt125m": synth.LayerShape(d=768, N=3072, h=12, dh=64, n=128, r=128, dtype="f32"),
    "f16-wide": synth.LayerShape(d=4096, N=4000, h=8, dh=128, n=1024, r=1024, dtype="f16"),
    # rows of 128+ 64-column slices: the one-kernel column-slice row-axpy, with a ragged
    # last slice, and (N rows) more rows than one staging batch
    "f32-slice": synth.LayerShape(d=8184, N=5000, h=4, dh=64, n=200, r=256, dtype="f32"),
    "f16-slice": synth.LayerShape(d=8200, N=6000, h=4, dh=128, n=100, r=512, dtype="f16"),
}


def _setup(name, B=1, seed=1):
    s = SHAPES[name].with_(B=B)
    w = synth.make_layer(s, seed, 0, DEV)
    p = synth.make_predictors(s, seed, 0, DEV)
    x = synth.make_input(s, seed, DEV)
    return s, w, p, x


@pytest.mark.parametrize("B", [1, 3])
def test_layernorm(B):
    for d in (768, 1032, 12288):
        x = synth.normal((B, d), 2.0, torch.float32, DEV, d) + 0.5
        y = torch.empty_like(x)
        dj.dejavu_layernorm(B, d, x, y, 1e-5)
        torch.cuda.synchronize()
        assert_close(host(y), O.layernorm(host(x)), 1e-6)
    # in place, and a constant row
    x = torch.full((1, 1024), 3.0, device=DEV)
    dj.dejavu_layernorm(1, 1024, x, x, 1e-5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(x).item() == 0


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", [1, 2, 4])
def test_predict(name, B):
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
        assert_close(host(z), z_ref, TOL[s.dtype])
        got = host(idx)[: int(cnt.item())]
        # bit-exact on identical scores
        assert np.array_equal(got, O.select(host(z), O.TOPK, k=k))
        # without exported logits the same sets come out
        idx2 = torch.empty_like(idx)
        cnt2 = torch.empty_like(cnt)
        dj.dejavu_predict(wt_code(s), B, s.d, s.r, n_out, y, P1, P2, dj.DJV_TOPK, k, 0.5, idx2, cnt2, None, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(idx2)[: int(cnt2.item())], got)


def _random_set(n, k, seed):
    g = np.random.default_rng(seed)
    return np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_sparse_mlp(name, B):
    print(f"sparse_mlp {name} B={B}", flush=True)
    s, w, p, x = _setup(name, B)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    ws = ws_for(s)
    Wn = oracle_layer(w)
    for k in (1, 37, (5 * s.N + 99) // 100, s.N):
        S = _random_set(s.N, k, k)
        idx, cnt, cap = idx_tensor(S)
        out = torch.empty(B, s.d, device=DEV)
        dj.dejavu_sparse_mlp(wt_code(s), B, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap,
                             None, out, ws)
        torch.cuda.synchronize()
        ref = O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S)
        assert_close(host(out), ref, TOL[s.dtype], (k, rel_l2(host(out), ref)))
        # with the residual, in place
        out2 = x.clone()
        dj.dejavu_sparse_mlp(wt_code(s), B, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap,
                             out2, out2, ws)
        torch.cuda.synchronize()
        assert_close(host(out2) - host(x), ref, TOL[s.dtype])


@pytest.mark.parametrize("name", list(SHAPES))
def test_dense_mlp(name):
    s, w, p, x = _setup(name, 2)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    out = torch.empty(2, s.d, device=DEV)
    dj.dejavu_dense_mlp(wt_code(s), 2, s.d, s.N, y, w["W1"], w["b1"], w["W2"], x, out, ws_for(s))
    torch.cuda.synchronize()
    Wn = oracle_layer(w)
    ref = O.dense_mlp(host(y), Wn.W1, Wn.b1, Wn.W2)
    assert_close(host(out) - host(x), ref, TOL[s.dtype])


def test_sparse_mlp_count_below_capacity_and_bad_index():
    s, w, p, x = _setup("f16-ragged", 1)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    ws = ws_for(s)
    Wn = oracle_layer(w)
    S = _random_set(s.N, 40, 2)
    idx = torch.full((100,), 0, dtype=torch.int32, device=DEV)
    idx[:40] = torch.from_numpy(S).to(DEV)
    cnt = torch.tensor([40], dtype=torch.int32, device=DEV)
    out = torch.empty(1, s.d, device=DEV)
    dj.dejavu_poll_device_error()
    dj.dejavu_sparse_mlp(wt_code(s), 1, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, 100, None, out, ws)
    assert dj.dejavu_poll_device_error() == 0
    assert_close(host(out), O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S), 1e-2)
    # an index past N contributes nothing and raises the device flag
    idx[5] = s.N + 11
    dj.dejavu_sparse_mlp(wt_code(s), 1, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, 100, None, out, ws)
    assert dj.dejavu_poll_device_error() & dj.DJV_FLAG_BAD_INDEX
    S2 = np.delete(S, 5)
    assert_close(host(out), O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S2), 1e-2)
    # a count above the capacity is clamped and flagged
    idx[5] = int(S[5])
    cnt.fill_(1000)
    dj.dejavu_sparse_mlp(wt_code(s), 1, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx[:40].clone(), cnt, 40,
                         None, out, ws)
    assert dj.dejavu_poll_device_error() & dj.DJV_FLAG_BAD_COUNT
    assert_close(host(out), O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S), 1e-2)
    # count 0: out = resid
    cnt.fill_(0)
    dj.dejavu_sparse_mlp(wt_code(s), 1, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, 100, x, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, x)


def _mha_case(s, w, x, S, scale, n=None):
    n = s.n if n is None else n
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    K0, V0 = host(w["K"]).copy(), host(w["V"]).copy()
    idx, cnt, cap = idx_tensor(S)
    out = torch.empty(s.B, s.d, device=DEV)
    dj.dejavu_sparse_mha(wt_code(s), s.B, s.d, s.h, s.dh, n, s.cap, y, w["Wqkv"], w["Wo"], w["K"], w["V"],
                         idx, cnt, cap, scale, None, out, ws_for(s))
    torch.cuda.synchronize()
    ref, kn, vn = O.sparse_mha(host(y), host(w["Wqkv"]), host(w["Wo"]), K0, V0, n, S, scale)
    return out, ref, kn, vn, K0, V0


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("B", [1, 2, 4])
def test_sparse_mha(name, B):
    print(f"sparse_mha {name} B={B}", flush=True)
    s, w, p, x = _setup(name, B)
    for S in ([0], [1, s.h - 1], list(range(0, s.h, 2)), list(range(s.h))):
        S = np.array(S, dtype=np.int32)
        out, ref, kn, vn, K0, V0 = _mha_case(s, w, x, S, s.dh ** -0.5)
        assert_close(host(out), ref, TOL[s.dtype], (S, rel_l2(host(out), ref)))
        K1, V1 = host(w["K"]), host(w["V"])
        for slot, i in enumerate(S):
            assert_close(K1[:, i, s.n], kn[:, slot], TOL[s.dtype])
            assert_close(V1[:, i, s.n], vn[:, slot], TOL[s.dtype])
        # other heads' position n and every other position are untouched
        mask = np.ones(s.h, dtype=bool)
        mask[S] = False
        assert np.array_equal(K1[:, mask], K0[:, mask]) and np.array_equal(V1[:, mask], V0[:, mask])
        assert np.array_equal(K1[:, :, : s.n], K0[:, :, : s.n])


@pytest.mark.parametrize("name", ["f32-ragged", "f16-ragged"])
def test_sparse_mha_edge_lengths(name):
    s, w, p, x = _setup(name, 1)
    S = np.array([2, 3], dtype=np.int32)
    for n in (0, 1, 127, 128, 129, 255, 256):
        out, ref, *_ = _mha_case(s, w, x, S, 1.0 / 8, n=n)
        assert_close(host(out), ref, TOL[s.dtype], n)
    # the literal formula (scale 1)
    out, ref, *_ = _mha_case(s, w, x, S, 1.0)
    assert_close(host(out), ref, TOL[s.dtype])


@pytest.mark.parametrize("name", list(SHAPES))
def test_dense_mha(name):
    s, w, p, x = _setup(name, 2)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    K0, V0 = host(w["K"]).copy(), host(w["V"]).copy()
    out = torch.empty(2, s.d, device=DEV)
    dj.dejavu_dense_mha(wt_code(s), 2, s.d, s.h, s.dh, s.n, s.cap, y, w["Wqkv"], w["Wo"], w["K"], w["V"],
                        s.dh ** -0.5, x, out, ws_for(s))
    torch.cuda.synchronize()
    ref, kn, vn = O.dense_mha(host(y), host(w["Wqkv"]), host(w["Wo"]), K0, V0, s.n, s.dh ** -0.5)
    assert_close(host(out) - host(x), ref, TOL[s.dtype])
    assert_close(host(w["K"])[:, :, s.n], kn, TOL[s.dtype])


def test_blocks_deterministic():
    s, w, p, x = _setup("f16-wide", 2)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    ws = ws_for(s)
    S = _random_set(s.N, 200, 9)
    idx, cnt, cap = idx_tensor(S)
    outs = []
    for _ in range(2):
        out = torch.empty(2, s.d, device=DEV)
        dj.dejavu_sparse_mlp(wt_code(s), 2, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap, x, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
