"""The fusion ablation's unfused path ([BLOG section 3.2 "Kernel Fusion"]): the kept rows
gathered into contiguous buffers (dejavu_gather_rows), then the dense MLP over them.  The
gather is checked exactly against indexing; the unfused MLP must equal the fused sparse MLP
bit for bit (same rows in the same order, same reductions) and the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host, idx_tensor, oracle_layer, rel_l2, ws_for, wt_code

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("rpu,cols", [(1, 1032), (1, 1), (3, 130), (128, 768)])
def test_gather_rows_exact(dtype, rpu, cols):
    print(f"gather {dtype} rpu={rpu} cols={cols}", flush=True)
    tdt = torch.float16 if dtype == "f16" else torch.float32
    units = 50
    W = synth.normal((units * rpu, cols), 1.0, tdt, DEV, 77)
    S = np.array([0, 3, 7, 8, 49], dtype=np.int32)
    idx, cnt, _ = idx_tensor(S)
    cap = 7  # two zero rows past the count
    idx_full = torch.zeros(cap, dtype=torch.int32, device=DEV)
    idx_full[: len(S)] = idx
    out = torch.full((cap * rpu, cols), 7.0, dtype=tdt, device=DEV)
    dj.dejavu_gather_rows(dj.DJV_F16 if dtype == "f16" else dj.DJV_F32, rpu, cols, units, W, idx_full, cnt,
                          cap, out)
    torch.cuda.synchronize()
    rows = (torch.as_tensor(S, device=DEV).long()[:, None] * rpu + torch.arange(rpu, device=DEV)[None]).reshape(-1)
    assert torch.equal(out[: len(S) * rpu], W[rows])
    assert torch.count_nonzero(out[len(S) * rpu:]).item() == 0
    assert dj.dejavu_poll_device_error() == 0


@pytest.mark.parametrize("name,B", [("f16-ragged", 1), ("f16-wide", 2), ("f32-ragged", 3)])
def test_unfused_mlp_equals_fused(name, B):
    print(f"unfused mlp {name} B={B}", flush=True)
    shapes = {
        "f16-ragged": synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16"),
        "f16-wide": synth.LayerShape(d=4096, N=4000, h=8, dh=128, n=1024, r=1024, dtype="f16"),
        "f32-ragged": synth.LayerShape(d=1032, N=1500, h=6, dh=64, n=300, r=136, dtype="f32"),
    }
    s = shapes[name].with_(B=B)
    w = synth.make_layer(s, 5, 0, DEV)
    x = synth.make_input(s, 5, DEV)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    k = (5 * s.N + 99) // 100
    S = np.sort(np.random.default_rng(3).choice(s.N, size=k, replace=False)).astype(np.int32)
    idx, cnt, cap = idx_tensor(S)
    wt = wt_code(s)
    ws = ws_for(s)
    fused = torch.empty(B, s.d, device=DEV)
    dj.dejavu_sparse_mlp(wt, B, s.d, s.N, y, w["W1"], w["b1"], w["W2"], idx, cnt, cap, x, fused, ws)
    W1g = torch.empty(cap, s.d, dtype=w["W1"].dtype, device=DEV)
    W2g = torch.empty_like(W1g)
    b1g = torch.empty(cap, dtype=w["b1"].dtype, device=DEV)
    dj.dejavu_gather_rows(wt, 1, s.d, s.N, w["W1"], idx, cnt, cap, W1g)
    dj.dejavu_gather_rows(wt, 1, s.d, s.N, w["W2"], idx, cnt, cap, W2g)
    dj.dejavu_gather_rows(wt, 1, 1, s.N, w["b1"], idx, cnt, cap, b1g)
    unfused = torch.empty(B, s.d, device=DEV)
    dj.dejavu_dense_mlp(wt, B, s.d, cap, y, W1g, b1g, W2g, x, unfused, ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, unfused)
    Wn = oracle_layer(w)
    ref = O.sparse_mlp(host(y), Wn.W1, Wn.b1, Wn.W2, S)
    assert_close(host(unfused) - host(x), ref, TOL[s.dtype])
