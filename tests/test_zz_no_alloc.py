"""The allocation-free sparse MLP (dejavu_sparse_mlp_no_alloc, static device scratch)
against dejavu_sparse_mlp with a workspace, through the C ABI: bit-identical outputs on
two calls in a row, the second smaller than the first, so the second runs on scratch the
first left behind.  Both are also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host

pytestmark = pytest.mark.gpu

# (weight dtype, B, d, N, kept neurons per call): an OPT-175B-shaped MLP at batch 2 with a
# 5%-per-token union, then an OPT-125m-shaped fp32 MLP at batch 1
CALLS = [("f16", 2, 12288, 49152, 4916), ("f32", 1, 768, 3072, 154)]


def _inputs(dtype, B, d, N, k, seed):
    dt = torch.float16 if dtype == "f16" else torch.float32
    W1 = synth.normal((N, d), synth.W_STD, dt, DEV, synth.seed_of(seed, 0, "W1"))
    W2 = synth.normal((N, d), synth.W_STD, dt, DEV, synth.seed_of(seed, 0, "W2"))
    b1 = torch.full((N,), synth.B1_VALUE, dtype=dt, device=DEV)
    x = synth.normal((B, d), 1.0, torch.float32, DEV, synth.seed_of(seed, 0, "x"))
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    S = np.sort(np.random.default_rng(seed).choice(N, size=k, replace=False)).astype(np.int32)
    idx = torch.from_numpy(S).to(DEV)
    cnt = torch.tensor([k], dtype=torch.int32, device=DEV)
    return W1, b1, W2, x, y, S, idx, cnt


def test_no_alloc_matches_workspace_call_twice():
    for i, (dtype, B, d, N, k) in enumerate(CALLS):
        print(f"no-alloc call {i}: {dtype} B={B} d={d} N={N} k={k}", flush=True)
        wt = dj.DJV_F16 if dtype == "f16" else dj.DJV_F32
        W1, b1, W2, x, y, S, idx, cnt = _inputs(dtype, B, d, N, k, seed=11 + i)
        ws = dj.workspace(dj.dejavu_workspace_bytes(B, d, N, 0, 0, 0, 0), DEV)
        ref_out = torch.empty(B, d, device=DEV)
        dj.dejavu_sparse_mlp(wt, B, d, N, y, W1, b1, W2, idx, cnt, k, x, ref_out, ws)
        out = torch.full((B, d), float("nan"), device=DEV)
        dj.dejavu_sparse_mlp_no_alloc(wt, B, d, N, y, W1, b1, W2, idx, cnt, k, x, out)
        torch.cuda.synchronize()
        assert dj.dejavu_poll_device_error() == 0
        assert torch.equal(out, ref_out), (i, (out - ref_out).abs().max().item())
        ref = O.sparse_mlp(host(y), host(W1), host(b1), host(W2), S)
        assert_close(host(out) - host(x), ref, TOL[dtype], i)


def test_no_alloc_repeated_on_one_stream():
    # several calls queued back to back on one stream share the scratch in order
    dtype, B, d, N, k = CALLS[1]
    W1, b1, W2, x, y, S, idx, cnt = _inputs(dtype, B, d, N, k, seed=5)
    outs = [torch.empty(B, d, device=DEV) for _ in range(3)]
    for o in outs:
        dj.dejavu_sparse_mlp_no_alloc(dj.DJV_F32, B, d, N, y, W1, b1, W2, idx, cnt, k, None, o)
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs[1:])
    assert_close(host(outs[0]), O.sparse_mlp(host(y), host(W1), host(b1), host(W2), S), TOL[dtype])
