"""Tensor-parallel shards on one GPU against the oracle.

A shard scores and selects over all heads and neurons, then lists only the kept units
of its own contiguous range, renumbered from the range's start; its weights and caches
are the range's rows.  Checks:
  * dejavu_select_range is bit-exact against the oracle's global selection cut to the
    range (every selection path: short rows, long rows, batch unions; ranges that start
    and end inside a 32-bit word, empty and full ranges);
  * sharded lookahead stacks and serial layers match the oracle layer by layer;
  * the shards' block outputs summed over the shards give the unsharded block output
    (the sum an all-reduce would form between GPUs)."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import configs
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, deterministic, host, rel_l2, ws_for, wt_code
from test_gpu_layer import Stack, check_stack

pytestmark = pytest.mark.gpu


def _ranges(n):
    return [(0, n), (37 % n, min(n, 1000)), (max(0, n - 5), n), (n // 2, n // 2), (0, min(64, n)),
            (min(64, n), min(640, n)), (1, n - 1)]


@pytest.mark.parametrize("n_out", [96, 1500, 49152])
@pytest.mark.parametrize("B", [1, 2, 5])
@pytest.mark.parametrize("mode", [dj.DJV_TOPK, dj.DJV_THRESHOLD])
def test_select_range_bit_exact(n_out, B, mode):
    print(f"select_range n_out={n_out} B={B} mode={mode}", flush=True)
    g = torch.Generator().manual_seed(n_out * 7 + B)
    z = torch.randn(B, n_out, generator=g).to(DEV)
    k = max(1, n_out // 20)
    t = 0.7
    ws = dj.workspace(4 * B * ((n_out + 31) // 32) + 256, DEV)
    want = O.select(host(z), O.TOPK if mode == dj.DJV_TOPK else O.THRESHOLD, k=k, t=t)
    for lo, hi in _ranges(n_out):
        idx = torch.full((max(hi - lo, 1),), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        dj.dejavu_select_range(B, n_out, z, mode, k, t, lo, hi, idx, cnt, ws)
        torch.cuda.synchronize()
        c = int(cnt.item())
        assert np.array_equal(host(idx)[:c], O.shard_set(want, lo, hi)), (lo, hi)


def test_select_range_rejects_bad_ranges():
    z = torch.zeros(1, 100, device=DEV)
    idx = torch.empty(100, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = dj.workspace(4096, DEV)
    for lo, hi in ((-1, 10), (10, 5), (0, 101)):
        with pytest.raises(dj.DejavuError):
            dj.dejavu_select_range(1, 100, z, dj.DJV_TOPK, 5, 0.5, lo, hi, idx, cnt, ws)


SMALL = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")


@pytest.mark.parametrize("g,i", [(2, 0), (2, 1), (4, 3)])
@pytest.mark.parametrize("lookahead", [True, False])
def test_shard_stack_top_k(g, i, lookahead):
    print(f"shard stack g={g} i={i} lookahead={lookahead}", flush=True)
    st = Stack(SMALL, 3, 41, k_A=2, k_M=75, shard=(g, i))
    x, tr = st.run(lookahead=lookahead)
    check_stack(st, host(x), tr, lookahead=lookahead)
    with deterministic():
        xd, trd = st.run(lookahead=lookahead)
        check_stack(st, host(xd), trd, lookahead=lookahead)
        x2, _ = st.run(lookahead=lookahead)
    assert np.array_equal(host(xd), host(x2))


@pytest.mark.parametrize("B,mode", [(3, dj.DJV_TOPK), (1, dj.DJV_THRESHOLD), (8, dj.DJV_TOPK)])
def test_shard_stack_batches_and_threshold(B, mode):
    print(f"shard stack B={B} mode={mode}", flush=True)
    s = SMALL.with_(B=B, d=1056, r=160)
    if mode == dj.DJV_TOPK:
        st = Stack(s, 2, 42, k_A=2, k_M=75, shard=(3, 1))
    else:
        st = Stack(s, 2, 42, k_A=0, k_M=0, mode=mode, t_A=0.6, t_M=0.7, shard=(3, 1))
    x, tr = st.run(lookahead=True)
    check_stack(st, host(x), tr, lookahead=True)


def test_shard_serial_layer_keeps_nothing_of_a_range():
    # a range holding none of the kept heads: the shard's attention part is zero
    st = Stack(SMALL, 1, 43, k_A=1, k_M=75, shard=(6, 0))
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)
    assert tr["counts"][0, 0] in (0, 1)


@pytest.mark.parametrize("B", [1, 5])
def test_shard_blocks_sum_to_unsharded_block(B):
    print(f"shard block sums B={B}", flush=True)
    s = SMALL.with_(B=B, d=1056, r=160)
    w = synth.make_layer(s, 44, 0, DEV)
    x = synth.make_input(s, 44, DEV)
    y = torch.from_numpy(O.layernorm(host(x)).astype(np.float32)).to(DEV)
    gen = torch.Generator().manual_seed(44)
    zA = torch.randn(B, s.h, generator=gen).to(DEV)
    zM = torch.randn(B, s.N, generator=gen).to(DEV)
    ws = ws_for(s)
    kA, kM = 2, 75

    def sets(z, n, k, lo, hi):
        idx = torch.empty(max(hi - lo, 1), dtype=torch.int32, device=DEV)
        cnt = torch.empty(1, dtype=torch.int32, device=DEV)
        dj.dejavu_select_range(B, n, z, dj.DJV_TOPK, k, 0.5, lo, hi, idx, cnt, ws)
        return idx, cnt

    def blocks(wl, h, N, sA, sM, capA, capM):
        att = torch.empty(B, s.d, device=DEV)
        mlp = torch.empty(B, s.d, device=DEV)
        dj.dejavu_sparse_mha(wt_code(s), B, s.d, h, s.dh, s.n, s.cap, y, wl["Wqkv"], wl["Wo"], wl["K"],
                             wl["V"], sA[0], sA[1], capA, s.dh ** -0.5, None, att, ws)
        dj.dejavu_sparse_mlp(wt_code(s), B, s.d, N, y, wl["W1"], wl["b1"], wl["W2"], sM[0], sM[1], capM,
                             None, mlp, ws)
        return att, mlp

    # unsharded reference on copies of the caches (each call appends K/V at position n)
    full = {k: v.clone() for k, v in w.items()}
    capA, capM = min(B * kA, s.h), min(B * kM, s.N)
    att_full, mlp_full = blocks(full, s.h, s.N, sets(zA, s.h, kA, 0, s.h), sets(zM, s.N, kM, 0, s.N),
                                capA, capM)
    for g in (2, 3):
        att_sum = torch.zeros(B, s.d, device=DEV)
        mlp_sum = torch.zeros(B, s.d, device=DEV)
        for i in range(g):
            hr, nr = configs.shard_range(s.h, g, i), configs.shard_range(s.N, g, i)
            wl = synth.shard_layer({k: v.clone() for k, v in w.items()}, hr, nr, s.dh)
            h, N = hr[1] - hr[0], nr[1] - nr[0]
            a, m = blocks(wl, h, N, sets(zA, s.h, kA, *hr), sets(zM, s.N, kM, *nr),
                          min(capA, h), min(capM, N))
            att_sum += a
            mlp_sum += m
        torch.cuda.synchronize()
        assert_close(host(att_sum), host(att_full), TOL[s.dtype], g)
        assert_close(host(mlp_sum), host(mlp_full), TOL[s.dtype], g)


@pytest.mark.slow
def test_opt175b_shard_layer():
    print("opt175b one layer, shard 3 of 8", flush=True)
    wl = configs.WORKLOADS["opt175b-1layer-fp16"]
    st = Stack(wl.shape, 1, 0, k_A=wl.k_A, k_M=wl.k_M, shard=(8, 3))
    assert (st.s.h, st.s.N) == (12, 6144)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)
