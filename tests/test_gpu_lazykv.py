"""Lazy K/V over several decode steps against the oracle.

Each step decodes one new token (a fresh seeded input) at the next position n through a
stack of layers.  With lazy K/V a step writes K/V only for its selected heads, saves its
attention input y, and before a head attends recomputes the K/V it skipped.  Checked per
step and layer (teacher-forced on the GPU's own layer inputs and sets): the attention
output equals the oracle's over the cache that computing every head's K/V at every step
gives, and at the end every cache entry the per-head valid lengths cover equals it.  A
control run without lazy K/V shows the stale entries a selected head would read."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV, TOL, assert_close, host, rel_l2, wt_code

pytestmark = pytest.mark.gpu


def _run_steps(s, L, T, seed, lazy, lookahead, B=1, mode=dj.DJV_TOPK, k_A=2, k_M=75):
    n0 = s.n
    shape = s.with_(B=B, n_cap=n0 + T + 1)
    w = [synth.make_layer(shape, seed, l, DEV) for l in range(L)]
    p = [synth.make_predictors(shape, seed, l, DEV) for l in range(L)]
    K0 = [host(wl["K"]).copy() for wl in w]
    V0 = [host(wl["V"]).copy() for wl in w]
    if lazy:
        for wl in w:
            wl["Y"] = torch.zeros(B, shape.cap, shape.d, device=DEV)
            wl["kv_len"] = torch.full((2, shape.h), n0, dtype=torch.int32, device=DEV)
    desc = [dj.make_layer(w[l], p[l]) for l in range(L)]
    steps = []
    for t in range(T):
        m = dj.make_model(wt_code(shape), B, shape.d, shape.N, shape.h, shape.dh, shape.r, n0 + t,
                          shape.cap, shape.dh ** -0.5, mode, k_A, k_M, 0.6, 0.7)
        ws = dj.workspace(dj.dejavu_workspace_bytes_model(m), DEV)
        f = lambda *sh: torch.zeros(*sh, dtype=torch.float32, device=DEV)
        i = lambda *sh: torch.full(sh, -1, dtype=torch.int32, device=DEV)
        tr = dict(x_in=f(L, B, shape.d), x_mid=f(L, B, shape.d), sets_A=i(L, shape.h),
                  sets_M=i(L, shape.N), counts=i(L, 2))
        x = synth.make_input(shape, seed + 100 + t, DEV)
        dj.dejavu_stack_decode(m, desc, x, lookahead, False, dj.make_trace(**tr), ws,
                               torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert dj.dejavu_poll_device_error() == 0
        steps.append({k: host(v) for k, v in tr.items()} | {"x_out": host(x)})
    return shape, w, K0, V0, steps


def _check(shape, w, K0, V0, steps, L):
    s, n0, tol = shape, shape.n, TOL[shape.dtype]
    ys = [[O.layernorm(st["x_in"][l]) for st in steps] for l in range(L)]
    for t, st in enumerate(steps):
        n = n0 + t
        for l in range(L):
            cA = int(st["counts"][l, 0])
            S_A = st["sets_A"][l, :cA].astype(np.int64)
            # the cache every head would hold had all heads computed K/V at every step
            K, V = O.cache_after_steps(host(w[l]["Wqkv"]), K0[l], V0[l], n0, ys[l][:t])
            Wqkv = host(w[l]["Wqkv"])[S_A]
            Wo = host(w[l]["Wo"]).reshape(s.h, s.dh, s.d)[S_A].reshape(-1, s.d)
            att, _, _ = O.sparse_mha(ys[l][t], Wqkv, Wo, K[:, S_A], V[:, S_A], n, np.arange(cA),
                                     s.dh ** -0.5)
            x_in, x_mid = st["x_in"][l].astype(np.float64), st["x_mid"][l].astype(np.float64)
            err = rel_l2(x_mid - x_in, att)
            assert err < tol, (t, l, err)
    # every entry covered by the final valid lengths equals the all-heads cache
    for l in range(L):
        K, V = O.cache_after_steps(host(w[l]["Wqkv"]), K0[l], V0[l], n0, ys[l])
        n_end = n0 + len(steps)
        kv_len = host(w[l]["kv_len"])[n_end & 1]
        Kg, Vg = host(w[l]["K"]), host(w[l]["V"])
        for i in range(s.h):
            hi = int(kv_len[i])
            assert n0 <= hi <= n_end
            if hi > n0:
                assert_close(Kg[:, i, n0:hi], K[:, i, n0:hi], tol, (l, i))
                assert_close(Vg[:, i, n0:hi], V[:, i, n0:hi], tol, (l, i))


SMALL = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")


@pytest.mark.parametrize("lookahead", [True, False])
def test_lazy_kv_steps_match_all_heads_cache(lookahead):
    print(f"lazy K/V 6 steps, 2 layers, lookahead={lookahead}", flush=True)
    L, T = 2, 6
    shape, w, K0, V0, steps = _run_steps(SMALL, L, T, 51, lazy=True, lookahead=lookahead)
    _check(shape, w, K0, V0, steps, L)
    # heads did skip steps and were selected again (the case lazy K/V exists for)
    sets = [[set(st["sets_A"][l, : int(st["counts"][l, 0])].tolist()) for st in steps]
            for l in range(L)]
    assert any(i in sets[l][t] and i not in sets[l][t - 1] for l in range(L) for t in range(1, T)
               for i in range(SMALL.h))


@pytest.mark.parametrize("B,mode", [(3, dj.DJV_TOPK), (1, dj.DJV_THRESHOLD), (6, dj.DJV_TOPK)])
def test_lazy_kv_batches_and_threshold(B, mode):
    print(f"lazy K/V B={B} mode={mode}", flush=True)
    s = SMALL.with_(d=1056, r=160)
    L, T = 2, 4
    shape, w, K0, V0, steps = _run_steps(s, L, T, 52, lazy=True, lookahead=True, B=B, mode=mode)
    _check(shape, w, K0, V0, steps, L)


# the recompute stages weight rows through LDS in chunks of 256 16-byte vectors: fp32 rows
# of 1200 (300 vectors: a full chunk and a ragged one, d_h 64) and fp16 rows of 4104 (513
# vectors: two full chunks and one vector)
@pytest.mark.parametrize("shape", [
    synth.LayerShape(d=1200, N=1200, h=8, dh=64, n=200, r=128, dtype="f32"),
    synth.LayerShape(d=4104, N=2000, h=6, dh=128, n=150, r=128, dtype="f16"),
], ids=["f32-d1200-dh64", "f16-d4104"])
def test_lazy_kv_weight_chunks(shape):
    print(f"lazy K/V {shape.dtype} d={shape.d} dh={shape.dh}", flush=True)
    L, T = 2, 6
    shape, w, K0, V0, steps = _run_steps(shape, L, T, 53, lazy=True, lookahead=True)
    _check(shape, w, K0, V0, steps, L)
    sets = [[set(st["sets_A"][l, : int(st["counts"][l, 0])].tolist()) for st in steps]
            for l in range(L)]
    assert any(i in sets[l][t] and i not in sets[l][t - 1] for l in range(L) for t in range(1, T)
               for i in range(shape.h))


def test_lazy_kv_saved_input_full_width():
    # rows as wide as the OPT-175B shape's: in the lookahead stack the save sums LN's moments of
    # x itself (48 values of the row per thread); every saved input equals LN of its layer input
    print("lazy K/V saved inputs at d=12288", flush=True)
    s = synth.LayerShape(d=12288, N=2048, h=4, dh=128, n=64, r=128, dtype="f16")
    L, T = 2, 3
    shape, w, K0, V0, steps = _run_steps(s, L, T, 54, lazy=True, lookahead=True, k_A=2, k_M=100)
    _check(shape, w, K0, V0, steps, L)
    for l in range(L):
        Y = host(w[l]["Y"])
        for t, st in enumerate(steps):
            assert_close(Y[:, shape.n + t], O.layernorm(st["x_in"][l]), TOL["f32"], (l, t))


def test_without_lazy_kv_a_reselected_head_reads_stale_entries():
    # the same steps without lazy K/V: a head that skipped a step attends over the cache's
    # old contents at that position, which differ from the all-heads cache
    L, T = 2, 6
    shape, w, K0, V0, steps = _run_steps(SMALL, L, T, 51, lazy=False, lookahead=True)
    s, n0 = shape, shape.n
    ys = [[O.layernorm(st["x_in"][l]) for st in steps] for l in range(L)]
    worst = 0.0
    for t, st in enumerate(steps):
        for l in range(L):
            cA = int(st["counts"][l, 0])
            S_A = st["sets_A"][l, :cA].astype(np.int64)
            K, V = O.cache_after_steps(host(w[l]["Wqkv"]), K0[l], V0[l], n0, ys[l][:t])
            Wqkv = host(w[l]["Wqkv"])[S_A]
            Wo = host(w[l]["Wo"]).reshape(s.h, s.dh, s.d)[S_A].reshape(-1, s.d)
            att, _, _ = O.sparse_mha(ys[l][t], Wqkv, Wo, K[:, S_A], V[:, S_A], n0 + t, np.arange(cA),
                                     s.dh ** -0.5)
            worst = max(worst, rel_l2(st["x_mid"][l].astype(np.float64) - st["x_in"][l], att))
    assert worst > 10 * TOL[s.dtype], worst
