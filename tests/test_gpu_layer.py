"""Whole sparse layers and stacks on the GPU against the oracle, teacher-forced layer by
layer: each layer's GPU input x and the GPU's selected sets are fed to the oracle.

Checks per layer:
  * the sets are exactly the oracle's selection on the GPU's own scores (bit-exact on
    identical scores), the GPU scores match the oracle's scores of the same input, and
    the sets are valid top-k sets of the oracle's scores within twice the score gap;
  * x' (after attention) and the layer output match the oracle to the dtype tolerance.
Also the full-size workloads: one OPT-125m layer (fp32), one OPT-175B-shaped layer and a
2-layer OPT-175B-shaped lookahead stack (the benchmark's launch configuration), a 3-layer
OPT-6.7B-shaped lookahead stack, one OPT-66B-shaped layer at batch 1 and 4."""
import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import configs
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import (DEV, TOL, assert_close, check_sets_valid, check_threshold_valid, deterministic, host, rel_l2,
                     wt_code)

pytestmark = pytest.mark.gpu


class Stack:
    """Seeded weights of L layers on the device plus the library descriptors."""

    def __init__(self, shape: synth.LayerShape, L: int, seed: int, k_A: int, k_M: int,
                 mode=dj.DJV_TOPK, t_A=0.5, t_M=0.5, shard=None):
        """shard = (g, i): shard i of g of a tensor-parallel split of `shape`'s heads and
        neurons (full predictors, the shard's slices of the full layer weights)."""
        self.full, self.L = shape, L
        if shard is None:
            self.hr, self.nr, sh = (0, shape.h), (0, shape.N), None
            self.s = shape
            self.w = [synth.make_layer(shape, seed, l, DEV) for l in range(L)]
        else:
            g, i = shard
            self.hr, self.nr = configs.shard_range(shape.h, g, i), configs.shard_range(shape.N, g, i)
            sh = (shape.h, self.hr[0], shape.N, self.nr[0])
            self.s = shape.with_(h=self.hr[1] - self.hr[0], N=self.nr[1] - self.nr[0])
            self.w = [synth.shard_layer(synth.make_layer(shape, seed, l, DEV), self.hr, self.nr, shape.dh)
                      for l in range(L)]
        self.sharded = shard is not None
        self.p = [synth.make_predictors(shape, seed, l, DEV) for l in range(L)]
        self.x0 = synth.make_input(shape, seed, DEV)
        self.k_A, self.k_M, self.mode, self.t_A, self.t_M = k_A, k_M, mode, t_A, t_M
        self.scale = shape.dh ** -0.5
        s = self.s
        self.m = dj.make_model(wt_code(s), s.B, s.d, s.N, s.h, s.dh, s.r, s.n, s.cap, self.scale, mode,
                               k_A, k_M, t_A, t_M, shard=sh)
        self.desc = [dj.make_layer(self.w[l], self.p[l]) for l in range(L)]
        self.ws = dj.workspace(dj.dejavu_workspace_bytes_model(self.m), DEV)
        # host copies of the caches before the step (the step appends at position n)
        self.K0 = [host(w["K"]).copy() for w in self.w]
        self.V0 = [host(w["V"]).copy() for w in self.w]

    def trace(self):
        s, L = self.s, self.L
        f = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device=DEV)
        i = lambda *shape: torch.full(shape, -1, dtype=torch.int32, device=DEV)
        t = dict(x_in=f(L, s.B, s.d), x_mid=f(L, s.B, s.d), z_A=f(L, s.B, self.full.h),
                 z_M=f(L, s.B, self.full.N),
                 sets_A=i(L, s.h), sets_M=i(L, s.N), counts=i(L, 2))
        return t, dj.make_trace(**t)

    def run(self, lookahead: bool, single_layer=False):
        t, tr = self.trace()
        x = self.x0.clone()
        if single_layer:
            dj.dejavu_sparse_layer(self.m, self.desc[0], x, tr, self.ws)
        else:
            dj.dejavu_stack_decode(self.m, self.desc, x, lookahead, False, tr, self.ws,
                                   torch.cuda.current_stream())
        torch.cuda.synchronize()
        # no out-of-range index and no count above its list's capacity on the device
        assert dj.dejavu_poll_device_error() == 0
        return x, {k: host(v) for k, v in t.items()}


def _rows(P, rows):
    """Gather predictor / weight rows on the device before copying to the host."""
    return host(P[torch.as_tensor(np.asarray(rows, dtype=np.int64), device=DEV)])


def check_stack(st: Stack, x_out, tr, lookahead: bool, sel_k=True):
    s, tol = st.s, TOL[st.s.dtype]
    for l in range(st.L):
        x_in, x_mid = tr["x_in"][l].astype(np.float64), tr["x_mid"][l].astype(np.float64)
        cA, cM = int(tr["counts"][l, 0]), int(tr["counts"][l, 1])
        S_A, S_M = tr["sets_A"][l, :cA], tr["sets_M"][l, :cM]
        zA, zM = tr["z_A"][l], tr["z_M"][l]
        # which input each predictor read
        if lookahead:
            src_A = src_M = tr["x_in"][max(l - 1, 0)]
        else:
            src_A, src_M = tr["x_in"][l], tr["x_mid"][l]
        p = st.p[l]
        zA_ref = O.predictor_logits_f64(O.layernorm(src_A), host(p["P1_A"]), host(p["P2_A"]))
        zM_ref = O.predictor_logits_f64(O.layernorm(src_M), host(p["P1_M"]), host(p["P2_M"]))
        assert_close(zA, zA_ref, tol, ("z_A", l))
        assert_close(zM, zM_ref, tol, ("z_M", l))
        # bit-exact selection on the GPU's own scores (a shard lists its part of the set)
        assert np.array_equal(S_A, O.shard_set(O.select(zA, st.mode, st.k_A, st.t_A), *st.hr)), l
        assert np.array_equal(S_M, O.shard_set(O.select(zM, st.mode, st.k_M, st.t_M), *st.nr)), l
        # every token's own set (the union above is made of these) is a valid selection on
        # the oracle's scores, within twice the score gap of that token
        for b in range(s.B):
            for z, z_ref, k, t in ((zA, zA_ref, st.k_A, st.t_A), (zM, zM_ref, st.k_M, st.t_M)):
                S_b = O.select(z[b:b + 1], st.mode, k, t)
                delta = float(np.abs(z[b] - z_ref[b]).max())
                if st.mode == dj.DJV_TOPK:
                    check_sets_valid(S_b, z_ref[b], k, delta)
                else:
                    check_threshold_valid(S_b, z_ref[b], float(O.logit_threshold(t)), delta)
        # attention half from the GPU's input and head set
        w = st.w[l]
        Sa = np.asarray(S_A, dtype=np.int64)
        ta = torch.as_tensor(Sa, device=DEV)
        Wqkv = host(w["Wqkv"][ta])
        Wo = host(w["Wo"].view(s.h, s.dh, s.d)[ta].reshape(-1, s.d))
        K0, V0 = st.K0[l][:, Sa], st.V0[l][:, Sa]
        att, kn, vn = O.sparse_mha(O.layernorm(x_in), Wqkv, Wo, K0, V0, s.n, np.arange(len(Sa)), st.scale)
        assert_close(x_mid - x_in, att, tol, (l, rel_l2(x_mid - x_in, att)))
        # appended K/V rows of the selected heads
        assert_close(host(w["K"][:, ta, s.n]), kn, tol, ("K append", l))
        assert_close(host(w["V"][:, ta, s.n]), vn, tol, ("V append", l))
        # MLP half from the GPU's x' and neuron set
        Sm = np.asarray(S_M, dtype=np.int64)
        tm = torch.as_tensor(Sm, device=DEV)
        mlp = O.sparse_mlp(O.layernorm(x_mid), host(w["W1"][tm]), host(w["b1"][tm]), host(w["W2"][tm]),
                           np.arange(len(Sm)))
        x_next = x_out if l == st.L - 1 else tr["x_in"][l + 1]
        assert_close(np.asarray(x_next, np.float64) - x_mid, mlp, tol, (l, rel_l2(x_next - x_mid, mlp)))


@pytest.mark.parametrize("dtype,B", [("f32", 1), ("f16", 1), ("f16", 3)])
def test_serial_layer_small(dtype, B):
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128 if dtype == "f16" else 64, n=300, r=136,
                         dtype=dtype, B=B)
    st = Stack(s, 1, 21, k_A=2, k_M=75)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)


def test_serial_layer_threshold_mode():
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")
    st = Stack(s, 1, 22, k_A=0, k_M=0, mode=dj.DJV_THRESHOLD, t_A=0.6, t_M=0.7)
    x, tr = st.run(lookahead=False, single_layer=True)
    assert 0 < tr["counts"][0, 1] < s.N
    check_stack(st, host(x), tr, lookahead=False)


@pytest.mark.parametrize("lookahead", [True, False])
def test_stack_small(lookahead):
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")
    st = Stack(s, 4, 23, k_A=2, k_M=75)
    x, tr = st.run(lookahead=lookahead)
    check_stack(st, host(x), tr, lookahead=lookahead)
    # with fixed-order reductions the same step again gives the same bits (the lookahead
    # stack's default adds the projections to x with atomics, in a scheduling order)
    with deterministic():
        xd, trd = st.run(lookahead=lookahead)
        check_stack(st, host(xd), trd, lookahead=lookahead)
        x2, _ = st.run(lookahead=lookahead)
    assert np.array_equal(host(xd), host(x2))
    if not lookahead:
        assert np.array_equal(host(x), host(xd))


# Sets whose sizes are known only on the device (threshold selection, or the union of
# per-token top-k sets) make the fused projection launches lay the rows of all their
# segments end to end and share every block among them.
@pytest.mark.parametrize("B,mode,t", [(1, dj.DJV_THRESHOLD, 0.6), (3, dj.DJV_THRESHOLD, 0.7),
                                      (3, dj.DJV_TOPK, None), (2, dj.DJV_TOPK, None),
                                      (4, dj.DJV_TOPK, None)])
def test_stack_device_counts(B, mode, t):
    print(f"lookahead stack with device counts B={B} mode={mode}", flush=True)
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16", B=B)
    if mode == dj.DJV_TOPK:
        st = Stack(s, 3, 25, k_A=2, k_M=75)
    else:
        st = Stack(s, 3, 25, k_A=0, k_M=0, mode=mode, t_A=t, t_M=t)
    x, tr = st.run(lookahead=True)
    assert (tr["counts"][:, 1] > 0).all() and (tr["counts"][:, 1] < s.N).all()
    check_stack(st, host(x), tr, lookahead=True)
    with deterministic():
        xd, trd = st.run(lookahead=True)
        check_stack(st, host(xd), trd, lookahead=True)
        x2, _ = st.run(lookahead=True)
    assert np.array_equal(host(xd), host(x2))


def test_stack_threshold_larger_shape():
    print("lookahead threshold stack d=4096", flush=True)
    s = synth.LayerShape(d=4096, N=16384, h=32, dh=128, n=512, r=1024, dtype="f16")
    st = Stack(s, 2, 26, k_A=0, k_M=0, mode=dj.DJV_THRESHOLD, t_A=0.6, t_M=0.7)
    x, tr = st.run(lookahead=True)
    assert (tr["counts"][:, 1] > 0).all() and (tr["counts"][:, 1] < s.N).all()
    check_stack(st, host(x), tr, lookahead=True)


@pytest.mark.parametrize("t,kept", [(0.999999, "none"), (1e-6, "all")])
def test_stack_threshold_keeps_none_or_all(t, kept):
    print(f"lookahead threshold stack keeping {kept}", flush=True)
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")
    st = Stack(s, 2, 27, k_A=0, k_M=0, mode=dj.DJV_THRESHOLD, t_A=t, t_M=t)
    x, tr = st.run(lookahead=True)
    want = (0, 0) if kept == "none" else (s.h, s.N)
    assert (tr["counts"] == np.array(want)).all(), tr["counts"]
    check_stack(st, host(x), tr, lookahead=True)
    if kept == "none":
        # nothing computed: each layer passes its input through unchanged
        assert np.array_equal(host(x), host(st.x0))


@pytest.mark.parametrize("k_A,k_M", [(0, 0), (0, 75), (2, 0)])
@pytest.mark.parametrize("lookahead", [True, False])
def test_stack_topk_keeps_nothing(k_A, k_M, lookahead):
    # top-k with k = 0: an empty list of capacity 0; the block it feeds adds nothing
    print(f"top-k stack k_A={k_A} k_M={k_M} lookahead={lookahead}", flush=True)
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")
    st = Stack(s, 3, 28, k_A=k_A, k_M=k_M)
    x, tr = st.run(lookahead=lookahead)
    assert (tr["counts"] == np.array([k_A, k_M])).all(), tr["counts"]
    check_stack(st, host(x), tr, lookahead=lookahead)
    if k_A == 0 and k_M == 0:
        assert np.array_equal(host(x), host(st.x0))


def test_dense_stack_matches_oracle():
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128, n=300, r=136, dtype="f16")
    st = Stack(s, 2, 24, k_A=2, k_M=75)
    t, tr = st.trace()
    x = st.x0.clone()
    dj.dejavu_stack_decode(st.m, st.desc, x, False, True, tr, st.ws)
    torch.cuda.synchronize()
    xs = host(t["x_in"])
    for l in range(2):
        Lw = O.LayerWeights(Wqkv=host(st.w[l]["Wqkv"]), Wo=host(st.w[l]["Wo"]), W1=host(st.w[l]["W1"]),
                            b1=host(st.w[l]["b1"]), W2=host(st.w[l]["W2"]), K=st.K0[l], V=st.V0[l])
        ref, _ = O.dense_layer(xs[l], Lw, s.n, st.scale)
        nxt = host(x) if l == 1 else xs[l + 1]
        assert_close(nxt - xs[l], ref - xs[l], TOL["f16"])


# ------------------------------------------------------------------------ full-size workloads
def _workload_stack(name, L=None, B=None):
    wl = configs.WORKLOADS[name]
    s = wl.shape if B is None else wl.shape.with_(B=B)
    return wl, Stack(s, L or wl.layers, 0, k_A=wl.k_A, k_M=wl.k_M)


def test_opt125m_layer_fp32():
    wl, st = _workload_stack("opt125m-1layer-fp32")
    assert (st.k_A, st.k_M) == (3, 154)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)


@pytest.mark.slow
def test_opt175b_layer():
    print("opt175b one layer", flush=True)
    wl, st = _workload_stack("opt175b-1layer-fp16")
    assert (st.k_A, st.k_M) == (20, 2458)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)


@pytest.mark.slow
def test_opt175b_lookahead_stack():
    # the benchmark's launch configuration (lookahead stack, fused launches) at its full
    # layer shape, two layers
    print("opt175b 2-layer lookahead", flush=True)
    wl, st = _workload_stack("opt175b-24layers-fp16", L=2)
    assert (st.k_A, st.k_M) == (20, 2458)
    x, tr = st.run(lookahead=True)
    check_stack(st, host(x), tr, lookahead=True)


@pytest.mark.slow
def test_opt6_7b_lookahead_stack():
    print("opt6.7b 3-layer lookahead", flush=True)
    wl, st = _workload_stack("opt6.7b-32layers-fp16", L=3)
    assert (st.k_A, st.k_M) == (7, 820)
    x, tr = st.run(lookahead=True)
    check_stack(st, host(x), tr, lookahead=True)


@pytest.mark.slow
@pytest.mark.parametrize("B", [1, 4])
def test_opt66b_layer(B):
    print(f"opt66b one layer B={B}", flush=True)
    wl, st = _workload_stack("opt66b-1layer-fp16", B=B)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)
    if B == 4:
        # union of per-token sets
        assert tr["counts"][0, 1] >= st.k_M and tr["counts"][0, 0] >= st.k_A
