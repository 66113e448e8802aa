"""End-to-end stack error: the oracle propagates the stack from x_0 on its own (no layer
fed the GPU's input), with the GPU's index sets so that both sides compute the same
sparse function, and the final outputs are compared.  Unlike the teacher-forced checks of
test_gpu_layer, the error here accumulates over the layers; it is printed and held to
the dtype tolerance.  The oracle's own sets from its own activations are also checked
to be valid selections within twice the score gap (they may differ only at near-ties)."""
import numpy as np
import pytest

import oracle as O
from contextual_sparsity_amd import synth
from helpers import TOL, check_sets_valid, host, rel_l2
from test_gpu_layer import Stack, _workload_stack

pytestmark = pytest.mark.gpu


def _end_to_end(st: Stack):
    s = st.s
    x, tr = st.run(lookahead=True)
    x0 = host(st.x0).astype(np.float64)
    xr = x0.copy()
    for l in range(st.L):
        w = st.w[l]
        Lw = O.LayerWeights(Wqkv=host(w["Wqkv"]), Wo=host(w["Wo"]), W1=host(w["W1"]), b1=host(w["b1"]),
                            W2=host(w["W2"]), K=st.K0[l], V=st.V0[l])
        cA, cM = int(tr["counts"][l, 0]), int(tr["counts"][l, 1])
        S_A, S_M = tr["sets_A"][l, :cA], tr["sets_M"][l, :cM]
        if st.mode == O.TOPK and s.B == 1:
            # the oracle's own scores from its own activations select the same sets up to
            # near-ties (the lookahead predictor of layer l reads LN of layer l-1's input)
            src = O.layernorm(xr_prev) if l > 0 else O.layernorm(xr)
            p = st.p[l]
            zA = O.predictor_logits_f64(src, host(p["P1_A"]), host(p["P2_A"]))[0]
            zM = O.predictor_logits_f64(src, host(p["P1_M"]), host(p["P2_M"]))[0]
            dA = float(np.abs(tr["z_A"][l][0] - zA).max())
            dM = float(np.abs(tr["z_M"][l][0] - zM).max())
            check_sets_valid(S_A, zA, st.k_A, dA)
            check_sets_valid(S_M, zM, st.k_M, dM)
        xr_prev = xr
        xr, _, _, _ = O.sparse_layer(xr, Lw, S_A, S_M, s.n, st.scale)
    err = rel_l2(host(x).astype(np.float64) - x0, xr - x0)
    print(f"end-to-end rel L2 over {st.L} layers ({s.dtype}): {err:.3e}", flush=True)
    return err


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_small_stack_end_to_end(dtype):
    s = synth.LayerShape(d=1032, N=1500, h=6, dh=128 if dtype == "f16" else 64, n=300, r=136, dtype=dtype)
    st = Stack(s, 6, 41, k_A=2, k_M=75)
    assert _end_to_end(st) < TOL[dtype]


@pytest.mark.slow
def test_opt6_7b_stack_end_to_end():
    print("opt6.7b 4-layer lookahead, end to end", flush=True)
    wl, st = _workload_stack("opt6.7b-32layers-fp16", L=4)
    assert _end_to_end(st) < TOL["f16"]
