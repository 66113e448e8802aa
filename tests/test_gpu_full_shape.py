"""The matrix-core form (batches above four tokens) against the oracle at the full layer
shapes it is measured at: one OPT-175B-shaped layer at batch 8 and 32, a 2-layer
OPT-175B-shaped lookahead stack at batch 16, and one OPT-66B-shaped layer at batch 8.

These are the launches of the batch sweep at their real sizes: 7 k-slices of the
matrix-core GEMV at d = 12288, unions of thousands of neurons and most heads, and a
workspace of about 150 MiB.  Every layer is checked as in the other layer tests
(teacher-forced on the GPU's own input and sets): scores, each token's set, x', the
appended K and V rows and the layer output, with the element-wise bound beside the
relative L2 error."""
import numpy as np
import pytest

from contextual_sparsity_amd import configs
from helpers import host
from test_gpu_layer import Stack, check_stack

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _stack(name, B, L=1, seed=0):
    wl = configs.WORKLOADS[name]
    return Stack(wl.shape.with_(B=B), L, seed, k_A=wl.k_A, k_M=wl.k_M)


@pytest.mark.parametrize("B", [8, 32])
def test_opt175b_layer_matrix_core(B):
    print(f"opt175b one layer B={B} (matrix cores)", flush=True)
    st = _stack("opt175b-1layer-fp16", B)
    x, tr = st.run(lookahead=False, single_layer=True)
    # unions of per-token sets: larger than one token's, at most all units
    assert st.k_A <= tr["counts"][0, 0] <= st.s.h and st.k_M <= tr["counts"][0, 1] <= st.s.N
    print(f"  union heads {tr['counts'][0, 0]} neurons {tr['counts'][0, 1]}", flush=True)
    check_stack(st, host(x), tr, lookahead=False)


def test_opt175b_lookahead_stack_batch16():
    print("opt175b 2-layer lookahead stack B=16 (matrix cores)", flush=True)
    st = _stack("opt175b-24layers-fp16", 16, L=2)
    x, tr = st.run(lookahead=True)
    assert (tr["counts"][:, 1] >= st.k_M).all()
    check_stack(st, host(x), tr, lookahead=True)


def test_opt66b_layer_batch8():
    print("opt66b one layer B=8 (matrix cores)", flush=True)
    st = _stack("opt66b-1layer-fp16", 8)
    x, tr = st.run(lookahead=False, single_layer=True)
    check_stack(st, host(x), tr, lookahead=False)
    # the layer's output is not its input (something was added)
    assert not np.array_equal(host(x), host(st.x0))
