"""GPU selection against the oracle: identical fp32 scores must give bit-identical index
sets (top-k with every tie pattern, threshold, batch unions, edge sizes)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from contextual_sparsity_amd import dejavu as dj
from contextual_sparsity_amd import synth
from helpers import DEV

pytestmark = pytest.mark.gpu


def _gpu_select(z: torch.Tensor, mode, k=0, t=0.5):
    B, n = z.shape
    idx = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = dj.workspace(dj.dejavu_workspace_bytes(B, 0, n, 0, 0, 0, 0), DEV)
    dj.dejavu_select(B, n, z, mode, k, t, idx, cnt, ws)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return idx[:c].cpu().numpy()


@pytest.mark.parametrize("n", [1, 7, 12, 96, 1000, 3072, 4097, 12289, 16384, 36864, 49152, 65536])
def test_topk_normal_scores(n):
    print(f"select topk n={n}", flush=True)
    for B in (1, 3):
        z = synth.make_scores(B, n, seed=n + B).to(DEV)
        zh = z.cpu().numpy()
        for k in sorted({0, 1, max(1, n // 20), (n * 20 + 99) // 100, n - 1, n}):
            if k < 0 or k > n:
                continue
            got = _gpu_select(z, dj.DJV_TOPK, k=k)
            ref = O.select(zh, O.TOPK, k=k)
            assert np.array_equal(got, ref), (n, B, k)


@pytest.mark.parametrize("alphabet", [(0.0, 1.0), (-0.0, 0.0, 2.5, -1.0), (math.nan, -math.inf, 0.5),
                                      (math.nan, math.nan, 0.5), (1.0, 1.0 + 2 ** -23, 1.0 - 2 ** -24)])
def test_topk_ties(alphabet):
    for n in (5, 64, 1031, 16384, 49152):
        z = synth.make_scores(2, n, seed=n, alphabet=alphabet).to(DEV)
        zh = z.cpu().numpy()
        for k in (0, 1, 2, n // 3, 20000 % (n + 1), n // 2, n):
            # repeated: a data race between the block's threads would show as a mismatch
            for _ in range(3 if n > 10000 else 1):
                got = _gpu_select(z[:1], dj.DJV_TOPK, k=k)
                assert np.array_equal(got, O.select(zh[:1], O.TOPK, k=k)), (alphabet, n, k)
            got = _gpu_select(z, dj.DJV_TOPK, k=k)
            assert np.array_equal(got, O.select(zh, O.TOPK, k=k)), (alphabet, n, k, "B=2")


@pytest.mark.parametrize("n", [4097, 16384])
def test_topk_dense_cluster(n):
    # normal scores with a cluster of near-equal values (ties, and keys that differ only in
    # their low bits) placed so that the k-th largest key falls inside it
    z = synth.make_scores(2, n, seed=n + 11)
    g = torch.Generator(device="cpu")
    g.manual_seed(n)
    for b in range(2):
        pos = torch.randperm(n, generator=g)[:2000]
        z[b, pos] = 3.0 + (torch.arange(2000) % 300).float() * 2.0 ** -22
    z = z.to(DEV)
    zh = z.cpu().numpy()
    for k in (5, 40, 820, 1500, 2000, 2100):
        got = _gpu_select(z[:1], dj.DJV_TOPK, k=k)
        assert np.array_equal(got, O.select(zh[:1], O.TOPK, k=k)), (n, k)
        got = _gpu_select(z, dj.DJV_TOPK, k=k)
        assert np.array_equal(got, O.select(zh, O.TOPK, k=k)), (n, k, "B=2")


def test_topk_golden_row():
    vals = [1.0, 3.0, 3.0, -0.0, 0.0, math.nan, 2.0, 3.0, -math.inf]
    z = torch.tensor([vals], dtype=torch.float32, device=DEV)
    for k in range(len(vals) + 1):
        assert np.array_equal(_gpu_select(z, dj.DJV_TOPK, k=k), O.topk_set(np.array(vals, np.float32), k))


@pytest.mark.parametrize("t", [0.5, 0.1, 0.3, 0.77, 0.999])
def test_threshold(t):
    for n, B in ((12, 1), (3072, 2), (49152, 4)):
        z = synth.make_scores(B, n, seed=17 + n).to(DEV) * 3.0
        z[0, : min(4, n)] = torch.tensor([0.0, -0.0, math.nan, -math.inf][: min(4, n)])
        zh = z.cpu().numpy()
        got = _gpu_select(z, dj.DJV_THRESHOLD, t=t)
        assert np.array_equal(got, O.select(zh, O.THRESHOLD, t=t)), (t, n, B)


def test_union_large_batch():
    # the selection call itself accepts any batch; the union is over all rows
    z = synth.make_scores(16, 3072, seed=5).to(DEV)
    got = _gpu_select(z, dj.DJV_TOPK, k=154)
    assert np.array_equal(got, O.select(z.cpu().numpy(), O.TOPK, k=154))


def test_select_deterministic():
    z = synth.make_scores(2, 49152, seed=3, alphabet=(0.0, 1.0, 2.0)).to(DEV)
    a = _gpu_select(z, dj.DJV_TOPK, k=2458)
    b = _gpu_select(z, dj.DJV_TOPK, k=2458)
    assert np.array_equal(a, b)
