"""The C ABI on a host without a GPU: the library loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments with the documented status
before making any HIP call (fake, never-dereferenced addresses are passed)."""
import ctypes
import os
import re
import subprocess

import pytest

from contextual_sparsity_amd import dejavu as dj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dejavu.h")

A = 0x10000000      # a 256-byte aligned fake device address (never dereferenced)
MIS = A + 4         # misaligned


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:djv_status|const char\*)\s+(dejavu_\w+)\s*\(", src, re.M)))


def test_header_and_binding_agree():
    assert _declared() == sorted(dj.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = dj.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dj.LIB_PATH], capture_output=True, text=True)
    syms = set(re.findall(r"\sT\s+(dejavu_\w+)", out.stdout))
    assert set(_declared()) <= syms
    assert "gfx950" in dj.dejavu_version()


def test_workspace_sizes():
    small = dj.dejavu_workspace_bytes(1, 768, 3072, 12, 64, 128, 129)
    big = dj.dejavu_workspace_bytes(1, 12288, 49152, 96, 128, 1024, 2049)
    b4 = dj.dejavu_workspace_bytes(4, 12288, 49152, 96, 128, 1024, 2049)
    assert 0 < small < big < b4
    assert b4 < 64 << 20          # modest: tens of MiB at the OPT-175B shape
    m = dj.make_model(dj.DJV_F16, 1, 12288, 49152, 96, 128, 1024, 2048, 2049, 128 ** -0.5,
                      dj.DJV_TOPK, 20, 2458)
    assert 0 < dj.dejavu_workspace_bytes_model(m) <= big
    # top-k with k = 0 (an empty list of capacity 0) is a valid model
    for k_A, k_M in ((0, 0), (0, 2458), (20, 0)):
        m0 = dj.make_model(dj.DJV_F16, 1, 12288, 49152, 96, 128, 1024, 2048, 2049, 128 ** -0.5,
                           dj.DJV_TOPK, k_A, k_M)
        assert 0 < dj.dejavu_workspace_bytes_model(m0) <= big
    with pytest.raises(dj.DejavuError) as e:
        dj.dejavu_workspace_bytes(-1)
    assert e.value.status == dj.DJV_EINVAL


def _status(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except dj.DejavuError as e:
        assert dj.dejavu_last_error() == e.message and e.message
        return e.status
    return dj.DJV_OK


WS = (A, 1 << 30)


def test_select_argument_errors():
    s = dj.dejavu_select
    assert _status(s, 0, 10, A, dj.DJV_TOPK, 1, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 0, A, dj.DJV_TOPK, 0, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 70000, A, dj.DJV_TOPK, 1, 0.5, A, A, WS) == dj.DJV_EUNSUPPORTED
    assert _status(s, 1, 10, A, dj.DJV_TOPK, 11, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, A, dj.DJV_TOPK, -1, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, A, dj.DJV_THRESHOLD, 0, 1.0, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, A, dj.DJV_THRESHOLD, 0, 0.0, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, A, 7, 0, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, None, dj.DJV_TOPK, 1, 0.5, A, A, WS) == dj.DJV_EINVAL
    assert _status(s, 1, 10, MIS, dj.DJV_TOPK, 1, 0.5, A, A, WS) == dj.DJV_EALIGN
    assert _status(s, 1, 10, A, dj.DJV_TOPK, 1, 0.5, A, A + 2, WS) == dj.DJV_EALIGN
    assert _status(s, 1, 10, A, dj.DJV_TOPK, 1, 0.5, A, A, (A, 0)) == dj.DJV_EWORKSPACE
    assert _status(s, 1, 10, A, dj.DJV_TOPK, 1, 0.5, A, A, (A + 16, 1 << 20)) == dj.DJV_EALIGN
    assert _status(s, 1, 10, A, dj.DJV_TOPK, 1, 0.5, A, A, None) == dj.DJV_EINVAL


def test_predict_argument_errors():
    p = dj.dejavu_predict
    ok = dict(wt=dj.DJV_F16, B=1, d=768, r=128, n_out=3072, y=A, P1=A, P2=A, mode=dj.DJV_TOPK,
              k=154, t=0.5, idx=A, count=A, logits=None, ws=WS)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(p, **a)
    assert call(wt=5) == dj.DJV_EINVAL
    assert call(B=0) == dj.DJV_EINVAL
    assert call(B=dj.DJV_MAX_BATCH + 1) == dj.DJV_EUNSUPPORTED
    # batches above the vector-ALU limit need fp16 weights and row lengths divisible by 32
    assert call(B=5, wt=dj.DJV_F32) == dj.DJV_EUNSUPPORTED
    assert call(B=5, d=776) == dj.DJV_EUNSUPPORTED
    assert call(B=5, r=136) == dj.DJV_EUNSUPPORTED
    assert call(d=100) == dj.DJV_EINVAL
    assert call(d=20000) == dj.DJV_EUNSUPPORTED
    assert call(r=0) == dj.DJV_EINVAL
    assert call(k=3073) == dj.DJV_EINVAL
    assert call(P2=None) == dj.DJV_EINVAL
    assert call(P1=MIS) == dj.DJV_EALIGN
    assert call(logits=MIS) == dj.DJV_EALIGN
    assert call(ws=(A, 16)) == dj.DJV_EWORKSPACE


def test_mlp_argument_errors():
    f = dj.dejavu_sparse_mlp
    ok = dict(wt=dj.DJV_F32, B=1, d=768, N=3072, y=A, W1=A, b1=A, W2=A, idx=A, count=A, cap=154,
              resid=None, out=A, ws=WS)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(f, **a)
    assert call(cap=0) == dj.DJV_EINVAL
    assert call(cap=3073) == dj.DJV_EINVAL
    assert call(idx=None) == dj.DJV_EINVAL
    assert call(count=A + 2) == dj.DJV_EALIGN
    assert call(W2=MIS) == dj.DJV_EALIGN
    assert call(resid=MIS) == dj.DJV_EALIGN
    assert call(out=None) == dj.DJV_EINVAL
    assert call(N=0) == dj.DJV_EINVAL
    assert call(B=6) == dj.DJV_EUNSUPPORTED  # fp32 weights stay on the vector ALU
    assert call(B=6, wt=dj.DJV_F16, d=776) == dj.DJV_EUNSUPPORTED
    assert call(ws=(A, 1024)) == dj.DJV_EWORKSPACE
    assert _status(dj.dejavu_dense_mlp, dj.DJV_F32, 1, 768, 3072, A, A, A, A, None, A, (A, 1024)) \
        == dj.DJV_EWORKSPACE


def test_mlp_no_alloc_argument_errors():
    """The allocation-free MLP rejects what dejavu_sparse_mlp rejects, and calls whose scratch
    exceeds the static buffer, all before its first HIP call."""
    f = dj.dejavu_sparse_mlp_no_alloc
    ok = dict(wt=dj.DJV_F32, B=1, d=768, N=3072, y=A, W1=A, b1=A, W2=A, idx=A, count=A, cap=154,
              resid=None, out=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(f, **a)
    assert call(cap=0) == dj.DJV_EINVAL
    assert call(cap=3073) == dj.DJV_EINVAL
    assert call(idx=None) == dj.DJV_EINVAL
    assert call(count=A + 2) == dj.DJV_EALIGN
    assert call(W1=MIS) == dj.DJV_EALIGN
    assert call(out=None) == dj.DJV_EINVAL
    assert call(B=6) == dj.DJV_EUNSUPPORTED
    # the OPT-175B MLP fits at batch 1 with every neuron; at batch 32 it does not
    need = dj.dejavu_workspace_bytes(32, 12288, 49152, 0, 0, 0, 0)
    assert need > dj.DJV_STATIC_SCRATCH_BYTES
    big = dict(wt=dj.DJV_F16, d=12288, N=49152)
    assert call(B=32, cap=49152, **big) == dj.DJV_EUNSUPPORTED
    assert "static scratch" in dj.dejavu_last_error()
    assert dj.dejavu_workspace_bytes(1, 12288, 49152, 0, 0, 0, 0) <= dj.DJV_STATIC_SCRATCH_BYTES


def test_mha_argument_errors():
    f = dj.dejavu_sparse_mha
    ok = dict(wt=dj.DJV_F16, B=1, d=768, h=12, dh=64, n=128, n_cap=129, y=A, Wqkv=A, Wo=A, Kc=A,
              Vc=A, head_idx=A, head_count=A, cap=3, scale=0.125, resid=None, out=A, ws=WS)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(f, **a)
    assert call(dh=96) == dj.DJV_EUNSUPPORTED
    assert call(n=129) == dj.DJV_EINVAL
    assert call(n=-1) == dj.DJV_EINVAL
    assert call(cap=13) == dj.DJV_EINVAL
    assert call(scale=float("nan")) == dj.DJV_EINVAL
    assert call(Kc=None) == dj.DJV_EINVAL
    assert call(Vc=MIS) == dj.DJV_EALIGN
    assert call(head_idx=None) == dj.DJV_EINVAL
    assert call(B=33) == dj.DJV_EUNSUPPORTED
    assert call(B=8, d=776) == dj.DJV_EUNSUPPORTED
    assert call(ws=(A, 64)) == dj.DJV_EWORKSPACE


def test_layer_and_stack_argument_errors():
    m = dj.make_model(dj.DJV_F16, 1, 768, 3072, 12, 64, 128, 128, 129, 0.125, dj.DJV_TOPK, 3, 154)
    w = {k: A for k in ("Wqkv", "Wo", "W1", "b1", "W2", "K", "V")}
    p = {k: A for k in ("P1_A", "P2_A", "P1_M", "P2_M")}
    L = dj.make_layer(w, p)
    assert _status(dj.dejavu_sparse_layer, m, L, A, None, (A, 16)) == dj.DJV_EWORKSPACE
    bad = dj.make_model(dj.DJV_F16, 1, 768, 3072, 12, 64, 128, 128, 129, 0.125, dj.DJV_TOPK, 13, 154)
    assert _status(dj.dejavu_sparse_layer, bad, L, A, None, WS) == dj.DJV_EINVAL
    bad = dj.make_model(dj.DJV_F16, 1, 768, 3072, 12, 64, 128, 128, 129, 0.125, dj.DJV_THRESHOLD, 0, 0,
                        t_A=1.5)
    assert _status(dj.dejavu_sparse_layer, bad, L, A, None, WS) == dj.DJV_EINVAL
    bad = dj.make_model(dj.DJV_F16, 1, 768, 3072, 12, 64, 128, 128, 129, 0.125, eps=0.0)
    assert _status(dj.dejavu_sparse_layer, bad, L, A, None, WS) == dj.DJV_EINVAL
    bad = dj.make_model(dj.DJV_F16, 16, 768, 3072, 12, 64, 136, 128, 129, 0.125)
    assert _status(dj.dejavu_sparse_layer, bad, L, A, None, WS) == dj.DJV_EUNSUPPORTED
    bad = dj.make_model(dj.DJV_F32, 16, 768, 3072, 12, 64, 128, 128, 129, 0.125)
    assert _status(dj.dejavu_sparse_layer, bad, L, A, None, WS) == dj.DJV_EUNSUPPORTED
    L2 = dj.make_layer(w, dict(p, P2_M=None))
    assert _status(dj.dejavu_sparse_layer, m, L2, A, None, WS) == dj.DJV_EINVAL
    assert _status(dj.dejavu_stack_decode, m, [L, L2], A, True, False, None, WS) == dj.DJV_EINVAL
    assert _status(dj.dejavu_stack_decode, m, [], A, True, False, None, WS) == dj.DJV_EINVAL
    assert _status(dj.dejavu_layernorm, 1, 768, A, A, 0.0) == dj.DJV_EINVAL
    assert _status(dj.dejavu_layernorm, 1, 768, MIS, A, 1e-5) == dj.DJV_EALIGN
    with pytest.raises(dj.DejavuError):
        dj.lib().dejavu_poll_device_error(None, None) and None or dj._check(
            dj.lib().dejavu_poll_device_error(None, None))


def test_mfma_min_batch_setting():
    assert _status(dj.dejavu_set_mfma_min_batch, 0) == dj.DJV_EINVAL
    assert _status(dj.dejavu_set_mfma_min_batch, dj.DJV_MAX_VALU_BATCH + 2) == dj.DJV_EINVAL
    old = dj.dejavu_set_mfma_min_batch(1)
    assert old == dj.DJV_MAX_VALU_BATCH + 1
    try:
        # workspace sizes do not depend on the setting
        a = dj.dejavu_workspace_bytes(2, 1024, 3000, 8, 128, 128, 200)
        dj.dejavu_set_mfma_min_batch(dj.DJV_MAX_VALU_BATCH + 1)
        assert dj.dejavu_workspace_bytes(2, 1024, 3000, 8, 128, 128, 200) == a
    finally:
        assert dj.dejavu_set_mfma_min_batch(old) in (1, dj.DJV_MAX_VALU_BATCH + 1)


def test_deterministic_setting():
    f = dj.lib().dejavu_set_deterministic
    assert f(2, None) == dj.DJV_EINVAL and f(-1, None) == dj.DJV_EINVAL
    old = dj.dejavu_set_deterministic(True)
    assert old is False
    try:
        assert dj.dejavu_set_deterministic(True) is True
    finally:
        assert dj.dejavu_set_deterministic(old) is True


def test_gather_rows_argument_errors():
    g = dj.dejavu_gather_rows
    ok = dict(wt=dj.DJV_F16, rpu=1, cols=768, units=3072, W=A, idx=A, count=A, cap=154, out=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(g, **a)
    assert call(wt=3) == dj.DJV_EINVAL
    assert call(rpu=0) == dj.DJV_EINVAL
    assert call(cols=0) == dj.DJV_EINVAL
    assert call(cap=0) == dj.DJV_EINVAL
    assert call(cap=3073) == dj.DJV_EINVAL
    assert call(W=None) == dj.DJV_EINVAL
    assert call(idx=None) == dj.DJV_EINVAL
    assert call(count=A + 2) == dj.DJV_EALIGN
    assert call(out=MIS) == dj.DJV_EALIGN          # 1536-byte rows need 16-byte alignment
    assert call(cols=2, out=A + 2) == dj.DJV_EALIGN  # 4-byte rows need 4-byte alignment


def test_read_probe_argument_errors():
    p = dj.dejavu_read_probe
    assert _status(p, A, A, nbytes=0) == dj.DJV_EINVAL
    assert _status(p, A, A, nbytes=24) == dj.DJV_EINVAL      # not a multiple of 16
    assert _status(p, None, A, nbytes=64) == dj.DJV_EINVAL
    assert _status(p, A, None, nbytes=64) == dj.DJV_EINVAL
    assert _status(p, A + 8, A, nbytes=64) == dj.DJV_EALIGN
    assert _status(p, A, A + 2, nbytes=64) == dj.DJV_EALIGN
