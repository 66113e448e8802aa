"""ctypes binding of libdejavu.so, with the C ABI's names.

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  Tensor arguments may be torch tensors (their ``data_ptr()`` is passed) or raw
integer addresses; ``None`` passes NULL.  Streams are torch streams, raw hipStream_t
integers or ``None`` (the current torch stream when a GPU is present, else NULL).
A non-zero status raises :class:`DejavuError` carrying the library's message.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
# DEJAVU_LIB selects another build of the same library (e.g. the sanitizer build of the
# host code); by default the in-tree libdejavu.so
LIB_PATH = os.environ.get("DEJAVU_LIB") or os.path.join(PKG, "libdejavu.so")

DJV_OK, DJV_EINVAL, DJV_EALIGN, DJV_EWORKSPACE, DJV_EUNSUPPORTED, DJV_EHIP = 0, -1, -2, -3, -4, -5
DJV_F32, DJV_F16 = 0, 1
DJV_TOPK, DJV_THRESHOLD = 0, 1
DJV_FLAG_BAD_INDEX, DJV_FLAG_BAD_COUNT = 1, 2
DJV_MAX_BATCH = 32
DJV_MAX_VALU_BATCH = 4

STATUS_NAMES = {0: "DJV_OK", -1: "DJV_EINVAL", -2: "DJV_EALIGN", -3: "DJV_EWORKSPACE",
                -4: "DJV_EUNSUPPORTED", -5: "DJV_EHIP"}

# every entry point declared in include/dejavu.h
EXPORTS = [
    "dejavu_workspace_bytes", "dejavu_workspace_bytes_model", "dejavu_layernorm", "dejavu_select",
    "dejavu_select_range", "dejavu_predict", "dejavu_sparse_mlp", "dejavu_sparse_mlp_no_alloc",
    "dejavu_dense_mlp",
    "dejavu_sparse_mha", "dejavu_dense_mha", "dejavu_neuron_norms", "dejavu_head_norms",
    "dejavu_sparse_layer", "dejavu_stack_decode", "dejavu_poll_device_error",
    "dejavu_set_mfma_min_batch", "dejavu_set_deterministic", "dejavu_gather_rows", "dejavu_profile_kernel",
    "dejavu_profile_count",
    "dejavu_read_probe", "dejavu_last_error", "dejavu_version",
]

DJV_PROF = {"off": 0, "qkv": 1, "mlp_up": 2, "mlp_down": 3, "o_proj": 4, "attn": 5, "pred_1": 6,
            "pred_2": 7, "select": 8}


class DejavuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class djv_model(ctypes.Structure):
    _fields_ = [("wt", ctypes.c_int), ("B", ctypes.c_int), ("d", ctypes.c_int), ("N", ctypes.c_int),
                ("h", ctypes.c_int), ("dh", ctypes.c_int), ("r", ctypes.c_int), ("n", ctypes.c_int),
                ("n_cap", ctypes.c_int), ("scale", ctypes.c_float), ("eps", ctypes.c_float),
                ("mode", ctypes.c_int), ("k_A", ctypes.c_int), ("k_M", ctypes.c_int),
                ("t_A", ctypes.c_float), ("t_M", ctypes.c_float), ("h_total", ctypes.c_int),
                ("h_offset", ctypes.c_int), ("N_total", ctypes.c_int), ("N_offset", ctypes.c_int)]


class djv_layer(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("Wqkv", "Wo", "W1", "b1", "W2", "Kc", "Vc", "P1_A", "P2_A", "P1_M", "P2_M",
                 "Y", "kv_len")]


class djv_trace(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("x_in", "x_mid", "z_A", "z_M", "sets_A", "sets_M", "counts")]


_LIB = None
_I, _F, _P, _SZ = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m contextual_sparsity_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "dejavu_workspace_bytes": [_I] * 7 + [ctypes.POINTER(_SZ)],
            "dejavu_workspace_bytes_model": [ctypes.POINTER(djv_model), ctypes.POINTER(_SZ)],
            "dejavu_layernorm": [_I, _I, _P, _P, _F, _P],
            "dejavu_select": [_I, _I, _P, _I, _I, _F, _P, _P, _P, _SZ, _P],
            "dejavu_select_range": [_I, _I, _P, _I, _I, _F, _I, _I, _P, _P, _P, _SZ, _P],
            "dejavu_neuron_norms": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
            "dejavu_head_norms": [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _P, _P, _SZ, _P],
            "dejavu_predict": [_I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _F, _P, _P, _P, _P, _SZ, _P],
            "dejavu_sparse_mlp": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _SZ, _P],
            "dejavu_sparse_mlp_no_alloc": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P],
            "dejavu_dense_mlp": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
            "dejavu_sparse_mha": [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _F,
                                  _P, _P, _P, _SZ, _P],
            "dejavu_dense_mha": [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _F, _P, _P, _P,
                                 _SZ, _P],
            "dejavu_sparse_layer": [ctypes.POINTER(djv_model), ctypes.POINTER(djv_layer), _P,
                                    ctypes.POINTER(djv_trace), _P, _SZ, _P],
            "dejavu_stack_decode": [ctypes.POINTER(djv_model), ctypes.POINTER(djv_layer), _I, _P, _I,
                                    _I, ctypes.POINTER(djv_trace), _P, _SZ, _P],
            "dejavu_poll_device_error": [_P, ctypes.POINTER(ctypes.c_uint32)],
            "dejavu_set_mfma_min_batch": [_I, ctypes.POINTER(_I)],
            "dejavu_set_deterministic": [_I, ctypes.POINTER(_I)],
            "dejavu_gather_rows": [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P],
            "dejavu_profile_kernel": [_I, ctypes.POINTER(_P), _I],
            "dejavu_profile_count": [ctypes.POINTER(_I)],
            "dejavu_read_probe": [_P, _SZ, _P, _P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dejavu_last_error.restype = ctypes.c_char_p
        L.dejavu_last_error.argtypes = []
        L.dejavu_version.restype = ctypes.c_char_p
        L.dejavu_version.argtypes = []
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != DJV_OK:
        raise DejavuError(status, lib().dejavu_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return DJV_F16
    if t.dtype == torch.float32:
        return DJV_F32
    raise TypeError(f"weights must be fp16 or fp32, got {t.dtype}")


# ------------------------------------------------------------------------------ entry points
def dejavu_version() -> str:
    return lib().dejavu_version().decode()


def dejavu_last_error() -> str:
    return lib().dejavu_last_error().decode()


def dejavu_workspace_bytes(B=0, d=0, N=0, h=0, dh=0, r=0, n_cap=0) -> int:
    out = _SZ(0)
    _check(lib().dejavu_workspace_bytes(B, d, N, h, dh, r, n_cap, ctypes.byref(out)))
    return out.value


def dejavu_workspace_bytes_model(m: djv_model) -> int:
    out = _SZ(0)
    _check(lib().dejavu_workspace_bytes_model(ctypes.byref(m), ctypes.byref(out)))
    return out.value


def workspace(nbytes: int, device="cuda"):
    """Caller-owned workspace: a 256-byte aligned uint8 device tensor (torch allocator)."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dejavu_layernorm(B, d, x, y, eps=1e-5, stream=None) -> None:
    _check(lib().dejavu_layernorm(B, d, _ptr(x), _ptr(y), eps, _stream(stream)))


def dejavu_select(B, n_out, z, mode, k, t, idx, count, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_select(B, n_out, _ptr(z), mode, k, t, _ptr(idx), _ptr(count), wp, wb,
                               _stream(stream)))


def dejavu_select_range(B, n_out, z, mode, k, t, lo, hi, idx, count, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_select_range(B, n_out, _ptr(z), mode, k, t, lo, hi, _ptr(idx), _ptr(count),
                                     wp, wb, _stream(stream)))


def dejavu_neuron_norms(wt, B, d, N, y, W1, b1, scores, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_neuron_norms(wt, B, d, N, _ptr(y), _ptr(W1), _ptr(b1), _ptr(scores), wp, wb,
                                     _stream(stream)))


def dejavu_head_norms(wt, B, d, h, dh, n, n_cap, y, Wqkv, Kc, Vc, scale, scores, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_head_norms(wt, B, d, h, dh, n, n_cap, _ptr(y), _ptr(Wqkv), _ptr(Kc), _ptr(Vc),
                                   scale, _ptr(scores), wp, wb, _stream(stream)))


def dejavu_predict(wt, B, d, r, n_out, y, P1, P2, mode, k, t, idx, count, logits, ws,
                   stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_predict(wt, B, d, r, n_out, _ptr(y), _ptr(P1), _ptr(P2), mode, k, t,
                                _ptr(idx), _ptr(count), _ptr(logits), wp, wb, _stream(stream)))


def dejavu_sparse_mlp(wt, B, d, N, y, W1, b1, W2, idx, count, cap, resid, out, ws,
                      stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_sparse_mlp(wt, B, d, N, _ptr(y), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(idx),
                                   _ptr(count), cap, _ptr(resid), _ptr(out), wp, wb,
                                   _stream(stream)))


def dejavu_sparse_mlp_no_alloc(wt, B, d, N, y, W1, b1, W2, idx, count, cap, resid, out,
                               stream=None) -> None:
    _check(lib().dejavu_sparse_mlp_no_alloc(wt, B, d, N, _ptr(y), _ptr(W1), _ptr(b1), _ptr(W2),
                                            _ptr(idx), _ptr(count), cap, _ptr(resid), _ptr(out),
                                            _stream(stream)))


DJV_STATIC_SCRATCH_BYTES = 16 << 20


def dejavu_dense_mlp(wt, B, d, N, y, W1, b1, W2, resid, out, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_dense_mlp(wt, B, d, N, _ptr(y), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(resid),
                                  _ptr(out), wp, wb, _stream(stream)))


def dejavu_sparse_mha(wt, B, d, h, dh, n, n_cap, y, Wqkv, Wo, Kc, Vc, head_idx, head_count, cap,
                      scale, resid, out, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_sparse_mha(wt, B, d, h, dh, n, n_cap, _ptr(y), _ptr(Wqkv), _ptr(Wo),
                                   _ptr(Kc), _ptr(Vc), _ptr(head_idx), _ptr(head_count), cap, scale,
                                   _ptr(resid), _ptr(out), wp, wb, _stream(stream)))


def dejavu_dense_mha(wt, B, d, h, dh, n, n_cap, y, Wqkv, Wo, Kc, Vc, scale, resid, out, ws,
                     stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_dense_mha(wt, B, d, h, dh, n, n_cap, _ptr(y), _ptr(Wqkv), _ptr(Wo),
                                  _ptr(Kc), _ptr(Vc), scale, _ptr(resid), _ptr(out), wp, wb,
                                  _stream(stream)))


def make_model(wt, B, d, N, h, dh, r, n, n_cap, scale, mode=DJV_TOPK, k_A=0, k_M=0, t_A=0.5,
               t_M=0.5, eps=1e-5, shard=None) -> djv_model:
    """shard: None, or (h_total, h_offset, N_total, N_offset) of a tensor-parallel shard
    whose weights hold h heads and N neurons."""
    sh = shard or (0, 0, 0, 0)
    return djv_model(wt, B, d, N, h, dh, r, n, n_cap, scale, eps, mode, k_A, k_M, t_A, t_M, *sh)


def make_layer(w: dict, p: Optional[dict] = None) -> djv_layer:
    """Layer descriptor from tensors named as in the layout of include/dejavu.h."""
    p = p or {}
    get = lambda dct, k: _ptr(dct.get(k))
    return djv_layer(get(w, "Wqkv"), get(w, "Wo"), get(w, "W1"), get(w, "b1"), get(w, "W2"),
                     get(w, "K"), get(w, "V"), get(p, "P1_A"), get(p, "P2_A"), get(p, "P1_M"),
                     get(p, "P2_M"), get(w, "Y"), get(w, "kv_len"))


def make_trace(x_in=None, x_mid=None, z_A=None, z_M=None, sets_A=None, sets_M=None,
               counts=None) -> djv_trace:
    return djv_trace(_ptr(x_in), _ptr(x_mid), _ptr(z_A), _ptr(z_M), _ptr(sets_A), _ptr(sets_M),
                     _ptr(counts))


def dejavu_sparse_layer(m: djv_model, layer: djv_layer, x, trace: Optional[djv_trace], ws,
                        stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib().dejavu_sparse_layer(ctypes.byref(m), ctypes.byref(layer), _ptr(x),
                                     ctypes.byref(trace) if trace is not None else None, wp, wb,
                                     _stream(stream)))


def dejavu_stack_decode(m: djv_model, layers: Sequence[djv_layer], x, lookahead: bool, dense: bool,
                        trace: Optional[djv_trace], ws, stream=None) -> None:
    arr = (djv_layer * len(layers))(*layers)
    wp, wb = _ws(ws)
    _check(lib().dejavu_stack_decode(ctypes.byref(m), arr, len(layers), _ptr(x), int(lookahead),
                                     int(dense), ctypes.byref(trace) if trace is not None else None,
                                     wp, wb, _stream(stream)))


def dejavu_poll_device_error(stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().dejavu_poll_device_error(_stream(stream), ctypes.byref(v)))
    return v.value


def dejavu_gather_rows(wt, rpu, cols, units, W, idx, count, cap, out, stream=None) -> None:
    """The unfused gather of the fusion ablation (see the header)."""
    _check(lib().dejavu_gather_rows(int(wt), int(rpu), int(cols), int(units), _ptr(W), _ptr(idx),
                                    _ptr(count), int(cap), _ptr(out), _stream(stream)))


def dejavu_set_mfma_min_batch(b: int) -> int:
    """Smallest batch that runs on the matrix cores (see the header); returns the old value."""
    prev = _I(0)
    _check(lib().dejavu_set_mfma_min_batch(int(b), ctypes.byref(prev)))
    return prev.value


def dejavu_set_deterministic(on: bool) -> bool:
    """Bitwise-reproducible lookahead stacks on or off (see the header); returns the old value."""
    prev = _I(0)
    _check(lib().dejavu_set_deterministic(int(bool(on)), ctypes.byref(prev)))
    return bool(prev.value)


def dejavu_profile_kernel(family, events=None) -> None:
    """Record the given events around launches of a kernel family (see the header).
    ``events``: a list of 2*capacity torch.cuda.Event(enable_timing=True) or raw handles;
    the binding keeps the handle array alive until the hook is switched off."""
    global _PROF_KEEP
    fam = DJV_PROF[family] if isinstance(family, str) else int(family)
    if fam == 0 or not events:
        _check(lib().dejavu_profile_kernel(0, None, 0))
        _PROF_KEEP = None
        return
    handles = []
    for e in events:
        if not isinstance(e, int):
            e.record()  # materialise the lazily created torch event on the current stream
            e = e.cuda_event
        handles.append(e)
    arr = (_P * len(handles))(*handles)
    _PROF_KEEP = arr
    _check(lib().dejavu_profile_kernel(fam, arr, len(handles) // 2))


def dejavu_profile_count() -> int:
    v = _I(0)
    _check(lib().dejavu_profile_count(ctypes.byref(v)))
    return v.value


_PROF_KEEP = None


def dejavu_read_probe(buf, out, nbytes=None, stream=None) -> None:
    """Plain streaming read of ``nbytes`` of ``buf`` (default: the whole device tensor; a
    multiple of 16 bytes); ``out`` is a one-element 32-bit device tensor (see the header)."""
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check(lib().dejavu_read_probe(_ptr(buf), ctypes.c_size_t(nbytes), _ptr(out), _stream(stream)))
