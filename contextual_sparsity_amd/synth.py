"""Seeded synthetic inputs for the sparse decode layer.

This module only draws random numbers and fills constants; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle are fed the tensors it
returns, so the two sides always see identical inputs.

Distributions (the OPT-shaped synthetic workload):
  weights (Wqkv, Wo, W1, W2)        N(0, 0.02^2), stored in the weight dtype
  b1                                the constant -0.05, stored in the weight dtype
  predictor weights (P1_*, P2_*)    N(0, 0.05^2), stored in the weight dtype
  layer input x                     N(0, 1), fp32 (the layer normalises it itself)
  cached K and V (positions < n)    N(0, 0.02^2 * d), the law of one entry of a
                                    LayerNorm-ed N(0, 1) embedding projected by
                                    N(0, 0.02^2) weights; stored in the weight dtype
Every tensor has its own stream, keyed by (seed, layer, tensor id), so a tensor does
not change when another one is added or resized.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Tuple

import torch

_TID = {"Wqkv": 1, "Wo": 2, "W1": 3, "W2": 4, "K": 5, "V": 6,
        "P1_A": 7, "P2_A": 8, "P1_M": 9, "P2_M": 10, "x": 11, "z": 12}

W_STD = 0.02
P_STD = 0.05
B1_VALUE = -0.05


@dataclass(frozen=True)
class LayerShape:
    """Shapes of one decoder layer and its predictors."""
    d: int            # model width
    N: int            # MLP neurons (4d)
    h: int            # attention heads
    dh: int           # head width
    n: int            # cached positions before this step
    r: int            # predictor hidden width
    B: int = 1        # sequences in the batch
    dtype: str = "f16"  # weight and KV-cache dtype: "f16" or "f32"
    n_cap: int = 0    # cache capacity per head (0: n + 1)

    @property
    def cap(self) -> int:
        return self.n_cap if self.n_cap else self.n + 1

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.float32

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


def seed_of(seed: int, layer: int, name: str) -> int:
    """Independent 63-bit stream key for (seed, layer, tensor name)."""
    v = (seed * 0x9E3779B97F4A7C15 + layer * 0xBF58476D1CE4E5B9 + _TID[name] * 0x94D049BB133111EB)
    v &= (1 << 64) - 1
    v ^= v >> 31
    return v & ((1 << 63) - 1)


def normal(shape, std: float, dtype, device, key: int) -> torch.Tensor:
    """N(0, std^2) samples drawn in fp32 from a generator seeded with ``key``, then
    rounded to ``dtype``.  Large tensors are drawn in slabs to bound temporaries."""
    g = torch.Generator(device=device)
    g.manual_seed(key)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    slab = 1 << 26
    for s in range(0, flat.numel(), slab):
        e = min(flat.numel(), s + slab)
        tmp = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        flat[s:e] = (tmp * std).to(dtype)
    return out


def make_layer(shape: LayerShape, seed: int, layer: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Weights and KV cache of one layer, in the stored layouts:
    Wqkv [h,3,dh,d], Wo [h*dh,d], W1 [N,d], b1 [N], W2 [N,d], K and V [B,h,cap,dh]."""
    s, dt = shape, shape.torch_dtype
    w = {
        "Wqkv": normal((s.h, 3, s.dh, s.d), W_STD, dt, device, seed_of(seed, layer, "Wqkv")),
        "Wo": normal((s.h * s.dh, s.d), W_STD, dt, device, seed_of(seed, layer, "Wo")),
        "W1": normal((s.N, s.d), W_STD, dt, device, seed_of(seed, layer, "W1")),
        "b1": torch.full((s.N,), B1_VALUE, dtype=dt, device=device),
        "W2": normal((s.N, s.d), W_STD, dt, device, seed_of(seed, layer, "W2")),
    }
    kv_std = W_STD * math.sqrt(s.d)
    w["K"] = normal((s.B, s.h, s.cap, s.dh), kv_std, dt, device, seed_of(seed, layer, "K"))
    w["V"] = normal((s.B, s.h, s.cap, s.dh), kv_std, dt, device, seed_of(seed, layer, "V"))
    return w


def make_predictors(shape: LayerShape, seed: int, layer: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Head predictor P1_A [r,d], P2_A [h,r] and neuron predictor P1_M [r,d], P2_M [N,r]."""
    s, dt = shape, shape.torch_dtype
    return {
        "P1_A": normal((s.r, s.d), P_STD, dt, device, seed_of(seed, layer, "P1_A")),
        "P2_A": normal((s.h, s.r), P_STD, dt, device, seed_of(seed, layer, "P2_A")),
        "P1_M": normal((s.r, s.d), P_STD, dt, device, seed_of(seed, layer, "P1_M")),
        "P2_M": normal((s.N, s.r), P_STD, dt, device, seed_of(seed, layer, "P2_M")),
    }


def make_input(shape: LayerShape, seed: int, device="cpu") -> torch.Tensor:
    """Layer input x [B, d], fp32 N(0, 1)."""
    return normal((shape.B, shape.d), 1.0, torch.float32, device, seed_of(seed, 0, "x"))


def make_scores(B: int, n_out: int, seed: int, device="cpu", alphabet=None) -> torch.Tensor:
    """Selection test scores [B, n_out] fp32: N(0, 1), or drawn uniformly from a small
    alphabet of values so that ties are frequent."""
    key = seed_of(seed, 0, "z")
    if alphabet is None:
        return normal((B, n_out), 1.0, torch.float32, device, key)
    g = torch.Generator(device="cpu")
    g.manual_seed(key)
    a = torch.tensor(alphabet, dtype=torch.float32)
    idx = torch.randint(0, len(alphabet), (B, n_out), generator=g)
    return a[idx].to(device)


def shard_layer(w: Dict[str, torch.Tensor], heads: Tuple[int, int], neurons: Tuple[int, int],
                dh: int) -> Dict[str, torch.Tensor]:
    """One tensor-parallel shard of a layer: the Wqkv blocks, Wo rows and caches of heads
    [lo, hi) and the W1, b1, W2 rows of neurons [lo, hi), as contiguous copies."""
    (h0, h1), (n0, n1) = heads, neurons
    return {"Wqkv": w["Wqkv"][h0:h1].contiguous(), "Wo": w["Wo"][h0 * dh:h1 * dh].contiguous(),
            "W1": w["W1"][n0:n1].contiguous(), "b1": w["b1"][n0:n1].contiguous(),
            "W2": w["W2"][n0:n1].contiguous(), "K": w["K"][:, h0:h1].contiguous(),
            "V": w["V"][:, h0:h1].contiguous()}
