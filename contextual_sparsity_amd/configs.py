"""OPT-shaped synthetic decode workloads.

Each workload is a layer shape, a layer count, the keep-percentages of MLP neurons
and attention heads, and whether the next layer's sets are predicted ahead (the
lookahead schedule) or each layer predicts its own sets in order (serial schedule).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

from .synth import LayerShape


def keep(pct: int, n: int) -> int:
    """Units kept at an integer keep-percentage: ceil(pct * n / 100) in integers."""
    if not (0 <= pct <= 100):
        raise ValueError("keep percentage must lie in [0, 100]")
    return (pct * n + 99) // 100


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    layers: int
    pct_M: int
    pct_A: int
    lookahead: bool

    @property
    def k_M(self) -> int:
        return keep(self.pct_M, self.shape.N)

    @property
    def k_A(self) -> int:
        return keep(self.pct_A, self.shape.h)

    @property
    def scale(self) -> float:
        return self.shape.dh ** -0.5


WORKLOADS: Dict[str, Workload] = {
    # one OPT-125m-shaped layer, fp32, serial prediction
    "opt125m-1layer-fp32": Workload(
        "opt125m-1layer-fp32", LayerShape(d=768, N=3072, h=12, dh=64, n=128, r=128, dtype="f32"),
        layers=1, pct_M=5, pct_A=20, lookahead=False),
    # 32 OPT-6.7B-shaped layers, fp16, lookahead predictor
    "opt6.7b-32layers-fp16": Workload(
        "opt6.7b-32layers-fp16", LayerShape(d=4096, N=16384, h=32, dh=128, n=1024, r=1024),
        layers=32, pct_M=5, pct_A=20, lookahead=True),
    # one OPT-66B-shaped layer, fp16, batch 1 (batch 4 via shape.with_(B=4))
    "opt66b-1layer-fp16": Workload(
        "opt66b-1layer-fp16", LayerShape(d=9216, N=36864, h=72, dh=128, n=2048, r=1024),
        layers=1, pct_M=5, pct_A=20, lookahead=False),
    # 24 OPT-175B-shaped layers, fp16, lookahead predictor
    "opt175b-24layers-fp16": Workload(
        "opt175b-24layers-fp16", LayerShape(d=12288, N=49152, h=96, dh=128, n=2048, r=1024),
        layers=24, pct_M=5, pct_A=20, lookahead=True),
    # one OPT-175B-shaped layer (the sweep's base point)
    "opt175b-1layer-fp16": Workload(
        "opt175b-1layer-fp16", LayerShape(d=12288, N=49152, h=96, dh=128, n=2048, r=1024),
        layers=1, pct_M=5, pct_A=20, lookahead=False),
}

# Sparsity and batch sweep on the OPT-175B layer shape: per-token keep-percentages of
# neurons and heads crossed with the batch size (union index sets)
SWEEP_PCT_M = (1, 2, 5, 10, 25, 50, 100)
SWEEP_PCT_A = (10, 20, 50, 100)
SWEEP_BATCH = (1, 2, 4, 8, 16, 32)


def shard_range(n: int, g: int, i: int) -> Tuple[int, int]:
    """Units [lo, hi) of shard i when n units are split over g shards in contiguous
    ranges, the first n % g shards one unit longer."""
    base, extra = divmod(n, g)
    lo = i * base + min(i, extra)
    return lo, lo + base + (1 if i < extra else 0)
