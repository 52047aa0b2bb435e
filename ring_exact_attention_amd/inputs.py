"""Seeded synthetic inputs for blockwise / ring attention workloads.

This module holds no attention arithmetic: it only draws seeded random
tensors with the shapes and value distributions of the workloads below, so
the HIP path and the CPU oracle can be fed the very same values.

The workloads stand in for the long-video cross-attention the LV-XAttn review
describes (short text queries against a very long visual key/value sequence;
"Core claim" quotes Video-MME averages of about 5.5K query tokens against
about 15.3M visual tokens over 16 workers); no dataset item is used.  Each
tensor is drawn in fp32 from a CPU or device ``torch.Generator`` and, for bf16
workloads, rounded once to bf16 (round-to-nearest-even); both sides read
those rounded values.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    SQ: int
    SKV: int
    D: int
    n: int
    dtype: str            # "f32" or "bf16"
    causal: bool = False
    std: float = 1.0      # Q, K, V ~ N(0,1) * std
    v_std: float | None = None
    hot_frac: float = 0.0  # fraction of K rows per (b, h) scaled by hot_scale
    hot_scale: float = 1.0
    E: int = 0            # recompute: visual feature width (0: no recompute)
    y_std: float = 0.0
    w_std: float = 0.0
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def resized(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 cross-attention, KV split into 4 blocks of 256.
    "tiny_f32": Workload("tiny_f32", B=1, H=1, SQ=128, SKV=1024, D=64, n=4, dtype="f32",
                         std=1.0, seed=1001),
    # LV-XAttn-shaped cross-attention: 2K text queries against one GPU's
    # 128K-token share of the visual sequence, 8 KV shards.
    "lvx_2k_128k": Workload("lvx_2k_128k", B=1, H=32, SQ=2048, SKV=131072, D=128, n=8,
                            dtype="bf16", std=0.5, seed=1002),
    # Short-query, memory-bound cross-attention; 1% of K rows scaled by 8.
    "shortq_256_256k": Workload("shortq_256_256k", B=4, H=16, SQ=256, SKV=262144, D=128, n=16,
                                dtype="bf16", std=1.0, hot_frac=0.01, hot_scale=8.0,
                                seed=1003),
    # Ring-Attention causal self-attention, 8 blocks of 8192.
    "causal_64k": Workload("causal_64k", B=1, H=32, SQ=65536, SKV=65536, D=128, n=8,
                           dtype="bf16", causal=True, std=0.5, seed=1004),
    # Cross-attention with K, V recomputed from shared visual features + backward.
    "recompute_bwd": Workload("recompute_bwd", B=1, H=32, SQ=2048, SKV=65536, D=128, n=8,
                              dtype="bf16", std=0.5, E=4096, y_std=0.02, w_std=0.02,
                              seed=1005),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device, std: float, dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_qkv(w: Workload, device="cpu", seed: int | None = None):
    """(q, k, v) with q [B,H,SQ,D], k/v [B,H,SKV,D] in the workload's dtype."""
    seed = w.seed if seed is None else seed
    g = _gen(device, seed)
    dt = w.torch_dtype
    q = _randn((w.B, w.H, w.SQ, w.D), g, device, w.std, dt)
    k = _randn((w.B, w.H, w.SKV, w.D), g, device, w.std, dt)
    v = _randn((w.B, w.H, w.SKV, w.D), g, device, w.std if w.v_std is None else w.v_std, dt)
    if w.hot_frac > 0.0:
        nhot = int(round(w.hot_frac * w.SKV))
        gp = _gen("cpu", seed + 7)
        for bh in range(w.B * w.H):
            rows = torch.randperm(w.SKV, generator=gp)[:nhot].to(device)
            kb = k.view(w.B * w.H, w.SKV, w.D)[bh]
            # multiplying by a power of two is exact in bf16 and fp32
            kb[rows] = (kb[rows].float() * w.hot_scale).to(dt)
    return q, k, v


def make_dout(w: Workload, device="cpu", seed: int | None = None, std: float = 1.0):
    """Upstream gradient dO [B,H,SQ,D] ~ N(0,1) * std in the workload's dtype."""
    seed = (w.seed if seed is None else seed) + 101
    g = _gen(device, seed)
    return _randn((w.B, w.H, w.SQ, w.D), g, device, std, w.torch_dtype)


def make_recompute(w: Workload, device="cpu", seed: int | None = None):
    """(y [B,SKV,E], wk_t [H*D,E], wv_t [H*D,E]) for the recompute workload.

    wk_t / wv_t hold W_k / W_v transposed (row n = h*D + d is column n of W).
    """
    seed = (w.seed if seed is None else seed) + 202
    g = _gen(device, seed)
    dt = w.torch_dtype
    y = _randn((w.B, w.SKV, w.E), g, device, w.y_std, dt)
    wk = _randn((w.H * w.D, w.E), g, device, w.w_std, dt)
    wv = _randn((w.H * w.D, w.E), g, device, w.w_std, dt)
    return y, wk, wv
