"""Tolerances and comparison helpers for GPU-vs-oracle parity tests.

Tolerances (the bar the tests enforce):
  fp32 inputs: max |O - O*| <= 1e-5 * max |O*|, |LSE - LSE*| <= 1e-5 * max(1, |LSE*|).
  bf16 inputs (fp32 accumulation): max |O - O*| <= 2e-2 and mean |O - O*| <= 2e-3;
    in addition ||O - O*||_F <= 1e-2 ||O*||_F (so an all-zero output of a
    near-uniform softmax cannot pass) and max |LSE - LSE*| <= 1e-3.
  The extra bf16 bounds follow from the arithmetic: scores are exact bf16
  products summed in fp32 (LSE error ~1e-6 relative), P is rounded once to
  bf16 (2^-9 relative, unbiased) and O once more on output.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_FRO = 1e-2
BF16_LSE_ABS = 1e-3
F32_REL = 1e-5
GRAD_REL_FRO = 2e-2


def to64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def check_fwd(o, lse, o_ref, lse_ref, dtype, what=""):
    """Compare GPU (o, lse) with oracle (o_ref, lse_ref); raises AssertionError."""
    o, lse = to64(o), to64(lse)
    o_ref, lse_ref = np.asarray(o_ref, np.float64), np.asarray(lse_ref, np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    if dtype == "f32":
        scale = max(np.abs(o_ref).max(), 1e-30)
        assert err.max() <= F32_REL * scale, f"{what}: max err {err.max():.3e} > {F32_REL}*{scale:.3e}"
        lerr = np.abs(lse[fin] - lse_ref[fin])
        bound = F32_REL * np.maximum(1.0, np.abs(lse_ref[fin]))
        assert np.all(lerr <= bound), f"{what}: LSE err {lerr.max():.3e}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max abs err {err.max():.3e}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs err {err.mean():.3e}"
        fro = np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
        assert fro <= BF16_REL_FRO, f"{what}: rel Frobenius err {fro:.3e}"
        if fin.any():
            lerr = np.abs(lse[fin] - lse_ref[fin]).max()
            assert lerr <= BF16_LSE_ABS, f"{what}: LSE max abs err {lerr:.3e}"
    return float(err.max())


def check_grad(g, g_ref, what=""):
    g, g_ref = to64(g), np.asarray(g_ref, np.float64)
    assert g.shape == g_ref.shape, (g.shape, g_ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    fro = np.linalg.norm(g - g_ref) / max(np.linalg.norm(g_ref), 1e-30)
    assert fro <= GRAD_REL_FRO, f"{what}: rel Frobenius err {fro:.3e}"
    return float(fro)


def sample_rows(B, H, SQ, n, per_head=8, seed=0):
    """Flat row indices: every (b, h) gets rows 0, SQ-1, both sides of every
    query-block boundary, and `per_head` seeded random rows."""
    g = np.random.default_rng(seed)
    special = {0, SQ - 1}
    for k in range(1, n):
        s = k * SQ // n
        special.update({s - 1, s})
    rows = []
    for bh in range(B * H):
        rs = set(x for x in special if 0 <= x < SQ)
        rs.update(g.integers(0, SQ, size=per_head).tolist())
        rows.extend(bh * SQ + r for r in sorted(rs))
    return np.array(rows, dtype=np.int64)
