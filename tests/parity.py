"""Tolerances and comparison helpers for GPU-vs-oracle parity tests.

Tolerances (the bar the tests enforce):
  fp32 inputs: max |O - O*| <= 1e-5 * max |O*|, |LSE - LSE*| <= 1e-5 * max(1, |LSE*|).
  bf16 inputs (fp32 accumulation): max |O - O*| <= 2e-2 and mean |O - O*| <= 2e-3;
    in addition ||O - O*||_F <= 1e-2 ||O*||_F (so an all-zero output of a
    near-uniform softmax cannot pass) and max |LSE - LSE*| <= 1e-3.
  The extra bf16 bounds follow from the arithmetic: scores are exact bf16
  products summed in fp32 (LSE error ~1e-6 relative), P is rounded once to
  bf16 (at most u = 2^-8 relative, unbiased) and O once more on output.

Gradients (bf16 outputs, fp32 accumulation), element by element:
  per block of 128 rows of one head:  max |g - g*| <= 2e-2 * max |g*| (block);
  per tensor:                          mean |g - g*| <= 6e-3 * mean |g*|;
  per row r:  ||g_r - g*_r|| <= 1.5e-2 ||g*_r|| + 1e-3 * rms_r ||g*_r||;
  and the relative Frobenius error <= 2e-2 as before.
  Derivation (u = 2^-8, the bf16 unit roundoff): an element is a sum of terms
  a_t (P dO for dV; scale dS K for dQ; scale dS Q for dK) each carrying at
  most k independent roundings of relative size <= u (P or dS to bf16; with
  K, V themselves rounded from an exact projection, k <= 4), then one output
  rounding.  Rounding errors of unrelated values are zero-mean with variance
  <= u^2/3, so the error is ~N(0, sigma^2), sigma <= sqrt(k/3) u sqrt(sum a_t^2),
  and sqrt(sum a_t^2) ~ rms|g| for sums of random-sign terms.  Block max:
  6 sigma + u max|g| <= (6 sqrt(4/3)/3 + 1) u max|g| = 3.3u = 1.3e-2 max|g|
  (max|g| >= 3 rms|g| over a block).  Mean: 0.8 sigma + 0.36u mean|g| (mean
  relative output rounding for log-uniform mantissas) <= 1.5u mean|g| =
  5.9e-3 mean|g|.  Row: rms relative sqrt(k/3 + 0.18) u = 1.23u, +24% for
  the chi spread of a 128-element row, 6e-3 < 1.5e-2; the floor covers rows
  whose exact gradient vanishes (causal row 0 of dQ, where dP and Delta are
  the same fp32 sum in two orders).
  dQ rows add one more term (dq_row_allowance): Delta = rowsum(dO * O) is
  formed from the forward's bf16 output, whose elements carry about two
  roundings, so Delta_i is off by dDelta_i ~ N(0, sigma_i^2), sigma_i =
  u sqrt(2/3) ||dO_i * O_i||, and dS_ij = P_ij (dP_ij - Delta_i) moves
  dQ_i by -scale dDelta_i sum_j P_ij K_j.  That is negligible against a long
  row's gradient, but a causal row with few keys whose exact gradient nearly
  cancels (dP_ij close to Delta_i for all its keys) sees it whole: its bound
  gets 6 scale sigma_i ||sum_j P_ij K_j||.
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
GRAD_BLOCK_MAX = 2e-2
GRAD_MEAN = 6e-3
GRAD_ROW = 1.5e-2
GRAD_ROW_FLOOR = 1e-3
U_BF16 = 2.0 ** -8


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


def dq_row_allowance(orc, q, k, v, do, scale, causal):
    """Per-row allowance [B*H, S_Q] for dQ from the rounding of Delta (module
    docstring): 6 scale sigma_i ||sum_j P_ij K_j|| with sigma_i = u sqrt(2/3)
    ||dO_i * O_i||; O and sum_j P_ij K_j (attention with V = K) from the oracle."""
    B, H, SQ, D = q.shape
    O, _ = orc.attn_fwd(q, k, v, scale, causal=causal)
    PK, _ = orc.attn_fwd(q, k, k, scale, causal=causal)
    sigma = U_BF16 * np.sqrt(2.0 / 3.0) * np.linalg.norm(to64(do) * O, axis=-1)
    return (6.0 * scale * sigma * np.linalg.norm(PK, axis=-1)).reshape(B * H, SQ)


def check_grad(g, g_ref, what="", block=128, row_extra=None):
    """Element-wise gradient check (bounds in the module docstring).  g and
    g_ref are [..., rows, D]; blocks are `block` consecutive rows of one
    leading index (one head).  Prints and returns the error summary,
    including the maximum relative error over elements with |g*| above 1e-3
    of the tensor's maximum."""
    g, g_ref = to64(g), np.asarray(g_ref, np.float64)
    assert g.shape == g_ref.shape, (g.shape, g_ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    D = g.shape[-1]
    g3 = g.reshape(-1, g.shape[-2], D)
    r3 = g_ref.reshape(-1, g.shape[-2], D)
    err = np.abs(g3 - r3)
    amax = np.abs(r3).max()
    big = np.abs(r3) > 1e-3 * amax
    max_rel = float((err[big] / np.abs(r3[big])).max()) if big.any() else 0.0
    fro = np.linalg.norm(g3 - r3) / max(np.linalg.norm(r3), 1e-300)
    mean_ratio = err.mean() / max(np.abs(r3).mean(), 1e-300)
    worst_block = 0.0
    for h in range(g3.shape[0]):
        for b0 in range(0, g3.shape[1], block):
            e = err[h, b0:b0 + block].max()
            m = np.abs(r3[h, b0:b0 + block]).max()
            ratio = e / m if m > 0 else (0.0 if e == 0 else np.inf)
            worst_block = max(worst_block, ratio)
    rn = np.linalg.norm(r3, axis=-1)
    en = np.linalg.norm(g3 - r3, axis=-1)
    rms_row = np.sqrt((rn ** 2).mean())
    extra = 0.0 if row_extra is None else np.asarray(row_extra, np.float64).reshape(rn.shape)
    row_ratio = en / (GRAD_ROW * rn + GRAD_ROW_FLOOR * rms_row + extra + 1e-300)
    print(f"grad {what}: max_rel {max_rel:.3e} block_max {worst_block:.3e} "
          f"mean {mean_ratio:.3e} fro {fro:.3e} row {row_ratio.max() * GRAD_ROW:.3e}", flush=True)
    assert worst_block <= GRAD_BLOCK_MAX, f"{what}: block max err {worst_block:.3e} of block max"
    assert mean_ratio <= GRAD_MEAN, f"{what}: mean abs err {mean_ratio:.3e} of mean |g*|"
    assert row_ratio.max() <= 1.0, f"{what}: row err {row_ratio.max():.3e} of its bound"
    assert fro <= GRAD_REL_FRO, f"{what}: rel Frobenius err {fro:.3e}"
    return dict(max_rel=max_rel, block_max=worst_block, mean=mean_ratio, fro=fro)


def ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    x = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def mode_sigma(q, k, v, scale, lse):
    """Per-element standard deviation of the difference between two
    computations of O that round each probability P_ij to bf16 independently
    (against different reference maxima) and otherwise agree up to fp32
    rounding: u * sqrt(2/3) * sqrt(sum_j (P_ij V_jd)^2), P = exp(s - LSE),
    with the oracle's LSE.  q [BH, SQ, D], k/v [BH, SKV, D] (float64)."""
    out = np.empty(q.shape, np.float64)
    for h in range(q.shape[0]):
        p = np.exp(scale * (q[h] @ k[h].T) - lse[h][:, None])
        out[h] = np.sqrt((p * p) @ (v[h] * v[h]))
    return U_BF16 * np.sqrt(2.0 / 3.0) * out


def check_modes_agree(o, ref, sigma, what=""):
    """Two bf16 outputs of different merge orders: |o - ref| <= 6 sigma + one
    bf16 ulp of the larger of the two (each side's final rounding is at most
    half an ulp)."""
    o, ref = to64(o), to64(ref)
    bound = 6.0 * sigma + ulp_bf16(np.maximum(np.abs(o), np.abs(ref)))
    ratio = np.abs(o - ref) / bound
    print(f"modes {what}: max err / bound {ratio.max():.3f}", flush=True)
    assert ratio.max() <= 1.0, f"{what}: err {np.abs(o - ref).max():.3e}, ratio {ratio.max():.3f}"


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
