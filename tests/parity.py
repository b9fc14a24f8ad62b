"""Helpers shared by the GPU parity tests, smoke() and the benchmark.

Tolerances (max abs error of O against the fp64 oracle; lse always <= 1e-3):
  * fp32 inputs: 1e-5;
  * fp16/bf16 inputs, fp32 output: 2e-2;
  * fp16/bf16 inputs and output: 2e-2 plus half a unit in the last place of the
    exact value in the output type -- the rounding any 16-bit store must add.
"""
from __future__ import annotations

import numpy as np

import oracle
from fa_inputs import AttentionInputs

LSE_TOL = 1e-3
_PREC = {"bf16": (8, -126), "f16": (11, -14)}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of `dtype` at each |x| (the bound of one RNE store)."""
    p, emin = _PREC[dtype]
    _, e = np.frexp(np.abs(x))
    e = np.where(x == 0, emin, np.maximum(e.astype(np.int64) - 1, emin))  # exponent of |x|
    return np.ldexp(0.5, e - (p - 1))


def o_bound(ref: np.ndarray, in_dtype: str, out_f32: bool) -> np.ndarray:
    if in_dtype in ("f32", "f64"):
        return np.full(ref.shape, 1e-5)
    if out_f32:
        return np.full(ref.shape, 2e-2)
    return 2e-2 + half_ulp(ref, in_dtype)


def to_device(x: AttentionInputs, device="cuda"):
    import torch
    out = []
    for name in ("q", "k", "v"):
        a = getattr(x, name)
        if x.dtype == "bf16":
            t = torch.from_numpy(a).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out.append(t.to(device))
    return out


def sample_rows(N: int, br: int, every: int) -> np.ndarray:
    """Rows 0..br+1, every query-tile boundary +-1, every `every`-th row, the last."""
    rows = set(range(min(N, br + 2)))
    for b0 in range(0, N, br):
        rows.update(r for r in (b0 - 1, b0, b0 + 1) if 0 <= r < N)
    rows.update(range(0, N, every))
    rows.add(N - 1)
    return np.array(sorted(rows), dtype=np.int64)


def oracle_heads(x: AttentionInputs, heads, rows=None, threads=0):
    """Oracle O and lse for the listed (b, h) query heads (rows optional).

    Returns o [len(heads), R, d] and lse [len(heads), R].
    """
    G = x.Hq // x.Hkv
    outs, lses = [], []
    for b, h in heads:
        q = _slice64(x, "q", b, h)
        k = _slice64(x, "k", b, h // G)
        v = _slice64(x, "v", b, h // G)
        o, lse = oracle.attention(q, k, v, x.causal, x.scale, rows=rows, threads=threads)
        outs.append(o[0, 0])
        lses.append(lse[0, 0])
    return np.stack(outs), np.stack(lses)


def _slice64(x: AttentionInputs, name: str, b: int, h: int) -> np.ndarray:
    from fa_inputs import storage_to_f64
    a = getattr(x, name)[b:b + 1, h:h + 1]
    v = storage_to_f64(np.ascontiguousarray(a), x.dtype)
    if x.descale is not None:
        v *= x.descale["qkv".index(name)]
    return v


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
            in_dtype: str, out_f32: bool, what: str = "") -> dict:
    """Check one comparison against the tolerance rules; returns error statistics."""
    o_gpu = np.asarray(o_gpu, np.float64)
    err = np.abs(o_gpu - o_ref)
    bound = o_bound(o_ref, in_dtype, out_f32)
    lerr = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
    stats = {"max_abs_o": float(err.max()), "max_abs_lse": float(lerr.max()),
             "worst_ratio": float((err / bound).max())}
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    assert (err <= bound).all(), f"{what}: O error {stats['max_abs_o']:.3g} exceeds bound " \
                                 f"(worst err/bound {stats['worst_ratio']:.3g})"
    assert (lerr <= LSE_TOL).all(), f"{what}: lse error {stats['max_abs_lse']:.3g} > {LSE_TOL}"
    return stats
