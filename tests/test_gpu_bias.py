"""GPU parity of the additive-bias forward pass (fa_fwd_bias) against the fp64
oracle's bias path.

The bias values are 16-bit inputs read exactly by both sides; the kernel adds
them to the fp32 scaled scores (log2 units), so the forward tolerance applies
unchanged: max abs O error 2e-2 plus half an ulp of the output type, lse 1e-3.
Rows whose every score is -inf must come out exactly O = 0, lse = -inf.
"""
import numpy as np
import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F
import oracle
import parity as PT

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16}


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if dt == "bf16" else t).cuda()


def make_bias(seed, shape, dt, kind):
    Bb, Hb, N, _ = shape
    if kind == "random":
        st = G.make_normal(seed, shape, dt, mult=2.0)
    elif kind == "alibi":                       # per-head slope times key - query distance
        slopes = 2.0 ** (-8.0 * (np.arange(Hb) + 1) / Hb)
        dist = np.arange(N)[None, :] - np.arange(N)[:, None]
        st = G.to_storage(G.round_to_dtype(slopes[None, :, None, None] * dist[None, None], dt), dt)
        st = np.broadcast_to(st, shape).copy()
    elif kind == "mask":                        # random -inf mask, key 0 always visible
        rng = np.random.default_rng(seed)
        b = np.where(rng.random(shape) < 0.3, -np.inf, 0.0)
        b[..., 0] = 0.0
        st = G.to_storage(b, dt)
    else:
        raise ValueError(kind)
    return st


def check(x, bias_st, o, lse, what):
    b64 = G.storage_to_f64(bias_st, x.dtype)
    o_ref, l_ref = oracle.attention_bias(x.f64("q"), x.f64("k"), x.f64("v"), b64, x.causal, x.scale)
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert (o[dead] == 0).all(), what
    live = ~dead
    PT.compare(o[live], lse[live], o_ref[live], l_ref[live], x.dtype, False, what)


def run(x, bias_st, padded_row=None):
    q, k, v = PT.to_device(x)
    b = _dev(bias_st, x.dtype)
    if padded_row is not None:                   # a row stride larger than N
        N = x.N
        wide = torch.zeros(b.shape[:2] + (N, padded_row), dtype=b.dtype, device=b.device)
        wide[..., :N] = b
        b = wide[..., :N]
    o, lse = F.fwd_bias(q, k, v, b, causal=x.causal, scale=x.scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


# (B, Hq, Hkv, N, d, dtype, causal, bias shape kind: "full" | "shared" | "head", kind)
CASES = [
    (1, 2, 2, 300, 128, "bf16", False, "full", "random"),
    (2, 4, 2, 257, 128, "bf16", True, "full", "random"),
    (1, 4, 1, 200, 64, "f16", False, "head", "alibi"),
    (2, 2, 2, 333, 64, "bf16", False, "shared", "mask"),
    (1, 2, 2, 129, 128, "f16", True, "full", "mask"),
    (1, 8, 8, 1024, 128, "bf16", True, "head", "alibi"),
]


def _id(c):
    B, Hq, Hkv, N, d, dt, causal, shp, kind = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-N{N}-d{d}-{'causal' if causal else 'full'}-{shp}-{kind}"


@pytest.mark.parametrize("cfg", CASES, ids=[_id(c) for c in CASES])
def test_bias_parity(cfg):
    B, Hq, Hkv, N, d, dt, causal, shp, kind = cfg
    x = G.make_inputs(9960 + N + d, B, Hq, Hkv, N, d, dt, causal)
    shape = {"full": (B, Hq, N, N), "shared": (1, 1, N, N), "head": (1, Hq, N, N)}[shp]
    bias = make_bias(9961 + N, shape, dt, kind)
    o, lse = run(x, bias)
    check(x, bias, o, lse, _id(cfg))


def test_bias_padded_rows_and_dead_rows():
    x = G.make_inputs(9970, 1, 2, 2, 100, 64, "bf16", False)
    bias = make_bias(9971, (1, 2, 100, 100), "bf16", "random")
    b64 = G.storage_to_f64(bias, "bf16")
    b64[0, 1, 37, :] = -np.inf                  # one row with no finite score
    b64[0, 0, 5, 1:] = -np.inf                  # one row that sees only key 0
    bias = G.to_storage(b64, "bf16")
    o, lse = run(x, bias, padded_row=104)
    check(x, bias, o, lse, "padded rows / dead rows")


def test_bias_zero_matches_plain_forward():
    x = G.make_inputs(9972, 1, 4, 4, 500, 128, "bf16", True)
    q, k, v = PT.to_device(x)
    zero = torch.zeros((1, 1, 500, 500), dtype=torch.bfloat16, device="cuda")
    o1, l1 = F.fwd_bias(q, k, v, zero, causal=True, scale=x.scale)
    o0, l0 = F.fwd(q, k, v, causal=True, scale=x.scale, tuning=(128, 32))
    torch.cuda.synchronize()
    a, b = o0.float().cpu().double().numpy(), o1.float().cpu().double().numpy()
    assert np.abs(a - b).max() <= 2 * PT.half_ulp(a, "bf16").max()
    assert (l0 - l1).abs().max().item() <= 1e-5
