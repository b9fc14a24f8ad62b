"""The LDS-poison debug library against the normal one, bit for bit.

libfa355_lds_poison.so is built from the same sources with FA355_LDS_POISON=1:
before each LDS stage is refilled, every byte of it is set to 0xff (a NaN as bf16,
fp16, fp32 and e4m3), and each refill has landed before the block in the other
stage is computed.  So:

  * a kernel that read LDS bytes no copy wrote (a padding slot, a row past N that
    the copy skipped instead of zeroing, a stage read before its copy landed) would
    produce NaN, or at least different bits, in the debug build;
  * a race between a copy and the reads of the stage it overwrites would show as a
    difference, since the debug build cannot overlap them.

Every entry point that stages through LDS is run on ragged shapes (N not a
multiple of any tile), through every built tiling of the forward pass, and the two
libraries' outputs are compared with torch.equal.
"""
import os

import numpy as np
import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F
from io_aware_attention_amd import fa355 as FB
import parity as PT

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not os.path.exists(FB.LDS_POISON_LIB_PATH),
                       reason="debug library not built (python -m io_aware_attention_amd.build --lds-poison)"),
]


def both(call):
    """call() under the normal library, then under the debug one; returns both results."""
    a = call()
    torch.cuda.synchronize()
    with F.use_library(FB.LDS_POISON_LIB_PATH):
        b = call()
        torch.cuda.synchronize()
    return a, b


def assert_same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        if x is None:
            assert y is None
            continue
        assert torch.isfinite(x.float()).all(), f"{what}: normal library, output {i}"
        assert torch.isfinite(y.float()).all(), f"{what}: debug library, output {i} not finite"
        assert torch.equal(x, y), f"{what}: output {i} differs, max |diff| " \
            f"{(x.float() - y.float()).abs().nan_to_num(float('inf')).max().item()}"


FWD = [
    # (B, Hq, Hkv, N, d, dtype, causal, tilings)
    (1, 4, 2, 300, 128, "bf16", True, [None, (128, 32), (64, 64), (256, 64), (128, 64)]),
    (2, 3, 3, 77, 64, "f16", False, [None, (128, 32), (64, 64), (256, 64)]),
    (1, 2, 1, 200, 256, "bf16", True, [None, (128, 64)]),
    (1, 2, 2, 300, 256, "f16", False, [None, (128, 64)]),
    (1, 2, 2, 129, 256, "f16", False, [None]),
    (1, 2, 2, 100, 64, "f32", True, [None, (32, 32), (64, 32), (128, 32)]),
    (1, 1, 1, 1, 128, "bf16", True, [None]),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dt,causal,tilings", FWD)
def test_forward(B, Hq, Hkv, N, d, dt, causal, tilings):
    x = G.make_inputs(9900 + N + d, B, Hq, Hkv, N, d, dt, causal)
    q, k, v = PT.to_device(x)
    for t in tilings:
        a, b = both(lambda: F.fwd(q, k, v, causal=causal, scale=x.scale, tuning=t))
        assert_same(a, b, f"fwd {dt} d{d} N{N} tile {t}")
    if dt != "f32":
        a, b = both(lambda: F.fwd(q, k, v, causal=causal, scale=x.scale, out_dtype=torch.float32))
        assert_same(a, b, f"fwd {dt} d{d} N{N} fp32 out")


def test_split():
    x = G.make_inputs(9911, 1, 4, 2, 500, 128, "bf16", True)
    q, k, v = PT.to_device(x)
    for s in (1, 3, 7):
        a, b = both(lambda: F.fwd_split(q, k, v, causal=True, scale=x.scale, num_splits=s))
        assert_same(a, b, f"split {s}")


def test_bias():
    x = G.make_inputs(9912, 2, 2, 1, 130, 64, "bf16", True)
    q, k, v = PT.to_device(x)
    bias = torch.from_numpy(G.make_normal(9913, (1, 2, 130, 130), "bf16", mult=2.0)).view(torch.bfloat16).cuda()
    a, b = both(lambda: F.fwd_bias(q, k, v, bias, causal=True, scale=x.scale))
    assert_same(a, b, "bias")


def test_fp8():
    x = G.make_inputs(9914, 1, 4, 2, 200, 128, "e4m3", True)
    q, k, v = PT.to_device(x)
    a, b = both(lambda: F.fwd_fp8(q, k, v, *x.descale, causal=True, scale=x.scale))
    assert_same(a, b, "fp8")


@pytest.mark.parametrize("causal", [True, False])
def test_decode(causal):
    x = G.make_decode_inputs(seed=9915, B=2, Hq=8, Hkv=2, Nq=3, Nk=1001, d=128, dtype="bf16",
                             causal=causal, recipe="lds poison test")
    q, k, v = (torch.from_numpy(getattr(x, n)).view(torch.bfloat16).cuda() for n in "qkv")
    for s in (1, 4):
        a, b = both(lambda: F.fwd_decode(q, k, v, causal=causal, scale=x.scale, num_splits=s))
        assert_same(a, b, f"decode causal={causal} splits {s}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dt,causal", [
    (1, 4, 2, 300, 128, "bf16", True),
    (2, 2, 2, 77, 64, "f16", False),
    (1, 2, 1, 150, 256, "bf16", True),
])
def test_backward(B, Hq, Hkv, N, d, dt, causal):
    x = G.make_inputs(9920 + N, B, Hq, Hkv, N, d, dt, causal)
    q, k, v = PT.to_device(x)
    g = torch.from_numpy(G.make_grad_output(9930 + N, (B, Hq, N, d), dt))
    g = (g.view(torch.bfloat16) if dt == "bf16" else g).cuda()
    o, lse = F.fwd(q, k, v, causal=causal, scale=x.scale)
    a, b = both(lambda: F.bwd(q, k, v, o, g, lse, causal=causal, scale=x.scale))
    assert_same(a, b, f"bwd {dt} d{d} N{N}")
    assert np.isfinite(a[0].cpu().numpy()).all()
