"""GPU parity of the split-KV forward pass (fa_fwd_split) against the fp64 oracle.

Split-KV computes the same function as the forward pass -- the merge of partial
results over disjoint key ranges is exact up to rounding -- so it is held to the
forward pass's tolerance (max abs O error 2e-2 plus half an ulp of the output
type, lse 1e-3), against the same oracle.
"""
import numpy as np
import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F
import oracle
import parity as PT

pytestmark = pytest.mark.gpu


def run_split(x, num_splits):
    q, k, v = PT.to_device(x)
    o, lse = F.fwd_split(q, k, v, causal=x.causal, scale=x.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


# (B, Hq, Hkv, N, d, dtype, causal, mult, num_splits)
CASES = [
    (1, 2, 2, 1000, 128, "bf16", True, 1.0, 4),
    (1, 2, 2, 1000, 128, "bf16", False, 1.0, 3),
    (1, 4, 1, 777, 64, "f16", True, 1.0, 7),
    (2, 4, 2, 333, 128, "f16", False, 2.0, 2),
    (1, 2, 2, 64, 128, "bf16", True, 1.0, 16),      # more splits than key blocks
    (1, 1, 1, 1, 64, "bf16", True, 1.0, 5),         # one row, one key
    (1, 2, 2, 2048, 128, "bf16", True, 3.0, 8),     # large scores: rescales inside splits
    (1, 3, 3, 129, 64, "bf16", False, 1.0, 1),
]


def _id(c):
    B, Hq, Hkv, N, d, dt, causal, mult, S = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-N{N}-d{d}-{'causal' if causal else 'full'}-S{S}" + \
        (f"-x{mult:g}" if mult != 1 else "")


@pytest.mark.parametrize("cfg", CASES, ids=[_id(c) for c in CASES])
def test_split_parity(cfg):
    B, Hq, Hkv, N, d, dt, causal, mult, S = cfg
    x = G.make_inputs(9900 + N + d + S, B, Hq, Hkv, N, d, dt, causal, mult=mult)
    o_ref, l_ref = oracle.attention(x.f64("q"), x.f64("k"), x.f64("v"), causal, x.scale)
    o, l = run_split(x, S)
    PT.compare(o, l, o_ref, l_ref, dt, False, _id(cfg))


def test_split_matches_unsplit_within_rounding():
    # One split is the forward pass (same 256 x 64 tiles at head dim 128) with an
    # extra fp32 round trip through the workspace: the two outputs differ at most
    # by the output rounding.
    x = G.make_inputs(9950, 1, 4, 4, 600, 128, "bf16", True)
    q, k, v = PT.to_device(x)
    o1, l1 = F.fwd_split(q, k, v, causal=True, scale=x.scale, num_splits=1)
    o0, l0 = F.fwd(q, k, v, causal=True, scale=x.scale, tuning=(256, 64))
    torch.cuda.synchronize()
    a, b = o0.float().cpu().double().numpy(), o1.float().cpu().double().numpy()
    assert np.abs(a - b).max() <= PT.half_ulp(a, "bf16").max() * 2
    assert torch.allclose(l0, l1, atol=1e-6, rtol=0)


def test_split_rejects_bad_counts():
    x = G.make_inputs(9951, 1, 1, 1, 64, 64, "bf16", False)
    q, k, v = PT.to_device(x)
    for S in (0, 17):
        with pytest.raises(F.FA355Error):
            F.fwd_split(q, k, v, num_splits=S)
