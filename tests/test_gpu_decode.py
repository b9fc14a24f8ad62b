"""GPU parity of decoding against a key/value cache (fa_fwd_decode) with the fp64
oracle's queries-against-a-longer-sequence path.

The decode kernel does the arithmetic of the forward kernel (16-bit weights as
matrix operands, fp32 accumulation, an exact merge of key-range pieces), so it is
held to the forward pass's tolerance: max abs O error 2e-2 plus half an ulp of the
output type, lse 1e-3.
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


def draw(seed, B, Hq, Hkv, Nq, Nk, d, dt, mult=1.0):
    st = G.Stream(seed)
    x = [st.normals(B * H * n * d).reshape(B, H, n, d) * mult
         for H, n in ((Hq, Nq), (Hkv, Nk), (Hkv, Nk))]
    return [G.to_storage(G.round_to_dtype(a, dt), dt) for a in x]


def dev(a, dt):
    t = torch.from_numpy(a)
    return (t.view(torch.bfloat16) if dt == "bf16" else t).cuda()


def run(st, dt, causal, scale, S):
    q, k, v = (dev(a, dt) for a in st)
    o, lse = F.fwd_decode(q, k, v, causal=causal, scale=scale, num_splits=S)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, num_splits (None = default), mult, scale)
CASES = [
    (1, 32, 8, 1, 4096, 128, "bf16", True, None, 1.0, None),     # 4 heads x 1 query per group
    (2, 8, 8, 1, 1000, 128, "bf16", True, 7, 1.0, None),         # MHA, ragged cache
    (1, 16, 2, 4, 777, 64, "f16", True, 16, 1.0, None),          # 8 heads x 4 queries = 32 rows
    (1, 4, 1, 8, 300, 128, "bf16", True, 3, 1.0, None),          # 4 x 8 = 32 rows
    (2, 6, 3, 5, 129, 64, "f16", False, 2, 1.0, None),           # non-causal
    (1, 2, 1, 3, 3, 128, "bf16", True, 1, 1.0, None),            # Nq = Nk
    (1, 8, 2, 2, 65, 128, "bf16", True, 4, 2.0, -0.1),           # negative scale
    (1, 4, 4, 1, 1, 64, "bf16", True, 1, 1.0, None),             # one key
    (1, 8, 1, 2, 2048, 128, "bf16", True, 8, 3.0, None),         # large scores: rescales
    (1, 2, 1, 1, 100, 128, "bf16", True, 50, 1.0, None),         # more pieces than blocks
    (1, 8, 2, 3, 5, 64, "f16", False, 2, 1.0, None),             # Nq close to Nk
]


def _id(c):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, S, mult, scale = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-Nq{Nq}-Nk{Nk}-d{d}-{'causal' if causal else 'full'}-S{S}" + \
        (f"-x{mult:g}" if mult != 1 else "") + (f"-s{scale:g}" if scale is not None else "")


@pytest.mark.parametrize("cfg", CASES, ids=[_id(c) for c in CASES])
def test_decode_parity(cfg):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, S, mult, scale = cfg
    sc = float(np.float32(1 / np.sqrt(d) if scale is None else scale))
    st = draw(9990 + Nk + Nq, B, Hq, Hkv, Nq, Nk, d, dt, mult)
    q, k, v = (G.storage_to_f64(a, dt) for a in st)
    o_ref, l_ref = oracle.attention_kv(q, k, v, causal, sc)
    o, l = run(st, dt, causal, sc, S)
    PT.compare(o, l, o_ref, l_ref, dt, False, _id(cfg))


def test_decode_full_size():
    # Llama-7B-class grouped-query decoding: B8, 32 query / 8 K/V heads, one new
    # token against an 8192-token cache, in the launch the benchmark times.
    B, Hq, Hkv, Nq, Nk, d = 8, 32, 8, 1, 8192, 128
    st = draw(4321, B, Hq, Hkv, Nq, Nk, d, "bf16")
    o, l = run(st, "bf16", True, float(np.float32(1 / np.sqrt(d))), None)
    q, k, v = (G.storage_to_f64(a, "bf16") for a in st)
    for b in (0, 5):
        o_ref, l_ref = oracle.attention_kv(q[b:b + 1], k[b:b + 1], v[b:b + 1], True,
                                           float(np.float32(1 / np.sqrt(d))))
        PT.compare(o[b:b + 1], l[b:b + 1], o_ref, l_ref, "bf16", False, f"decode full b={b}")


def test_decode_deterministic_and_split_invariant():
    st = draw(4322, 1, 16, 4, 2, 3000, 128, "bf16")
    a = run(st, "bf16", True, 0.088, 12)
    b = run(st, "bf16", True, 0.088, 12)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = run(st, "bf16", True, 0.088, 1)
    # Different piece counts merge different fp32 partials: equal to rounding.
    assert np.abs(a[0] - c[0]).max() <= 2 * PT.half_ulp(c[0], "bf16").max()
    assert np.abs(a[1] - c[1]).max() <= 1e-5
