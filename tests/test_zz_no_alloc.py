"""fa_fwd_decode_noalloc: decoding with the partial results in the library's static
per-GPU workspace instead of caller-allocated buffers.  It runs the kernels of
fa_fwd_decode, so on the same inputs and piece count its outputs must equal that
entry point's bit for bit -- on consecutive calls sharing the workspace, the later
one smaller, so that stale partial results of the first call would show.
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


def inputs(seed, B, Hq, Hkv, Nq, Nk, d, dt):
    st = G.Stream(seed)
    x = [st.normals(B * H * n * d).reshape(B, H, n, d) for H, n in ((Hq, Nq), (Hkv, Nk), (Hkv, Nk))]
    x = [G.to_storage(G.round_to_dtype(a, dt), dt) for a in x]
    tens = [torch.from_numpy(a) for a in x]
    tens = [(t.view(torch.bfloat16) if dt == "bf16" else t).cuda() for t in tens]
    return x, tens


def both(q, k, v, causal, S, stream=None):
    """(o, lse) of fa_fwd_decode and of fa_fwd_decode_noalloc on the same inputs."""
    B, Hq, Nq, d = q.shape
    o_ref, l_ref = F.fwd_decode(q, k, v, causal=causal, num_splits=S, stream=stream)
    # Outputs pre-filled with garbage: every element must be written by the call.
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, Nq), 7.0, dtype=torch.float32, device=q.device)
    F.fwd_decode_noalloc(q, k, v, o, lse, causal=causal, num_splits=S, stream=stream)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, lse


# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, num_splits) -- consecutive calls, each
# smaller than the one before it.
SEQUENCE = [
    (8, 32, 8, 1, 8192, 128, "bf16", True, 16),     # grouped-query decoding, 8192-token cache
    (1, 16, 2, 4, 777, 64, "f16", True, 3),         # 8 heads x 4 queries per K/V head, ragged
    (1, 2, 1, 1, 100, 128, "bf16", False, 2),       # tiny
]


def test_two_calls_in_a_row_match_fa_fwd_decode():
    for i, (B, Hq, Hkv, Nq, Nk, d, dt, causal, S) in enumerate(SEQUENCE):
        print(f"noalloc call {i}: B{B} H{Hq}x{Hkv} Nq{Nq} Nk{Nk} d{d} {dt} S{S}", flush=True)
        assert F.decode_noalloc_bytes(B, Hq, Nq, d, S) <= F.NOALLOC_SCRATCH_BYTES
        x, (q, k, v) = inputs(777 + i, B, Hq, Hkv, Nq, Nk, d, dt)
        o_ref, l_ref, o, lse = both(q, k, v, causal, S)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), i
        assert torch.equal(lse, l_ref), i
        if i > 0:
            # and the oracle's tolerance for the later, smaller calls
            q64, k64, v64 = (G.storage_to_f64(a, dt) for a in x)
            sc = float(np.float32(1 / np.sqrt(d)))
            o64, l64 = oracle.attention_kv(q64, k64, v64, causal, sc)
            PT.compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o64, l64,
                       dt, False, f"noalloc call {i}")


def test_largest_workspace_and_one_over():
    # 256 pieces x 15 batches x 8 query heads, d = 128: 15.1 MiB of the 16 MiB.
    B, Hq, Hkv, Nq, Nk, d, S = 15, 8, 1, 1, 256 * 4 * 32, 128, 256
    assert F.decode_noalloc_bytes(B, Hq, Nq, d, S) <= F.NOALLOC_SCRATCH_BYTES
    assert F.decode_noalloc_bytes(B + 1, Hq, Nq, d, S) > F.NOALLOC_SCRATCH_BYTES
    print("noalloc: largest workspace", flush=True)
    _, (q, k, v) = inputs(4242, B, Hq, Hkv, Nq, Nk, d, "bf16")
    o_ref, l_ref, o, lse = both(q, k, v, True, S)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)
    # One batch more does not fit: rejected before any launch, outputs untouched.
    _, (q, k, v) = inputs(4243, B + 1, Hq, Hkv, Nq, 64, d, "bf16")
    o = torch.full_like(q, 3.0)
    with pytest.raises(F.FA355Error) as e:
        F.fwd_decode_noalloc(q, k, v, o, None, causal=True, num_splits=S)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())


def test_side_stream_and_no_lse():
    print("noalloc: side stream, lse NULL", flush=True)
    _, (q, k, v) = inputs(99, 2, 8, 2, 2, 1000, 128, "bf16")
    s = torch.cuda.Stream()
    o_ref, l_ref = F.fwd_decode(q, k, v, causal=True, num_splits=7)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    with torch.cuda.stream(s):
        F.fwd_decode_noalloc(q, k, v, o, None, causal=True, num_splits=7, stream=s)
    s.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
