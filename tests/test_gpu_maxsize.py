"""The largest sizes the C ABI accepts, checked through properties with a closed form.

A head's K, V (and Q, O) must fit 32-bit byte offsets: N d 2 <= INT_MAX - 65536 for
16-bit inputs, i.e. N <= 8,388,351 at d = 128 and 4,194,175 at d = 256 (the
kernel split by role), each with a ragged last tile.  Inputs
of that size are built on the device, and the expected result comes from integer
counting rather than from the oracle:

  * Q = e_0 (every row), K = 0 except rows j = 0 mod 1024 where K[j, 0] = 32, and
    scale = 1: a score is 32 for those "marked" keys and 0 for the rest;
  * V[j, c] = bit (c mod 24) of j: every row of V is distinct over its columns, so
    reading a wrong K or V row anywhere changes the result.

For a query that sees keys 0 .. m-1 (m = i + 1 under the causal mask), with
M = ceil(m / 1024) marked keys, U = m - M unmarked and E = e^32,
    O[c] = (E * cm_b + (call_b - cm_b)) / (E * M + U),   lse = log(E * M + U),
where b = c mod 24, call_b counts the j < m with bit b set and cm_b the marked ones
(j = 1024 k, k < M: bit b of j is bit b - 10 of k).  This is the definition of
softmax attention evaluated exactly for these inputs.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_attention_amd as F
import parity as PT

pytestmark = pytest.mark.gpu

D = 128
N_MAX = (2**31 - 1 - 65536) // (D * 2)          # 8,388,351
MARK = 1024
A = 32.0


def count_bit(m: np.ndarray, b: int) -> np.ndarray:
    """Number of j in [0, m) with bit b set (m: int64 array)."""
    period = 1 << (b + 1)
    return (m // period) * (1 << b) + np.maximum(0, (m % period) - (1 << b))


def expected(m: np.ndarray, d: int = D):
    """O [len(m), d] and lse [len(m)] for queries that see keys 0 .. m-1."""
    M = (m + MARK - 1) // MARK
    U = m - M
    E = math.exp(A)
    o = np.empty((len(m), d))
    for c in range(d):
        b = c % 24
        call = count_bit(m, b).astype(np.float64)
        cm = count_bit(M, b - 10).astype(np.float64) if b >= 10 else np.zeros(len(m))
        o[:, c] = (E * cm + (call - cm)) / (E * M + U)
    lse = A + np.log(M + U * math.exp(-A))
    return o, lse


def build(n: int, heads: int, dev="cuda", d: int = D):
    bf = dict(dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, heads, n, d, **bf)
    k[:, :, ::MARK, 0] = A
    j = torch.arange(n, dtype=torch.int32, device=dev)
    bits = (torch.arange(d, dtype=torch.int32, device=dev) % 24)
    v = torch.empty(1, heads, n, d, **bf)
    step = 1 << 20
    for s in range(0, n, step):                 # chunks keep the int32 temporary small
        v[0, :, s:s + step] = ((j[s:s + step, None] >> bits[None, :]) & 1).to(torch.bfloat16)
    return k, v


@pytest.mark.parametrize("d", [128, 256])
def test_forward_at_largest_n(d):
    dev = "cuda"
    n_max = (2**31 - 1 - 65536) // (d * 2)
    k, v = build(n_max, 1, d=d)
    q = torch.zeros(1, 1, n_max, d, dtype=torch.bfloat16, device=dev)
    q[..., 0] = 1.0
    o, lse = F.fwd(q, k, v, causal=True, scale=1.0)
    torch.cuda.synchronize()
    del q, k, v
    rows = PT.sample_rows(n_max, 256 if d == 128 else 128, 9973)
    ri = torch.from_numpy(rows).to(dev)
    og = o[0, 0].index_select(0, ri).float().cpu().double().numpy()
    lg = lse[0, 0].index_select(0, ri).cpu().double().numpy()
    o_ref, l_ref = expected(rows + 1, d)
    stats = PT.compare(og, lg, o_ref, l_ref, "bf16", False, f"N={n_max} d={d} causal, {len(rows)} rows")
    print(f"N={n_max} d={d}: {len(rows)} rows, {stats}", flush=True)


def test_decode_at_largest_cache():
    # The decode kernel reads one block past the end: Nk + 32 rows must fit.
    dev = "cuda"
    nk = (2**31 - 1 - 65536) // (D * 2) - 32
    k, v = build(nk, 2)
    q = torch.zeros(1, 8, 2, D, dtype=torch.bfloat16, device=dev)
    q[..., 0] = 1.0
    o, lse = F.fwd_decode(q, k, v, causal=True, scale=1.0)
    torch.cuda.synchronize()
    # Query i of the two sees keys j <= i + nk - 2, i.e. m = nk - 1 + i of them.
    o_ref, l_ref = expected(np.array([nk - 1, nk], dtype=np.int64))
    og = o[0].float().cpu().double().numpy()          # [8 heads, 2, D]
    lg = lse[0].cpu().double().numpy()
    for h in range(8):
        PT.compare(og[h], lg[h], o_ref, l_ref, "bf16", False, f"decode Nk={nk} head {h}")
