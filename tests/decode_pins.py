"""Pins of the oracle's queries-against-a-longer-key-sequence path (decoding with a
key/value cache), against things other than itself:

* torch's fp64 ``scaled_dot_product_attention`` with an explicit boolean mask that
  keeps key j for query i iff j <= i + Nk - Nq (a library routine fed the reading
  "the queries are the last Nq positions"), grouped-query heads by ``enable_gqa``,
  and ``torch.logsumexp`` of the masked scores;
* 50-digit decimal brute force on tiny inputs (no max subtraction);
* the suffix property: the last Nq rows of square causal attention over all Nk
  positions equal the cached-decode result for those Nq queries;
* closed forms: one key (O = v_0, lse = scale q.k_0); Nq = Nk reduces to the
  square path exactly.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np
import torch

import oracle
from fa_inputs import Stream


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    assert np.isfinite(a).all() and (err <= tol).all(), f"{what}: max err {err.max()} > {tol}"


def _draw(seed, B, Hq, Hkv, Nq, Nk, d, mult=1.0):
    st = Stream(seed)
    q = st.normals(B * Hq * Nq * d).reshape(B, Hq, Nq, d) * mult
    k = st.normals(B * Hkv * Nk * d).reshape(B, Hkv, Nk, d) * mult
    v = st.normals(B * Hkv * Nk * d).reshape(B, Hkv, Nk, d) * mult
    return q, k, v


CASES = [  # (B, Hq, Hkv, Nq, Nk, d, scale)
    (1, 1, 1, 1, 37, 16, 0.25),
    (2, 4, 1, 3, 64, 32, 0.17),
    (1, 8, 2, 4, 129, 64, -0.11),
    (1, 2, 2, 16, 16, 8, 0.3),
    (2, 6, 3, 5, 300, 16, 0.2),
]


def pin_decode_torch(lib):
    for n, (B, Hq, Hkv, Nq, Nk, d, scale) in enumerate(CASES):
        q, k, v = _draw(5100 + n, B, Hq, Hkv, Nq, Nk, d)
        for causal in (False, True):
            o, lse = oracle.attention_kv(q, k, v, causal, scale, lib=lib)
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nk)[None, :]
            keep = (j <= i + (Nk - Nq)) if causal else torch.ones(Nq, Nk, dtype=torch.bool)
            tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
            ot = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=keep, scale=scale, enable_gqa=Hq != Hkv)
            _close(o, ot.numpy(), 1e-12, f"decode O {(B, Hq, Hkv, Nq, Nk, d)} c={causal}")
            krep = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
            s = scale * torch.matmul(tq, krep.transpose(-1, -2).contiguous())
            s = s.masked_fill(~keep, float("-inf"))
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12,
                   f"decode lse {(B, Hq, Hkv, Nq, Nk, d)} c={causal}")


def pin_decode_brute_force(lib):
    B, Hq, Hkv, Nq, Nk, d, scale = 1, 2, 1, 3, 7, 4, 0.6
    q, k, v = _draw(5200, B, Hq, Hkv, Nq, Nk, d)
    o, lse = oracle.attention_kv(q, k, v, True, scale, lib=lib)
    with localcontext() as ctx:
        ctx.prec = 50
        for h in range(Hq):
            for i in range(Nq):
                js = range(i + Nk - Nq + 1)
                e = [(Decimal(scale) * sum(Decimal(q[0, h, i, t]) * Decimal(k[0, 0, j, t])
                                           for t in range(d))).exp() for j in js]
                den = sum(e)
                for t in range(d):
                    num = sum(e[a] * Decimal(v[0, 0, j, t]) for a, j in enumerate(js))
                    assert abs(float(num / den) - o[0, h, i, t]) <= 1e-13, (h, i, t)
                assert abs(float(den.ln()) - lse[0, h, i]) <= 1e-13, (h, i)


def pin_decode_suffix(lib):
    # Square causal attention over all Nk positions, rows Nk - Nq .. Nk - 1, is the
    # cached decode of those Nq queries.
    B, Hq, Hkv, Nk, Nq, d, scale = 1, 4, 2, 90, 6, 32, 0.18
    qf, k, v = _draw(5300, B, Hq, Hkv, Nk, Nk, d)
    o_sq, l_sq = oracle.attention(qf, k, v, True, scale, lib=lib)
    o, lse = oracle.attention_kv(np.ascontiguousarray(qf[:, :, Nk - Nq:]), k, v, True, scale, lib=lib)
    _close(o, o_sq[:, :, Nk - Nq:], 1e-13, "suffix O")
    _close(lse, l_sq[:, :, Nk - Nq:], 1e-13, "suffix lse")


def pin_decode_closed_forms(lib):
    q, k, v = _draw(5400, 1, 3, 1, 2, 1, 16)
    for causal in (False, True):
        if causal:
            q1 = np.ascontiguousarray(q[:, :, :1])
            o, lse = oracle.attention_kv(q1, k, v, True, 0.5, lib=lib)
            qq = q1
        else:
            o, lse = oracle.attention_kv(q, k, v, False, 0.5, lib=lib)
            qq = q
        _close(o, np.broadcast_to(v, o.shape), 1e-15, "one key: O = v0")
        _close(lse, 0.5 * (qq * k).sum(-1), 1e-13, "one key: lse = scale q.k0")
    # Nq = Nk is the square path.
    q, k, v = _draw(5401, 2, 4, 2, 33, 33, 16)
    for causal in (False, True):
        a = oracle.attention_kv(q, k, v, causal, 0.25, lib=lib)
        b = oracle.attention(q, k, v, causal, 0.25, lib=lib)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # More queries than keys is allowed without a causal mask, not with one.
    q, k, v = _draw(5402, 1, 1, 1, 5, 3, 8)
    oracle.attention_kv(q, k, v, False, 0.3, lib=lib)
    try:
        oracle.attention_kv(q, k, v, True, 0.3, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("causal with Nq > Nk must be rejected")


def all_decode_pins(lib):
    pin_decode_torch(lib)
    pin_decode_brute_force(lib)
    pin_decode_suffix(lib)
    pin_decode_closed_forms(lib)
