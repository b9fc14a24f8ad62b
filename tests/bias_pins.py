"""Pins of the oracle's additive-bias path against things other than itself.

* a zero bias, and a -inf bias above the diagonal without causal masking, give
  exactly what the plain (resp. causal) path gives;
* a bias constant along each row changes nothing in O (softmax is shift
  invariant) and moves lse by that constant;
* torch: softmax(scale Q K^T + bias) V in fp64 with matmul / softmax;
* broadcasting: a [1,1,N,N] bias equals the same bias repeated to [B,Hq,N,N];
* a row whose every score is -inf attends to nothing: O = 0, lse = -inf.
"""
from __future__ import annotations

import numpy as np

import oracle


def _draw(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)), rng)


def pin_bias_reductions(lib):
    q, k, v, rng = _draw(7400, 2, 4, 2, 9, 5)
    o0, l0 = oracle.attention(q, k, v, False, 0.7, lib=lib)
    o1, l1 = oracle.attention_bias(q, k, v, np.zeros((1, 1, 9, 9)), False, 0.7, lib=lib)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    tri = np.where(np.tril(np.ones((9, 9), bool)), 0.0, -np.inf)[None, None]
    oc, lc = oracle.attention(q, k, v, True, 0.7, lib=lib)
    ob, lb = oracle.attention_bias(q, k, v, tri, False, 0.7, lib=lib)
    assert np.array_equal(oc, ob) and np.array_equal(lc, lb)


def pin_bias_row_shift(lib):
    q, k, v, rng = _draw(7401, 1, 2, 2, 7, 4)
    c = rng.standard_normal((1, 2, 7, 1)) * 3
    o0, l0 = oracle.attention(q, k, v, True, 0.5, lib=lib)
    o1, l1 = oracle.attention_bias(q, k, v, np.broadcast_to(c, (1, 2, 7, 7)), True, 0.5, lib=lib)
    assert np.abs(o1 - o0).max() <= 1e-13 and np.abs(l1 - (l0 + c[..., 0])).max() <= 1e-13


def pin_bias_torch(lib):
    import torch
    for seed, (B, Hq, Hkv, N, d, causal, scale) in enumerate(
            [(2, 4, 2, 8, 5, False, 0.9), (1, 3, 1, 11, 6, True, -0.4)]):
        q, k, v, rng = _draw(7410 + seed, B, Hq, Hkv, N, d)
        bias = rng.standard_normal((B, Hq, N, N)) * 2
        bias[rng.random(bias.shape) < 0.2] = -np.inf
        bias[..., 0] = 0.0                     # every row keeps key 0 visible
        o, lse = oracle.attention_bias(q, k, v, bias, causal, scale, lib=lib)
        G = Hq // Hkv
        tq, tk, tv, tb = (torch.tensor(a) for a in (q, k, v, bias))
        kk, vv = tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1)
        s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous()) + tb
        if causal:
            s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
        ref = torch.matmul(torch.softmax(s, -1), vv).numpy()
        assert np.abs(o - ref).max() <= 1e-12, seed
        assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() <= 1e-12, seed


def pin_bias_broadcast_and_empty_rows(lib):
    q, k, v, rng = _draw(7420, 2, 2, 2, 6, 3)
    b1 = rng.standard_normal((1, 1, 6, 6))
    o1, l1 = oracle.attention_bias(q, k, v, b1, False, 1.1, lib=lib)
    o2, l2 = oracle.attention_bias(q, k, v, np.repeat(np.repeat(b1, 2, 0), 2, 1), False, 1.1, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    bh = rng.standard_normal((1, 2, 6, 6))
    oh, lh = oracle.attention_bias(q, k, v, bh, False, 1.1, lib=lib)
    oh2, lh2 = oracle.attention_bias(q, k, v, np.repeat(bh, 2, 0), False, 1.1, lib=lib)
    assert np.array_equal(oh, oh2) and np.array_equal(lh, lh2)
    dead = np.zeros((1, 1, 6, 6))
    dead[0, 0, 3, :] = -np.inf
    o, l = oracle.attention_bias(q, k, v, dead, False, 1.1, lib=lib)
    assert np.array_equal(o[:, :, 3], np.zeros_like(o[:, :, 3])) and np.all(l[:, :, 3] == -np.inf)
    assert np.isfinite(o).all() and np.isfinite(np.delete(l, 3, axis=2)).all()


def all_bias_pins(lib):
    pin_bias_reductions(lib)
    pin_bias_row_shift(lib)
    pin_bias_torch(lib)
    pin_bias_broadcast_and_empty_rows(lib)
