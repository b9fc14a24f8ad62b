"""Pins of the gradient oracle against things other than itself.

Each pin takes an oracle library handle (the real one, or a planted-mistake copy
in test_oracle_mutants.py) and raises AssertionError on disagreement:

* central finite differences of the forward oracle's loss sum(O * dO), in fp64
  (the forward oracle is itself pinned by oracle_pins.py);
* torch autograd through a plain fp64 attention written with matmul / softmax;
* exact identities of the gradient: the softmax Jacobian annihilates constants,
  so every row of dS sums to zero and sum_j dK_j = 0; sum_j P_ij = 1, so
  sum_j dV_j = sum_i dO_i over the query heads of a key/value head; constant V
  rows leave nothing for Q and K to change;
* closed forms: one key (N = 1), and causal row 0, where O_0 = V_0.
"""
from __future__ import annotations

import numpy as np

import oracle

# (B, Hq, Hkv, N, d, causal, scale)
SHAPES = [
    (1, 1, 1, 6, 4, False, 0.5),
    (1, 2, 1, 7, 3, True, 0.9),
    (2, 4, 2, 5, 8, True, -0.3),
    (1, 3, 3, 9, 5, False, 1.3),
]


def _draw(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    g = rng.standard_normal((B, Hq, N, d))
    return q, k, v, g


def pin_grad_finite_differences(lib, quick=False):
    shapes = SHAPES[:2] if quick else SHAPES
    eps = 1e-6
    for n, (B, Hq, Hkv, N, d, causal, scale) in enumerate(shapes):
        q, k, v, g = _draw(7000 + n, B, Hq, Hkv, N, d)
        dq, dk, dv = oracle.grads(q, k, v, g, causal, scale, lib=lib)

        def loss(q_, k_, v_):
            o, _ = oracle.attention(q_, k_, v_, causal, scale, lib=lib)
            return float((o * g).sum())

        for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                           loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            err = np.abs(fd - gr).max()
            assert err <= 1e-6 * max(1.0, np.abs(fd).max()), (name, n, err)


def pin_grad_autograd(lib):
    import torch
    for n, (B, Hq, Hkv, N, d, causal, scale) in enumerate(SHAPES):
        q, k, v, g = _draw(7100 + n, B, Hq, Hkv, N, d)
        dq, dk, dv = oracle.grads(q, k, v, g, causal, scale, lib=lib)
        G = Hq // Hkv
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        kk = tk.repeat_interleave(G, dim=1)
        vv = tv.repeat_interleave(G, dim=1)
        s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
        if causal:
            mask = torch.ones(N, N, dtype=torch.bool).tril()
            s = s.masked_fill(~mask, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vv)
        (o * torch.tensor(g)).sum().backward()
        for name, mine, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            err = np.abs(mine - ref.numpy()).max()
            assert err <= 1e-12 * max(1.0, np.abs(ref.numpy()).max()), (name, n, err)


def pin_grad_invariants(lib):
    for n, (B, Hq, Hkv, N, d, causal, scale) in enumerate(SHAPES):
        q, k, v, g = _draw(7200 + n, B, Hq, Hkv, N, d)
        dq, dk, dv = oracle.grads(q, k, v, g, causal, scale, lib=lib)
        G = Hq // Hkv
        # sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
        assert np.abs(dk.sum(axis=2)).max() <= 1e-12 * max(1.0, np.abs(dk).max()), ("sum dK", n)
        # sum_j dV_j = sum over the group's query heads and rows of dO_i
        gs = g.reshape(B, Hkv, G, N, d).sum(axis=(2, 3))
        assert np.abs(dv.sum(axis=2) - gs).max() <= 1e-12 * max(1.0, np.abs(gs).max()), ("sum dV", n)
        # constant V rows: O no longer depends on Q or K
        vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
        dq0, dk0, dv0 = oracle.grads(q, k, vc, g, causal, scale, lib=lib)
        assert np.abs(dq0).max() <= 1e-13 and np.abs(dk0).max() <= 1e-13, ("const V", n)


def pin_grad_closed_forms(lib):
    # One key: P = 1, so dV_0 = sum_i dO_i (over the group), dQ = dK = 0.
    q, k, v, g = _draw(7300, 1, 2, 1, 1, 4)
    dq, dk, dv = oracle.grads(q, k, v, g, False, 0.8, lib=lib)
    assert np.abs(dv[0, 0, 0] - g[0, :, 0].sum(axis=0)).max() <= 1e-14
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    # Causal: row 0 sees only key 0, so dQ_0 = 0, and dO_0 flows into dV_0 alone.
    q, k, v, g = _draw(7301, 1, 1, 1, 4, 3)
    g0 = np.zeros_like(g)
    g0[0, 0, 0] = g[0, 0, 0]
    dq, dk, dv = oracle.grads(q, k, v, g0, True, 0.6, lib=lib)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    assert np.abs(dv[0, 0, 0] - g0[0, 0, 0]).max() <= 1e-15 and np.abs(dv[0, 0, 1:]).max() == 0.0
    # Two keys, one query, d = 1: dq = scale * p0 p1 (k0 - k1) (v0 - v1) g.
    q = np.array([[[[0.7]]]]); k = np.array([[[[0.3], [-1.1]]]]); v = np.array([[[[2.0], [0.5]]]])
    q2 = np.concatenate([q, q], axis=2)          # query row 1 sees both keys
    g2 = np.array([[[[0.0], [1.5]]]])
    sc = 0.9
    s0, s1 = sc * 0.7 * 0.3, sc * 0.7 * -1.1
    p0 = np.exp(s0) / (np.exp(s0) + np.exp(s1)); p1 = 1 - p0
    dq, dk, dv = oracle.grads(q2, k, v, g2, True, sc, lib=lib)
    want = sc * p0 * p1 * (0.3 - -1.1) * (2.0 - 0.5) * 1.5
    assert abs(dq[0, 0, 1, 0] - want) <= 1e-14, (dq[0, 0, 1, 0], want)
