"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` takes a loaded oracle library (``oracle.load(path)``) and raises
AssertionError when the oracle disagrees with:

* brute force in 50-digit decimal arithmetic, without max subtraction, on tiny
  inputs (the definition of "FlashAttention (VI)", eq. Attention, evaluated a
  different way);
* torch's own fp64 ``scaled_dot_product_attention`` (a library routine; it also
  fixes the causal diagonal and the grouped-query head mapping independently);
* closed forms: N = 1, N = 2, Q = 0 / scale = 0 (means of the visible V rows),
  V = I (the output is the softmax matrix, checked against scipy's softmax);
* invariants: softmax rows sum to 1, constant V rows are reproduced, causal row 0
  is V[0] exactly, joint permutations of K and V rows leave non-causal output
  unchanged, the last causal row equals the last non-causal row, grouped-query
  output equals multi-head output over repeated K/V, row subsets and thread counts
  change nothing;
* the blocked online-softmax reference, to 1e-12 at many tilings.

The same functions run on deliberately broken copies of the oracle sources
(tests/test_oracle_mutants.py) to show that every plausible mistake is caught.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np
import scipy.special
import torch

import oracle
from fa_inputs import make_inputs


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    ok = np.isfinite(a).all() and np.isfinite(b).all() and bool((err <= tol).all())
    assert ok, f"{what}: max err {np.nanmax(err) if err.size else 0} > {tol} (finite={np.isfinite(a).all()})"


def _inp(seed, B, Hq, Hkv, N, d, causal, scale=None, mult=1.0):
    x = make_inputs(seed, B, Hq, Hkv, N, d, "f64", causal, scale=scale, mult=mult)
    return x, x.f64("q"), x.f64("k"), x.f64("v")


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, causal, scale):
    """sum_j e^{s_ij} v_j / sum_j e^{s_ij} and ln sum_j e^{s_ij}, 50 digits, no max shift."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(scale)
        for b in range(B):
            for h in range(Hq):
                kv = h * Hkv // Hq          # consecutive query heads share a K/V head
                for i in range(N):
                    num = [Decimal(0)] * d
                    den = Decimal(0)
                    for j in range(N):
                        if causal and j > i:
                            continue
                        s = sc * sum(Decimal(q[b, h, i, t]) * Decimal(k[b, kv, j, t])
                                     for t in range(d))
                        w = s.exp()
                        den += w
                        for t in range(d):
                            num[t] += w * Decimal(v[b, kv, j, t])
                    o[b, h, i] = [float(x / den) for x in num]
                    lse[b, h, i] = float(den.ln())
    return o, lse


def pin_brute_force(lib, quick=False):
    Ns = (1, 2, 3, 5, 8, 13)
    ds = (1, 2, 4, 8)
    heads = ((1, 1), (2, 1), (4, 2))
    seed = 3000
    for N in Ns:
        for d in ds:
            for Hq, Hkv in heads:
                if quick and (d, Hq) not in ((2, 4), (8, 2), (1, 1)):
                    continue
                for causal in (False, True):
                    seed += 1
                    B = 2 if (N + d) % 3 == 0 else 1
                    # scores reach |s| of order 10-20
                    _, q, k, v = _inp(seed, B, Hq, Hkv, N, d, causal, scale=1.5, mult=2.0)
                    o, lse = oracle.attention(q, k, v, causal, 1.5, lib=lib)
                    ob, lb = _brute(q, k, v, causal, 1.5)
                    _close(o, ob, 1e-13, f"brute O N={N} d={d} H={Hq}/{Hkv} c={causal}")
                    _close(lse, lb, 1e-13, f"brute lse N={N} d={d} H={Hq}/{Hkv} c={causal}")


# ------------------------------------------------------------ torch routine
_TORCH_CASES = (
    ((2, 4, 2, 200, 64), 0.125),
    ((1, 8, 1, 77, 32), 0.5),
    ((1, 3, 3, 129, 128), -0.3),
    ((3, 6, 2, 64, 16), None),
)


def pin_torch_sdpa(lib):
    seed = 4000
    for (B, Hq, Hkv, N, d), scale in _TORCH_CASES:
        for causal in (False, True):
            seed += 1
            x, q, k, v = _inp(seed, B, Hq, Hkv, N, d, causal, scale=scale)
            o, lse = oracle.attention(q, k, v, causal, x.scale, lib=lib)
            tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
            # torch's is_causal masks before scaling, which breaks for a negative
            # scale; there the same lower-triangular mask goes in as attn_mask.
            mask = None
            if causal and x.scale < 0:
                mask = torch.ones(N, N, dtype=torch.bool).tril()
            ot = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=mask, is_causal=causal and mask is None,
                scale=x.scale, enable_gqa=Hq != Hkv)
            _close(o, ot.numpy(), 1e-12, f"sdpa O {(B, Hq, Hkv, N, d)} c={causal}")
            krep = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
            s = x.scale * torch.matmul(tq, krep.transpose(-1, -2).contiguous())
            if causal:
                s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12,
                   f"logsumexp {(B, Hq, Hkv, N, d)} c={causal}")


# ------------------------------------------------------------- closed forms
def pin_closed_forms(lib):
    # N = 1: the only key is visible, so O = V[0] and lse = s_00.
    for causal in (False, True):
        x, q, k, v = _inp(5001, 2, 4, 2, 1, 16, causal)
        o, lse = oracle.attention(q, k, v, causal, x.scale, lib=lib)
        kvh = [0, 0, 1, 1]
        _close(o, v[:, kvh], 0.0, "N=1 O")
        s00 = x.scale * np.einsum("bht,bht->bh", q[:, :, 0], k[:, kvh, 0])
        _close(lse[:, :, 0], s00, 1e-14, "N=1 lse")

    # N = 2, non-causal: O_i = (e^{s_i0} v_0 + e^{s_i1} v_1) / (e^{s_i0} + e^{s_i1}).
    x, q, k, v = _inp(5002, 1, 1, 1, 2, 8, False, scale=0.7, mult=2.0)
    o, lse = oracle.attention(q, k, v, False, x.scale, lib=lib)
    s = x.scale * (q[0, 0] @ k[0, 0].T)
    w = np.exp(s)
    _close(o[0, 0], (w @ v[0, 0]) / w.sum(1, keepdims=True), 1e-14, "N=2 O")
    _close(lse[0, 0], np.log(w.sum(1)), 1e-14, "N=2 lse")

    # Q = 0 or scale = 0: uniform weights over the visible keys.
    for causal in (False, True):
        for mode in ("q0", "scale0"):
            x, q, k, v = _inp(5003, 1, 2, 1, 37, 8, causal)
            scale = x.scale
            if mode == "q0":
                q = np.zeros_like(q)
            else:
                scale = 0.0
            o, lse = oracle.attention(q, k, v, causal, scale, lib=lib)
            vv = v[0, 0]
            if causal:
                ref = np.cumsum(vv, axis=0) / np.arange(1, 38)[:, None]
                cnt = np.arange(1, 38, dtype=np.float64)
            else:
                ref = np.broadcast_to(vv.mean(axis=0), vv.shape)
                cnt = np.full(37, 37.0)
            for h in range(2):
                _close(o[0, h], ref, 1e-14, f"{mode} O c={causal}")
                _close(lse[0, h], np.log(cnt), 1e-14, f"{mode} lse c={causal}")

    # V = I (N = d): O is the softmax matrix itself.
    for causal in (False, True):
        x, q, k, _ = _inp(5004, 1, 1, 1, 24, 24, causal, mult=1.5)
        eye = np.eye(24)[None, None]
        o, _ = oracle.attention(q, k, eye, causal, x.scale, lib=lib)
        s = x.scale * (q[0, 0] @ k[0, 0].T)
        if causal:
            s = np.where(np.tril(np.ones((24, 24), bool)), s, -np.inf)
        ref = scipy.special.softmax(s, axis=1)
        _close(o[0, 0], ref, 1e-15, f"V=I O c={causal}")
        _close(oracle.probs(q, k, causal, x.scale, lib=lib)[0, 0], ref, 1e-15,
               f"V=I probs c={causal}")


# --------------------------------------------------------------- invariants
def pin_invariants(lib):
    # Softmax rows sum to 1.
    for causal in (False, True):
        x, q, k, _ = _inp(6001, 2, 4, 2, 50, 16, causal, mult=2.0)
        p = oracle.probs(q, k, causal, x.scale, lib=lib)
        _close(p.sum(-1), np.ones(p.shape[:-1]), 1e-14, f"row sums c={causal}")
        assert (p >= 0).all(), "negative probability"
        if causal:
            assert (p[..., np.triu_indices(50, 1)[0], np.triu_indices(50, 1)[1]] == 0).all()

    # Constant V rows give that row back.
    for causal in (False, True):
        x, q, k, v = _inp(6002, 1, 4, 2, 64, 32, causal, mult=2.0)
        c = v[:, :, :1, :]
        vc = np.broadcast_to(c, v.shape).copy()
        o, _ = oracle.attention(q, k, vc, causal, x.scale, lib=lib)
        _close(o, np.repeat(np.broadcast_to(c, v.shape), 2, axis=1), 1e-14,
               f"constant V c={causal}")

    # Causal row 0 is V[0] exactly; the last causal row is the last full row.
    x, q, k, v = _inp(6003, 2, 4, 4, 45, 16, True)
    oc, lc = oracle.attention(q, k, v, True, x.scale, lib=lib)
    on, ln_ = oracle.attention(q, k, v, False, x.scale, lib=lib)
    _close(oc[:, :, 0], v[:, :, 0], 0.0, "causal row 0")
    _close(oc[:, :, -1], on[:, :, -1], 0.0, "last causal row")
    _close(lc[:, :, -1], ln_[:, :, -1], 0.0, "last causal lse")

    # Joint permutation of K and V rows leaves non-causal output unchanged.
    x, q, k, v = _inp(6004, 1, 2, 2, 70, 16, False, mult=2.0)
    perm = np.random.default_rng(6004).permutation(70)
    o1, l1 = oracle.attention(q, k, v, False, x.scale, lib=lib)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, x.scale, lib=lib)
    _close(o1, o2, 1e-14, "permutation O")
    _close(l1, l2, 1e-14, "permutation lse")

    # Grouped-query output equals multi-head output over repeated K/V heads.
    for causal in (False, True):
        x, q, k, v = _inp(6005, 2, 8, 2, 33, 16, causal)
        og, lg = oracle.attention(q, k, v, causal, x.scale, lib=lib)
        om, lm = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                  causal, x.scale, lib=lib)
        _close(og, om, 0.0, f"GQA vs MHA O c={causal}")
        _close(lg, lm, 0.0, f"GQA vs MHA lse c={causal}")

    # Row subsets and thread counts change nothing.
    x, q, k, v = _inp(6006, 2, 2, 1, 300, 16, True)
    of, lf = oracle.attention(q, k, v, True, x.scale, threads=1, lib=lib)
    rows = np.array([299, 0, 5, 128, 1, 77])
    orr, lrr = oracle.attention(q, k, v, True, x.scale, rows=rows, threads=3, lib=lib)
    _close(orr, of[:, :, rows], 0.0, "row subset O")
    _close(lrr, lf[:, :, rows], 0.0, "row subset lse")
    om, lm = oracle.attention(q, k, v, True, x.scale, threads=7, lib=lib)
    _close(om, of, 0.0, "thread count O")


# ------------------------------------------------------ blocked vs naive
_TILINGS = ((1, 1), (7, 5), (16, 16), (32, 32), (64, 128), (128, 64))


def pin_blocked_agrees(lib, quick=False):
    seed = 7000
    shapes = ((1, 2, 1, 1, 8), (1, 1, 1, 2, 8), (1, 2, 2, 33, 16), (2, 4, 2, 100, 32),
              (1, 2, 1, 129, 64))
    for (B, Hq, Hkv, N, d) in shapes:
        for causal in (False, True):
            seed += 1
            x, q, k, v = _inp(seed, B, Hq, Hkv, N, d, causal, mult=3.0)
            o, lse = oracle.attention(q, k, v, causal, x.scale, lib=lib)
            for br, bc in (_TILINGS[:3] if quick else _TILINGS):
                ob, lb = oracle.blocked(q, k, v, causal, x.scale, br, bc, lib=lib)
                _close(ob, o, 1e-12, f"blocked O {(B, Hq, Hkv, N, d)} c={causal} {br}x{bc}")
                _close(lb, lse, 1e-12, f"blocked lse {(B, Hq, Hkv, N, d)} c={causal} {br}x{bc}")


ORACLE_PINS = (pin_brute_force, pin_torch_sdpa, pin_closed_forms, pin_invariants)
BLOCKED_PINS = (pin_blocked_agrees,)
