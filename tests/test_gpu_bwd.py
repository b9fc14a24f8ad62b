"""GPU parity of the backward pass: libfa355's fa_bwd against the fp64 gradient
oracle, through the C ABI.

The kernels get the oracle's O (rounded to the input type) and lse (rounded to
fp32), so what is measured is the backward arithmetic alone.  Its rounding
steps, and the elementwise bound each one contributes (u = 2^-8 for bf16, 2^-11
for fp16: the unit roundoff of the operand type):

* P is recomputed in fp32 (exp2 of an fp32 score minus the fp32 lse: relative
  error below ~1e-5) and rounded to the input type as an operand of dV:
      |dV err|_jt <= (u + 1e-5) sum_i P_ij |dO_it|
* D_i = dO_i . O_i reads the rounded O: |D err|_i <= u sum_t |dO_it| |O_it|
  (+ fp32 accumulation, d 2^-24 of the same sum);
* dS_ij = P_ij (dP_ij - D_i) is rounded to the input type as an operand:
      |dS err|_ij <= P_ij |D err|_i + u |dS_ij| + 1e-5 P_ij |dP_ij - D_i|
* dQ = scale dS K and dK = scale dS^T Q accumulate in fp32:
      |dQ err|_it <= |scale| sum_j |dS err|_ij |K_jt|,
      |dK err|_jt <= |scale| sum_i |dS err|_ij |Q_it|.
The tests allow twice these bounds (plus 1e-6 of the largest reference value for
exact zeros), computed per element from the oracle's P, dP and D.
"""
import numpy as np
import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F
import oracle

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16}
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def case(B, Hq, Hkv, N, d, dt, causal, mult=1.0, scale=None, seed=0):
    x = G.make_inputs(seed, B, Hq, Hkv, N, d, dt, causal, scale=scale, mult=mult)
    g = G.make_grad_output(seed + 1, (B, Hq, N, d), dt)
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    dout = G.storage_to_f64(g, dt)
    o, lse = oracle.attention(q, k, v, causal, x.scale)
    o_st = G.to_storage(G.round_to_dtype(o, dt), dt)
    return x, g, dout, o_st, lse


def run_bwd(x, g, o_st, lse):
    dt = x.dtype
    q, k, v = (_dev(getattr(x, n), dt) for n in "qkv")
    dq, dk, dv = F.bwd(q, k, v, _dev(o_st, dt), _dev(g, dt),
                       torch.from_numpy(lse.astype(np.float32)).cuda(), causal=x.causal,
                       scale=x.scale)
    torch.cuda.synchronize()
    return dq.cpu().double().numpy(), dk.cpu().double().numpy(), dv.cpu().double().numpy()


def bounds(x, dout, o_st):
    """Elementwise error bounds of dQ, dK, dV (module docstring)."""
    dt, u = x.dtype, UNIT[x.dtype]
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    o = G.storage_to_f64(o_st, dt)
    G_ = x.Hq // x.Hkv
    kk = np.repeat(k, G_, axis=1)
    vv = np.repeat(v, G_, axis=1)
    p = oracle.probs(q, k, x.causal, x.scale)                     # [B,Hq,N,N]
    dp = dout @ np.swapaxes(vv, -1, -2)
    dd = (p * dp).sum(-1, keepdims=True)
    ds = p * (dp - dd)
    d_err = (u + x.d * 2.0 ** -24) * (np.abs(dout) * np.abs(o)).sum(-1, keepdims=True)
    ds_err = p * d_err + u * np.abs(ds) + 1e-5 * p * np.abs(dp - dd)
    sc = abs(x.scale)
    b_dq = sc * ds_err @ np.abs(kk)
    b_dk = sc * np.swapaxes(ds_err, -1, -2) @ np.abs(q)
    b_dv = (u + 1e-5) * np.swapaxes(p, -1, -2) @ np.abs(dout)
    B, Hkv, N, d = k.shape
    b_dk = b_dk.reshape(B, Hkv, G_, N, d).sum(2)
    b_dv = b_dv.reshape(B, Hkv, G_, N, d).sum(2)
    return b_dq, b_dk, b_dv


def check(name, got, ref, bound):
    assert np.isfinite(got).all(), f"{name}: non-finite"
    tol = 2.0 * bound + 1e-6 * max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref)
    worst = (err / tol).max()
    assert worst <= 1.0, f"{name}: max err {err.max():.3g}, worst err/bound {worst:.3f}"
    return err.max()


# (B, Hq, Hkv, N, d, dtype, causal, mult, scale)
CASES = [
    (1, 2, 2, 256, 128, "bf16", True, 1.0, None),
    (2, 4, 2, 333, 128, "bf16", False, 1.0, None),
    (1, 4, 1, 200, 64, "f16", True, 1.0, None),
    (1, 2, 1, 130, 64, "bf16", False, 1.0, -0.2),
    (1, 2, 2, 1, 128, "f16", True, 1.0, None),
    (1, 2, 2, 31, 64, "bf16", True, 1.0, None),
    (1, 2, 2, 512, 128, "bf16", True, 3.0, None),
    (1, 3, 3, 257, 64, "f16", False, 2.0, None),
    (1, 4, 4, 1024, 128, "bf16", True, 1.0, None),
    (2, 8, 2, 160, 128, "f16", True, 1.0, None),
    # Enough query tiles (B * Hq * ceil(N / 256) >= 256) for 256-query dQ workgroups,
    # with a ragged last tile.
    (8, 16, 4, 300, 128, "bf16", True, 1.0, None),
    (16, 16, 16, 260, 64, "f16", False, 1.0, None),
    # Head dim 256: two wavefront pairs per dK/dV workgroup (64 keys), one wavefront
    # per SIMD; 128-query dQ workgroups.
    (1, 2, 2, 200, 256, "bf16", True, 1.0, None),
    (1, 4, 2, 130, 256, "f16", False, 1.0, None),
    (1, 2, 1, 97, 256, "bf16", True, 2.0, -0.3),
    (1, 2, 2, 1024, 256, "bf16", True, 3.0, None),
]


def _id(c):
    B, Hq, Hkv, N, d, dt, causal, mult, scale = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-N{N}-d{d}-{'causal' if causal else 'full'}" + \
        (f"-x{mult:g}" if mult != 1 else "") + (f"-s{scale:g}" if scale is not None else "")


@pytest.mark.parametrize("cfg", CASES, ids=[_id(c) for c in CASES])
def test_bwd_parity(cfg):
    B, Hq, Hkv, N, d, dt, causal, mult, scale = cfg
    x, g, dout, o_st, lse = case(B, Hq, Hkv, N, d, dt, causal, mult, scale, seed=9700 + N + d)
    dq, dk, dv = run_bwd(x, g, o_st, lse)
    rq, rk, rv = oracle.grads(x.f64("q"), x.f64("k"), x.f64("v"), dout, causal, x.scale)
    bq, bk, bv = bounds(x, dout, o_st)
    check("dq", dq, rq, bq)
    check("dk", dk, rk, bk)
    check("dv", dv, rv, bv)


def test_bwd_deterministic():
    x, g, dout, o_st, lse = case(1, 4, 2, 300, 128, "bf16", True, seed=9801)
    a = run_bwd(x, g, o_st, lse)
    b = run_bwd(x, g, o_st, lse)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_bwd_wide_and_narrow_dq_tiles_agree():
    # Eight batches take 256-query dQ workgroups, one batch alone takes 128-query
    # ones; each query row sums the same key blocks in the same order either way, so
    # the gradients of batch 0 are bit-identical.
    x, g, dout, o_st, lse = case(8, 16, 4, 300, 128, "bf16", True, seed=9803)
    full = run_bwd(x, g, o_st, lse)
    x0 = G.AttentionInputs(1, x.Hq, x.Hkv, x.N, x.d, x.dtype, x.causal, x.scale, x.seed,
                           x.q[:1], x.k[:1], x.v[:1])
    one = run_bwd(x0, g[:1], o_st[:1], lse[:1])
    for u, w in zip(full, one):
        assert np.array_equal(u[:1], w)


def test_bwd_gqa_equals_repeated_heads():
    # dK, dV of a shared K/V head are the sums of what each query head would give it
    # with its own copy; dQ is the same either way.
    x, g, dout, o_st, lse = case(1, 4, 2, 200, 64, "bf16", True, seed=9802)
    dq, dk, dv = run_bwd(x, g, o_st, lse)
    xm = G.AttentionInputs(x.B, x.Hq, x.Hq, x.N, x.d, x.dtype, x.causal, x.scale, x.seed,
                           x.q, np.repeat(x.k, 2, axis=1), np.repeat(x.v, 2, axis=1))
    dq2, dk2, dv2 = run_bwd(xm, g, o_st, lse)
    assert np.array_equal(dq, dq2)
    rk = dk2.reshape(1, 2, 2, 200, 64).sum(2)
    rv = dv2.reshape(1, 2, 2, 200, 64).sum(2)
    assert np.abs(dk - rk).max() <= 1e-5 * np.abs(rk).max()
    assert np.abs(dv - rv).max() <= 1e-5 * np.abs(rv).max()


def test_bwd_full_size_two_heads_elementwise():
    # The headline layer (B1 H32 N4096 d128 causal) in the launch configuration the
    # benchmark times, with heads 0 and 31 checked element by element against the
    # fp64 gradient oracle under the bounds of test_bwd_parity.  Heads are
    # independent (one K/V head per query head), so those two get the oracle's O
    # (rounded to bf16) and lse; the other 30 take the GPU forward's.
    x = G.workload("bf16_h32_n4096_d128_causal")
    assert x.Hq == x.Hkv
    g = G.make_grad_output(4243, (x.B, x.Hq, x.N, x.d), "bf16")
    q, k, v = (_dev(getattr(x, n), "bf16") for n in "qkv")
    o, lse = F.fwd(q, k, v, causal=True, scale=x.scale)
    heads = (0, x.Hq - 1)
    one = {}
    for h in heads:
        xh = G.AttentionInputs(1, 1, 1, x.N, x.d, "bf16", True, x.scale, x.seed,
                               x.q[:, h:h + 1], x.k[:, h:h + 1], x.v[:, h:h + 1])
        dh = G.storage_to_f64(g[:, h:h + 1], "bf16")
        oh, lh = oracle.attention(xh.f64("q"), xh.f64("k"), xh.f64("v"), True, x.scale)
        oh_st = G.to_storage(G.round_to_dtype(oh, "bf16"), "bf16")
        o[:, h:h + 1] = _dev(oh_st, "bf16")
        lse[:, h:h + 1] = torch.from_numpy(lh.astype(np.float32)).cuda()
        one[h] = (xh, dh, oh_st)
    print("bwd full size: B1 H32 N4096 d128 causal, heads", heads, flush=True)
    dq, dk, dv = F.bwd(q, k, v, o, _dev(g, "bf16"), lse, causal=True, scale=x.scale)
    torch.cuda.synchronize()
    for h in heads:
        xh, dh, oh_st = one[h]
        rq, rk, rv = oracle.grads(xh.f64("q"), xh.f64("k"), xh.f64("v"), dh, True, x.scale)
        bq, bk, bv = bounds(xh, dh, oh_st)
        for name, got, ref, b in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
            check(f"{name} head {h}", got[:, h:h + 1].cpu().double().numpy(), ref, b)


@pytest.mark.parametrize("name", ["bf16_h32_n4096_d128_causal", "bf16_h8_n8192_d256_causal_x3"])
def test_bwd_full_size_invariants(name):
    # The headline layer (B1 H32 N4096 d128 causal) and the head-dim-256 layer (B1 H8
    # N8192 causal, inputs x3) end to end: forward on the GPU, then backward, in the
    # launch configuration the benchmark times.  A property that holds at any size:
    # sum_j dV_j = sum_i (sum_j P_ij) dO_i = sum_i dO_i, up to the rounding of P to
    # bf16 (u = 2^-8 relative) and the forward lse's error (< 1e-3):
    # |sum_j dV_jt - sum_i dO_it| <= 2 (u + 1e-3) sum_i |dO_it|.
    x = G.workload(name)
    g = G.make_grad_output(4242, (x.B, x.Hq, x.N, x.d), "bf16")
    q, k, v = (_dev(getattr(x, n), "bf16") for n in "qkv")
    o, lse = F.fwd(q, k, v, causal=True, scale=x.scale)
    dg = _dev(g, "bf16")
    dq, dk, dv = F.bwd(q, k, v, o, dg, lse, causal=True, scale=x.scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    sdv = dv.double().sum(dim=2)
    sdo = dg.double().sum(dim=2)
    bound = 2 * (2.0 ** -8 + 1e-3) * dg.double().abs().sum(dim=2)
    assert ((sdv - sdo).abs() <= bound).all()
