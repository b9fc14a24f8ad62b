"""Seeded random sweep of GPU parity cases over the whole C ABI.

Each case draws its shape and options from a fixed-seed generator (so the sweep
is the same on every run): batch, query and K/V head counts (GQA groups 1, 2, 4),
sequence length (1 .. 700, so single rows, partial tiles and several tiles all
occur), head dim, causal flag, scale of either sign, input magnitude, tiling and,
for split-KV, the split count.  Every case is compared with the fp64 oracle under
the same tolerance as the hand-picked cases of the same entry point.
"""
import numpy as np
import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F
import oracle
import parity as PT

pytestmark = pytest.mark.gpu

TILES = {64: [(128, 64), (64, 64), (128, 32), (256, 64)],
         128: [(128, 64), (64, 64), (128, 32), (256, 64)],
         256: [(128, 64), (128, 32)]}


def draw(seed, dims=(64, 128, 256), nmax=700):
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2]))
    G_ = int(r.choice([1, 2, 4]))
    N = int(r.choice([int(r.integers(1, 40)), int(r.integers(40, nmax + 1))]))
    d = int(r.choice(dims))
    scale = float(r.choice([-1.0, 1.0])) * float(r.uniform(0.3, 1.5)) / np.sqrt(d)
    return dict(B=int(r.choice([1, 2])), Hq=Hkv * G_, Hkv=Hkv, N=N, d=d,
                causal=bool(r.integers(0, 2)), scale=scale, mult=float(r.choice([1.0, 2.0])),
                r=r)


def _tag(c):
    return f"B{c['B']}-H{c['Hq']}x{c['Hkv']}-N{c['N']}-d{c['d']}-{'causal' if c['causal'] else 'full'}" \
           f"-s{c['scale']:+.3f}-x{c['mult']:g}"


@pytest.mark.parametrize("seed", range(20))
def test_random_forward(seed):
    c = draw(31000 + seed)
    dt = str(c["r"].choice(["bf16", "f16"]))
    tl = TILES[c["d"]][int(c["r"].integers(0, len(TILES[c["d"]])))]
    out_f32 = bool(c["r"].integers(0, 2)) and tl != (64, 64)    # 64 x 64: 16-bit output only
    x = G.make_inputs(31000 + seed, c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], dt, c["causal"],
                      scale=c["scale"], mult=c["mult"])
    o_ref, l_ref = oracle.attention(x.f64("q"), x.f64("k"), x.f64("v"), x.causal, x.scale)
    q, k, v = PT.to_device(x)
    o, l = F.fwd(q, k, v, causal=x.causal, scale=x.scale, tuning=tl,
                 out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    PT.compare(o.float().cpu().double().numpy(), l.cpu().double().numpy(), o_ref, l_ref, dt,
               out_f32, f"{dt} {_tag(c)} tile{tl} f32out={out_f32}")


@pytest.mark.parametrize("seed", range(8))
def test_random_split(seed):
    c = draw(32000 + seed, dims=(64, 128))
    dt = str(c["r"].choice(["bf16", "f16"]))
    S = int(c["r"].integers(1, 17))
    x = G.make_inputs(32000 + seed, c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], dt, c["causal"],
                      scale=c["scale"], mult=c["mult"])
    o_ref, l_ref = oracle.attention(x.f64("q"), x.f64("k"), x.f64("v"), x.causal, x.scale)
    q, k, v = PT.to_device(x)
    o, l = F.fwd_split(q, k, v, causal=x.causal, scale=x.scale, num_splits=S)
    torch.cuda.synchronize()
    PT.compare(o.float().cpu().double().numpy(), l.cpu().double().numpy(), o_ref, l_ref, dt,
               False, f"{dt} {_tag(c)} S{S}")


@pytest.mark.parametrize("seed", range(6))
def test_random_bias(seed):
    c = draw(33000 + seed, dims=(64, 128), nmax=400)
    dt = str(c["r"].choice(["bf16", "f16"]))
    N = c["N"]
    shape = [(1, 1, N, N), (1, c["Hq"], N, N), (c["B"], c["Hq"], N, N)][int(c["r"].integers(0, 3))]
    x = G.make_inputs(33000 + seed, c["B"], c["Hq"], c["Hkv"], N, c["d"], dt, c["causal"],
                      scale=c["scale"], mult=c["mult"])
    bias = G.storage_to_f64(G.make_normal(33500 + seed, shape, dt), dt)
    # Mask about a tenth of the pairs, keeping each row's diagonal key visible.
    mask = c["r"].random(shape) < 0.1
    mask &= ~np.eye(N, dtype=bool)[None, None]
    bias = np.where(mask, -np.inf, bias)
    o_ref, l_ref = oracle.attention_bias(x.f64("q"), x.f64("k"), x.f64("v"), bias, x.causal, x.scale)
    st = G.to_storage(bias, dt)
    tb = torch.from_numpy(st)
    tb = (tb.view(torch.bfloat16) if dt == "bf16" else tb).cuda()
    q, k, v = PT.to_device(x)
    o, l = F.fwd_bias(q, k, v, tb, causal=x.causal, scale=x.scale)
    torch.cuda.synchronize()
    PT.compare(o.float().cpu().double().numpy(), l.cpu().double().numpy(), o_ref, l_ref, dt,
               False, f"{dt} {_tag(c)} bias{shape[:2]}")


@pytest.mark.parametrize("seed", range(6))
def test_random_fp8(seed):
    import test_gpu_fp8 as T8
    c = draw(34000 + seed, dims=(64, 128), nmax=500)
    x = G.make_inputs(34000 + seed, c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], "e4m3", c["causal"],
                      scale=c["scale"], mult=c["mult"])
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    o_ref, l_ref = oracle.attention(q, k, v, x.causal, x.scale)
    w = oracle.probs(q, k, x.causal, x.scale)
    o, lse = T8.run_fp8(x)
    T8.check(f"e4m3 {_tag(c)}", o, lse, o_ref, l_ref, *T8.bounds(x, w, o_ref))


@pytest.mark.parametrize("seed", range(6))
def test_random_backward(seed):
    import test_gpu_bwd as TB
    c = draw(35000 + seed, dims=(64, 128), nmax=300)
    dt = str(c["r"].choice(["bf16", "f16"]))
    x, g, dout, o_st, lse = TB.case(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], dt, c["causal"],
                                    c["mult"], c["scale"], seed=35000 + seed)
    dq, dk, dv = TB.run_bwd(x, g, o_st, lse)
    rq, rk, rv = oracle.grads(x.f64("q"), x.f64("k"), x.f64("v"), dout, x.causal, x.scale)
    bq, bk, bv = TB.bounds(x, dout, o_st)
    TB.check(f"dq {_tag(c)}", dq, rq, bq)
    TB.check(f"dk {_tag(c)}", dk, rk, bk)
    TB.check(f"dv {_tag(c)}", dv, rv, bv)


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    import test_gpu_decode as TD
    r = np.random.default_rng(36000 + seed)
    Hkv = int(r.choice([1, 2, 4]))
    G_ = int(r.choice([1, 2, 4, 8]))
    Nq = int(r.integers(1, 32 // G_ + 1))
    Nk = int(r.integers(Nq, 1500))
    d = int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f16"]))
    causal = bool(r.integers(0, 2))
    S = int(r.integers(1, 40))
    scale = float(r.choice([-1.0, 1.0])) * float(r.uniform(0.3, 1.5)) / np.sqrt(d)
    B = int(r.choice([1, 2, 3]))
    st = TD.draw(36000 + seed, B, Hkv * G_, Hkv, Nq, Nk, d, dt, float(r.choice([1.0, 2.0])))
    q, k, v = (G.storage_to_f64(a, dt) for a in st)
    o_ref, l_ref = oracle.attention_kv(q, k, v, causal, scale)
    o, l = TD.run(st, dt, causal, scale, S)
    PT.compare(o, l, o_ref, l_ref, dt, False,
               f"{dt} B{B} H{Hkv * G_}x{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} S{S} s{scale:+.3f}")
