"""Seeded synthetic inputs for the attention forward pass.

This module holds no attention arithmetic. It draws random numbers and rounds
them to the storage dtypes, and it is the one piece of code that both sides of a
parity check share: the fp64 CPU oracle gets the exact values of the stored
tensors, the GPU library gets the stored tensors themselves.

Random numbers
    SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014).  Output k (k = 0, 1, ...) of the stream with seed s
    is mix(s + (k+1)*0x9E3779B97F4A7C15 mod 2^64), which makes the generator
    counter-based and lets numpy draw any slice of the stream directly.
    A uniform is (x >> 11) * 2^-53 in [0, 1).  Normals come in pairs by the
    Box-Muller transform (Box and Muller, 1958) from uniforms (2p, 2p+1):
    r = sqrt(-2 ln(1 - u0)), n0 = r cos(2 pi u1), n1 = r sin(2 pi u1).

Fill order
    Q, then K, then V, each in row-major [B, H, N, d] order; every tensor starts on
    a fresh normal pair.  When a per-head query bias is requested, Hq uniforms
    follow V and beta_h = 2 u_h is added to every element of Q[:, h].  Values are
    multiplied (then biased) in fp64 and rounded once, fp64 -> storage dtype,
    round-to-nearest-even.

8-bit inputs ("e4m3")
    OCP e4m3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; normals
    (1 + f/8) 2^(E-7) for E = 1..15, subnormals f 2^-9, largest finite 448 (code
    0x7e), codes 0x7f / 0xff NaN.  Each tensor gets one descale, the fp32 value of
    max|x| / 448 (1 for an all-zero tensor); the stored codes are x / descale,
    clipped to [-448, 448] and rounded once to e4m3, and the value of an element is
    descale * e4m3(code) (exact in fp64).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "splitmix64", "Stream", "round_to_dtype", "to_storage", "storage_to_f64",
    "AttentionInputs", "make_inputs", "WORKLOADS", "workload", "quantize_e4m3",
    "DecodeInputs", "make_decode_inputs", "DECODE_WORKLOADS",
]

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 19  # normal pairs per numpy pass (bounds temporaries, feeds threads)
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, step: int, fn) -> None:
    """fn(start, stop) over [0, n) in chunks, on a thread pool (numpy drops the GIL)."""
    starts = range(0, n, step)
    if len(starts) <= 1:
        for a in starts:
            fn(a, min(n, a + step))
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda a: fn(a, min(n, a + step)), starts))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream seeded with `seed`."""
    with np.errstate(over="ignore"):
        k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def _uniform53(z: np.ndarray) -> np.ndarray:
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


class Stream:
    """A cursor over one seeded SplitMix64 stream, counted in uniforms."""

    def __init__(self, seed: int):
        self.seed = int(seed)
        self.pos = 0

    def uniforms(self, count: int) -> np.ndarray:
        u = _uniform53(splitmix64(self.seed, self.pos, count))
        self.pos += count
        return u

    def normals(self, count: int) -> np.ndarray:
        """`count` N(0,1) draws; consumes 2*ceil(count/2) uniforms."""
        pairs = (count + 1) // 2
        out = np.empty(2 * pairs, dtype=np.float64)
        base = self.pos

        def fill(p0, p1):
            u = _uniform53(splitmix64(self.seed, base + 2 * p0, 2 * (p1 - p0)))
            r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
            t = (2.0 * math.pi) * u[1::2]
            out[2 * p0:2 * p1:2] = r * np.cos(t)
            out[2 * p0 + 1:2 * p1:2] = r * np.sin(t)

        _chunked(pairs, _CHUNK, fill)
        self.pos += 2 * pairs
        return out[:count]


# (precision p in bits incl. the implicit one, minimum normal exponent, largest finite)
_FORMATS = {
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
    "f16": (11, -14, 65504.0),
    "e4m3": (4, -6, 448.0),
}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values once, to nearest-even, onto the grid of `dtype`.

    Returns fp64 values that the dtype represents exactly (so the result is the
    exact value of the stored tensor).  Subnormals are kept; overflow goes to inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16" and x.size > 4096:
        return _round_bf16_fast(x)
    return _round_general(x, dtype)


def _round_general(x: np.ndarray, dtype: str) -> np.ndarray:
    p, emin, big = _FORMATS[dtype]
    _, e = np.frexp(x)  # |x| in [2^(e-1), 2^e)
    sh = np.maximum(e.astype(np.int64) - p, emin - p + 1)
    r = np.ldexp(np.round(np.ldexp(x, -sh)), sh)  # np.round: ties to even
    r = np.where(np.abs(r) > big, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), x, r)


def _round_bf16_fast(x: np.ndarray) -> np.ndarray:
    """Same result as _round_general(x, "bf16"), by integer rounding of the fp64 bits.

    In bf16's normal range, keeping the top 7 of fp64's 52 fraction bits with
    round-half-even is: add 2^44 - 1 plus the lowest kept bit, clear the 45 low bits
    (a carry correctly bumps the exponent).  Values outside that range go through
    the general path.
    """
    flat = np.ascontiguousarray(x).reshape(-1)
    out = np.empty_like(flat)
    lo, hi = 2.0 ** -126, float.fromhex("0x1.fep127")
    keep = np.uint64(~((1 << 45) - 1) & 0xFFFFFFFFFFFFFFFF)

    def work(a, b):
        xs = flat[a:b]
        bits = xs.view(np.uint64)
        lsb = (bits >> np.uint64(45)) & np.uint64(1)
        r = ((bits + (np.uint64((1 << 44) - 1) + lsb)) & keep).view(np.float64)
        ax = np.abs(xs)
        odd = ~((ax >= lo) & (ax <= hi))
        if odd.any():
            r = np.where(odd, _round_general(xs, "bf16"), r)
        out[a:b] = r

    _chunked(flat.size, 1 << 20, work)
    return out.reshape(x.shape)


def to_storage(x_rounded: np.ndarray, dtype: str) -> np.ndarray:
    """Pack values already on the dtype grid into their storage array.

    bf16 is returned as int16 bit patterns (numpy has no bf16), f16 as float16,
    f32 as float32.
    """
    if dtype == "f64":
        return np.ascontiguousarray(x_rounded, dtype=np.float64)
    if dtype == "f32":
        return x_rounded.astype(np.float32)
    if dtype == "f16":
        return x_rounded.astype(np.float16)
    if dtype == "bf16":
        bits = x_rounded.astype(np.float32).view(np.uint32) >> np.uint32(16)
        return bits.astype(np.uint16).view(np.int16)
    if dtype == "e4m3":
        return _e4m3_codes(x_rounded)
    raise ValueError(dtype)


def _e4m3_codes(r: np.ndarray) -> np.ndarray:
    """uint8 codes of values already on the e4m3 grid (finite, |r| <= 448)."""
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    if not (np.isfinite(a).all() and (a <= 448.0).all()):
        raise ValueError("e4m3 values must be finite and at most 448 in magnitude")
    m, e = np.frexp(a)                        # a = m 2^e, m in [0.5, 1)
    normal = a >= 2.0 ** -6
    E = np.where(normal, e.astype(np.int64) + 6, 0)
    F = np.where(normal, (2.0 * m - 1.0) * 8.0, a * 2.0 ** 9)
    if not np.array_equal(F, np.round(F)):
        raise ValueError("value not on the e4m3 grid")
    sign = np.signbit(r).astype(np.int64) << 7
    return (sign | (E << 3) | F.astype(np.int64)).astype(np.uint8)


def _e4m3_values(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c).view(np.uint8).astype(np.int64)
    E, F = (c >> 3) & 15, c & 7
    v = np.where(E == 0, F * 2.0 ** -9, (1.0 + F / 8.0) * np.exp2(E - 7.0))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return np.where(c & 0x80, -v, v)


def quantize_e4m3(x: np.ndarray) -> tuple[np.ndarray, float]:
    """Per-tensor e4m3 quantisation (module docstring): returns (codes, descale)."""
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    y = np.clip(x / descale, -448.0, 448.0)
    return _e4m3_codes(round_to_dtype(y, "e4m3")), descale


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a storage array produced by `to_storage`."""
    if dtype == "bf16":
        u32 = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return _e4m3_values(a)
    return a.astype(np.float64)


@dataclass
class AttentionInputs:
    """One seeded problem: storage arrays plus everything needed to describe it."""
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: float          # an fp32 value, held as a Python float
    seed: int
    q: np.ndarray         # storage arrays, shapes [B,Hq,N,d] / [B,Hkv,N,d]
    k: np.ndarray
    v: np.ndarray
    recipe: str = ""
    extra: dict = field(default_factory=dict)
    descale: tuple | None = None   # e4m3 inputs: (q, k, v) descales

    def f64(self, name: str) -> np.ndarray:
        x = storage_to_f64(getattr(self, name), self.dtype)
        if self.descale is not None:
            x *= self.descale["qkv".index(name)]
        return x

    @property
    def flops(self) -> float:
        """4*B*Hq*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str,
                causal: bool, scale: float | None = None, mult: float = 1.0,
                q_head_bias: bool = False, recipe: str = "") -> AttentionInputs:
    """Draw Q, K, V for one problem in the module's fill order and round them."""
    st = Stream(seed)
    shp_q, shp_kv = (B, Hq, N, d), (B, Hkv, N, d)
    q = st.normals(int(np.prod(shp_q))).reshape(shp_q)
    k = st.normals(int(np.prod(shp_kv))).reshape(shp_kv)
    v = st.normals(int(np.prod(shp_kv))).reshape(shp_kv)
    extra = {}
    if mult != 1.0:
        q *= mult
        k *= mult
        v *= mult
    if q_head_bias:
        beta = 2.0 * st.uniforms(Hq)
        q += beta[None, :, None, None]
        extra["q_head_bias"] = beta
    out, descale = [], None
    if dtype == "e4m3":
        descale = []
        for x in (q, k, v):
            codes, ds = quantize_e4m3(x)
            out.append(codes)
            descale.append(ds)
        descale = tuple(descale)
    else:
        for x in (q, k, v):
            out.append(to_storage(round_to_dtype(x, dtype), dtype))
            del x
    return AttentionInputs(B, Hq, Hkv, N, d, dtype, bool(causal),
                           default_scale(d) if scale is None else float(np.float32(scale)),
                           int(seed), out[0], out[1], out[2], recipe, extra, descale)


def make_normal(seed: int, shape, dtype: str, mult: float = 1.0) -> np.ndarray:
    """Seeded N(0,1) draws (times mult) of `shape`, rounded to dtype, as storage."""
    st = Stream(seed)
    g = st.normals(int(np.prod(shape))).reshape(shape)
    if mult != 1.0:
        g *= mult
    return to_storage(round_to_dtype(g, dtype), dtype)


def make_grad_output(seed: int, shape, dtype: str, mult: float = 1.0) -> np.ndarray:
    """A seeded upstream gradient dL/dO (see make_normal)."""
    return make_normal(seed, shape, dtype, mult)


# The six measured workloads.  Shapes follow the pages' layers: a 4096-token
# Llama-7B layer (32 heads of 128), BERT-large at sequence 512, 32/8 grouped-query
# heads, and long contexts with inputs scaled by 3 to exercise the rescaling.
WORKLOADS = {
    "f32_h1_n128_d64": dict(seed=1001, B=1, Hq=1, Hkv=1, N=128, d=64, dtype="f32",
                            causal=False, tuning=(32, 32)),
    "bf16_h32_n4096_d128_causal": dict(seed=1002, B=1, Hq=32, Hkv=32, N=4096, d=128,
                                       dtype="bf16", causal=True),
    "f16_b16_h16_n512_d64_qbias": dict(seed=1003, B=16, Hq=16, Hkv=16, N=512, d=64,
                                       dtype="f16", causal=False, q_head_bias=True),
    "bf16_gqa_b4_hq32_hkv8_n8192_d128_causal": dict(seed=1004, B=4, Hq=32, Hkv=8,
                                                    N=8192, d=128, dtype="bf16",
                                                    causal=True),
    "bf16_h16_n32768_d128_causal_x3": dict(seed=1005, B=1, Hq=16, Hkv=16, N=32768,
                                           d=128, dtype="bf16", causal=True, mult=3.0),
    "bf16_h8_n8192_d256_causal_x3": dict(seed=1006, B=1, Hq=8, Hkv=8, N=8192, d=256,
                                         dtype="bf16", causal=True, mult=3.0),
    # Few heads, long context: too few query tiles to fill the GPU without split-KV.
    "bf16_h2_n16384_d128_causal": dict(seed=1007, B=1, Hq=2, Hkv=2, N=16384, d=128,
                                       dtype="bf16", causal=True),
    # The 4096-token layer with e4m3 inputs and per-tensor descales.
    "e4m3_h32_n4096_d128_causal": dict(seed=1008, B=1, Hq=32, Hkv=32, N=4096, d=128,
                                       dtype="e4m3", causal=True),
}


@dataclass
class DecodeInputs:
    """Nq new queries per head against an Nk-row key/value cache (storage arrays)."""
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    scale: float
    seed: int
    q: np.ndarray         # [B, Hq, Nq, d]
    k: np.ndarray         # [B, Hkv, Nk, d]
    v: np.ndarray
    recipe: str = ""

    def f64(self, name: str) -> np.ndarray:
        return storage_to_f64(getattr(self, name), self.dtype)

    @property
    def flops(self) -> float:
        """4*d per visible (query, key) pair."""
        if self.causal:
            pairs = sum(self.Nk - self.Nq + i + 1 for i in range(self.Nq))
        else:
            pairs = self.Nq * self.Nk
        return 4.0 * self.B * self.Hq * pairs * self.d


def make_decode_inputs(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                       dtype: str, causal: bool = True, scale: float | None = None,
                       recipe: str = "") -> DecodeInputs:
    """Draw Q, then K, then V (normal, row-major) and round each once to dtype."""
    st = Stream(seed)
    q = st.normals(B * Hq * Nq * d).reshape(B, Hq, Nq, d)
    k = st.normals(B * Hkv * Nk * d).reshape(B, Hkv, Nk, d)
    v = st.normals(B * Hkv * Nk * d).reshape(B, Hkv, Nk, d)
    out = [to_storage(round_to_dtype(x, dtype), dtype) for x in (q, k, v)]
    return DecodeInputs(B, Hq, Hkv, Nq, Nk, d, dtype, bool(causal),
                        default_scale(d) if scale is None else float(np.float32(scale)),
                        int(seed), out[0], out[1], out[2], recipe)


# Decoding workloads: one new token per sequence against a long cache, grouped-query
# heads 32/8 (the pages' GQA example), batch 8.
DECODE_WORKLOADS = {
    "bf16_decode_b8_hq32_hkv8_nk8192_d128": dict(seed=1009, B=8, Hq=32, Hkv=8, Nq=1, Nk=8192,
                                                 d=128, dtype="bf16", causal=True),
    "bf16_decode_b1_hq32_hkv8_nk32768_d128": dict(seed=1010, B=1, Hq=32, Hkv=8, Nq=1, Nk=32768,
                                                  d=128, dtype="bf16", causal=True),
}


def workload(name: str):
    """Generate one of the named workloads (may take seconds for the large ones)."""
    if name in DECODE_WORKLOADS:
        return make_decode_inputs(recipe=name, **DECODE_WORKLOADS[name])
    w = dict(WORKLOADS[name])
    w.pop("tuning", None)
    return make_inputs(recipe=name, **w)
