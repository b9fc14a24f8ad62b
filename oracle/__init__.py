"""fp64 CPU oracle of attention, forward and gradients -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The product library never does, and this
package imports nothing from it: the two share no code.  Inputs reach both sides
from ``fa_inputs`` (seeded draws only).

Two independent C implementations sit behind these wrappers:

* ``attention`` / ``probs`` -- the plain definition softmax(Q K^T * scale) V with a
  two-pass softmax over materialised score rows (attention_oracle.c);
  ``attention_kv`` the same for queries against a longer key/value sequence;
* ``blocked`` -- the tiled online-softmax merge equations, key/value blocks outer,
  query blocks inner, per-row state (blocked_reference.c);
* ``grads`` -- dQ, dK, dV of the plain definition by the chain rule, one softmax
  row at a time (attention_grad_oracle.c).

Every function here is pinned by tests against things other than itself (high
precision brute force, closed forms, invariants, torch's own attention routine).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ("attention_oracle.c", "blocked_reference.c", "attention_grad_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
CFLAGS = ("-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread")

_lib = None


def build(out: str = LIB_PATH, sources: tuple[str, ...] | None = None) -> str:
    """Compile the oracle sources with gcc into a shared library at `out`."""
    srcs = [s if os.path.isabs(s) else os.path.join(HERE, s) for s in (sources or SOURCES)]
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, *srcs, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load a built oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp, i64, ip = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_attention_fwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                         ip, ctypes.c_double, dp, i64, ip]
    lib.oracle_attention_fwd.restype = ip
    lib.oracle_attention_probs.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, ip,
                                           ctypes.c_double]
    lib.oracle_attention_probs.restype = ip
    lib.blocked_attention_fwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                          ip, ctypes.c_double, i64, i64]
    lib.blocked_attention_fwd.restype = ip
    lib.oracle_attention_fwd_bias.argtypes = [dp, dp, dp, dp, i64, i64, i64, dp, dp, i64, i64,
                                              i64, i64, i64, ip, ctypes.c_double, ip]
    lib.oracle_attention_fwd_bias.restype = ip
    lib.oracle_attention_fwd_kv.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                                            ip, ctypes.c_double, ip]
    lib.oracle_attention_fwd_kv.restype = ip
    lib.oracle_attention_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                         ip, ctypes.c_double, ip]
    lib.oracle_attention_bwd.restype = ip
    return lib


def _get(lib):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load()
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(q, k, v):
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or (v is not None and v.shape != k.shape):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    return B, Hq, Hkv, N, d


def attention(q, k, v, causal: bool, scale: float, rows=None, threads: int = 0,
              lib=None):
    """Exact attention of fp64 inputs.

    q: [B,Hq,N,d]; k, v: [B,Hkv,N,d].  Returns (o, lse): o is [B,Hq,R,d] and lse
    [B,Hq,R], with R = N, or the given query rows in the given order.
    """
    L = _get(lib)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = N if r is None else len(r)
    o = np.empty((B, Hq, R, d), np.float64)
    lse = np.empty((B, Hq, R), np.float64)
    rc = L.oracle_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                _ptr(r), R, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attention_fwd failed with {rc}")
    return o, lse


def attention_kv(q, k, v, causal: bool, scale: float, threads: int = 0, lib=None):
    """Exact attention of Nq queries against Nk keys/values (decoding with a cache).

    q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]; when causal, Nq <= Nk and query i sees keys
    j <= i + Nk - Nq (the queries are the last Nq positions).  Returns (o, lse).
    """
    L = _get(lib)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    o = np.empty((B, Hq, Nq, d), np.float64)
    lse = np.empty((B, Hq, Nq), np.float64)
    rc = L.oracle_attention_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                   int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attention_fwd_kv failed with {rc}")
    return o, lse


def attention_bias(q, k, v, bias, causal: bool, scale: float, threads: int = 0, lib=None):
    """Exact attention with an additive bias on the scaled scores.

    bias broadcasts to [B,Hq,N,N] (leading dimensions of size 1 are shared).
    Rows whose every score is -inf give o = 0 and lse = -inf.  Returns (o, lse).
    """
    L = _get(lib)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    bias = np.asarray(bias, dtype=np.float64)
    if bias.ndim != 4 or bias.shape[2:] != (N, N) or bias.shape[0] not in (1, B) \
            or bias.shape[1] not in (1, Hq):
        raise ValueError(f"bias shape {bias.shape} does not broadcast to {(B, Hq, N, N)}")
    bias = np.ascontiguousarray(bias)
    sb = 0 if bias.shape[0] == 1 else bias.shape[1] * N * N
    sh = 0 if bias.shape[1] == 1 else N * N
    o = np.empty((B, Hq, N, d), np.float64)
    lse = np.empty((B, Hq, N), np.float64)
    rc = L.oracle_attention_fwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), sb, sh, N,
                                     _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
                                     float(scale), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attention_fwd_bias failed with {rc}")
    return o, lse


def probs(q, k, causal: bool, scale: float, lib=None) -> np.ndarray:
    """The softmax matrix P, [B,Hq,N,N], zeros where masked (small inputs only)."""
    L = _get(lib)
    q, k = _f64(q), _f64(k)
    B, Hq, Hkv, N, d = _shapes(q, k, None)
    p = np.empty((B, Hq, N, N), np.float64)
    rc = L.oracle_attention_probs(_ptr(q), _ptr(k), _ptr(p), B, Hq, Hkv, N, d,
                                  int(bool(causal)), float(scale))
    if rc != 0:
        raise ValueError(f"oracle_attention_probs failed with {rc}")
    return p


def blocked(q, k, v, causal: bool, scale: float, br: int, bc: int, lib=None):
    """The tiled online-softmax reference with Br x Bc tiles.  Returns (o, lse)."""
    L = _get(lib)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    o = np.empty((B, Hq, N, d), np.float64)
    lse = np.empty((B, Hq, N), np.float64)
    rc = L.blocked_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                 int(br), int(bc))
    if rc != 0:
        raise ValueError(f"blocked_attention_fwd failed with {rc}")
    return o, lse


def grads(q, k, v, dout, causal: bool, scale: float, threads: int = 0, lib=None):
    """Gradients of sum(O * dout) for O = attention(q, k, v): returns (dq, dk, dv).

    q, dout: [B,Hq,N,d]; k, v: [B,Hkv,N,d]; outputs have the shapes of q, k, v.
    """
    L = _get(lib)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError(f"dout shape {dout.shape} != q shape {q.shape}")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = L.oracle_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attention_bwd failed with {rc}")
    return dq, dk, dv
