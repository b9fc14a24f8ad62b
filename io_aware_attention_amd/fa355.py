"""ctypes binding of libfa355 -- argument marshalling only.

Every step of the attention forward and backward passes runs in the library's HIP
kernels; this
module only turns torch tensors into pointers, sizes and a stream, and turns
status codes into exceptions.  torch provides device memory and streams.  If the
built library is missing, importing the binding's functions raises: there is no
fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa355.so")
# The debug build of the same sources (LDS stages filled with NaN bytes before each
# refill, no overlap of staging with compute): must give the same bits.
LDS_POISON_LIB_PATH = os.path.join(HERE, "libfa355_lds_poison.so")

F32, F16, BF16 = 0, 1, 2
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_ARG, ERR_HIP = 0, -1, -2, -3, -4, -5, -6

# Every exported symbol, as declared in include/fa355.h.
EXPORTS = ("fa_fwd", "fa_fwd_ex", "fa_fwd_check", "fa_fwd_split", "fa_fwd_bias", "fa_bwd",
           "fa_fwd_fp8", "fa_fwd_decode", "fa_fwd_decode_noalloc", "fa_status_str",
           "fa_version")


class FA355Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fa355 error {status}: {msg}")
        self.status = status


class Tuning(ctypes.Structure):
    _fields_ = [("br", ctypes.c_int), ("bc", ctypes.c_int)]


class Plan(ctypes.Structure):
    _fields_ = [("br", ctypes.c_int), ("bc", ctypes.c_int), ("waves", ctypes.c_int),
                ("grid", ctypes.c_int), ("lds_bytes", ctypes.c_int)]


_lib = None


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise FA355Error(ERR_HIP, f"{path} is not built; run "
                         "`python -m io_aware_attention_amd.build` first")
    L = ctypes.CDLL(path)
    vp, ip, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    common = [vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, fp]
    L.fa_fwd.argtypes = common + [ip, vp]
    L.fa_fwd.restype = ip
    L.fa_fwd_ex.argtypes = common + [ip, ip, ctypes.POINTER(Tuning), vp]
    L.fa_fwd_ex.restype = ip
    L.fa_fwd_check.argtypes = common + [ip, ip, ctypes.POINTER(Tuning), ctypes.POINTER(Plan)]
    L.fa_fwd_check.restype = ip
    L.fa_fwd_split.argtypes = common + [ip, ip, vp, vp, vp]
    L.fa_fwd_split.restype = ip
    ll = ctypes.c_longlong
    L.fa_fwd_bias.argtypes = [vp, vp, vp, vp, vp, vp, ll, ll, ll] + [ip] * 6 + [fp, ip, vp]
    L.fa_fwd_bias.restype = ip
    L.fa_bwd.argtypes = [vp] * 10 + [ip, ip, ip, ip, ip, ip, fp, ip, vp]
    L.fa_bwd.restype = ip
    L.fa_fwd_fp8.argtypes = common + [fp, fp, fp, vp]
    L.fa_fwd_fp8.restype = ip
    L.fa_fwd_decode.argtypes = [vp] * 5 + [ip] * 7 + [fp, ip, ip, vp, vp, vp]
    L.fa_fwd_decode.restype = ip
    L.fa_fwd_decode_noalloc.argtypes = [vp] * 5 + [ip] * 7 + [fp, ip, ip, vp]
    L.fa_fwd_decode_noalloc.restype = ip
    L.fa_status_str.argtypes = [ip]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = ip
    return L


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Routes this module's calls to another build of the library (e.g. the LDS
    poison debug build) inside the `with` block.  Not thread-safe."""
    global _lib
    prev = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def _check(rc: int):
    if rc != OK:
        raise FA355Error(rc, status_str(rc))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t not in codes:
        raise FA355Error(ERR_UNSUPPORTED, f"dtype {t} not supported")
    return codes[t]


def _tuning(tuning):
    if tuning is None:
        return None
    br, bc = tuning
    return ctypes.byref(Tuning(int(br), int(bc)))


def _qkv_shapes(q, k, v, same_len: bool = True):
    """(B, Hq, Hkv, N, Nk, d) of 4-D q [B,Hq,N,d] and k, v [B,Hkv,Nk,d] that agree in
    B and d (and N = Nk when same_len), with one dtype; FA355Error otherwise."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FA355Error(ERR_SHAPE, "q, k, v must be 4-D [B,H,N,d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape) or (same_len and Nk != N):
        raise FA355Error(ERR_SHAPE, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise FA355Error(ERR_UNSUPPORTED, "q, k, v must share a dtype")
    return B, Hq, Hkv, N, Nk, d


def _given(name, t, shape, dtype):
    """A caller-provided output or workspace must have exactly this shape and dtype
    and be contiguous (the library writes it as a dense array of that size)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise FA355Error(ERR_ARG, f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} (got {t.dtype} {tuple(t.shape)})")


def _on_device(device, **tensors):
    """Every tensor handed to the library is a contiguous tensor on `device`."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.device != device:
            raise FA355Error(ERR_ARG, f"{name} must be a contiguous tensor on {device}")


def plan(B, Hq, Hkv, N, d, causal, dtype, out_dtype=None, tuning=None, scale=None) -> Plan:
    """The launch fa_fwd_ex would make for these sizes (no GPU needed)."""
    dt = _dtype_code(dtype)
    odt = dt if out_dtype is None else _dtype_code(out_dtype)
    p = Plan()
    fake = 1 << 40  # distinct, 16-byte-aligned host addresses: only compared, never read
    span = B * max(Hq, Hkv) * N * d * 8 + 4096
    rc = lib().fa_fwd_check(fake, fake + span, fake + 2 * span, fake + 3 * span,
                            fake + 4 * span, B, Hq, Hkv, N, d, int(bool(causal)),
                            float(1.0 / math.sqrt(d) if scale is None else scale),
                            dt, odt, _tuning(tuning), ctypes.byref(p))
    _check(rc)
    return p


def fwd(q, k, v, causal: bool = False, scale: float | None = None, *, out_dtype=None,
        o=None, lse=None, return_lse: bool = True, tuning=None, stream=None):
    """Attention forward on torch device tensors.

    q: [B,Hq,N,d]; k, v: [B,Hkv,N,d]; all contiguous, same dtype (fp32, fp16 or
    bf16).  scale defaults to 1/sqrt(d).  out_dtype may be torch.float32 for 16-bit
    inputs.  o / lse may be given (preallocated); otherwise they are allocated
    with torch.  tuning is an optional (br, bc).  Returns (o, lse) (lse is None when
    return_lse is False).  The kernel runs on `stream` (default: torch's current
    stream); the call returns once it is enqueued.
    """
    import torch
    L = lib()
    B, Hq, Hkv, N, _, d = _qkv_shapes(q, k, v)
    dt = _dtype_code(q.dtype)
    odt_t = q.dtype if out_dtype is None else out_dtype
    odt = _dtype_code(odt_t)
    _given("o", o, (B, Hq, N, d), odt_t)
    _given("lse", lse, (B, Hq, N), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if o is None:
        o = torch.empty((B, Hq, N, d), dtype=odt_t, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                     None if lse is None else lse.data_ptr(),
                     B, Hq, Hkv, N, d, int(bool(causal)), float(scale), dt, odt,
                     _tuning(tuning), ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, *,
        dq=None, dk=None, dv=None, delta=None, stream=None):
    """Attention backward on torch device tensors: returns (dq, dk, dv), fp32.

    q, o, dout: [B,Hq,N,d]; k, v: [B,Hkv,N,d]; all contiguous, one 16-bit dtype.
    lse: [B,Hq,N] fp32 from the forward pass with the same causal flag and scale.
    dq / dk / dv / delta (the [B,Hq,N] fp32 workspace) may be preallocated.
    """
    import torch
    L = lib()
    B, Hq, Hkv, N, _, d = _qkv_shapes(q, k, v)
    for name, t in (("o", o), ("dout", dout)):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype:
            raise FA355Error(ERR_SHAPE, f"{name} must match q in shape and dtype")
    if tuple(lse.shape) != (B, Hq, N) or lse.dtype != torch.float32:
        raise FA355Error(ERR_SHAPE, "lse must be fp32 [B,Hq,N]")
    _given("dq", dq, (B, Hq, N, d), torch.float32)
    _given("dk", dk, (B, Hkv, N, d), torch.float32)
    _given("dv", dv, (B, Hkv, N, d), torch.float32)
    _given("delta", delta, (B, Hq, N), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, Hq, N, d), **f32) if dq is None else dq
    dk = torch.empty((B, Hkv, N, d), **f32) if dk is None else dk
    dv = torch.empty((B, Hkv, N, d), **f32) if dv is None else dv
    delta = torch.empty((B, Hq, N), **f32) if delta is None else delta
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                  B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _dtype_code(q.dtype),
                  ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return dq, dk, dv


def split_count(B: int, Hq: int, N: int, causal: bool, cus: int = 256, d: int = 128) -> int:
    """A split count that fills the GPU: about two workgroups per compute unit at
    head dim 128 (256-row tiles, one resident per CU) and four at 64 (128-row
    tiles), keeping at least four 64-key blocks per split (1 = no split).  On
    B1 H2 N16384 d128 causal this picks 4; 3 to 6 measured within 2 % of each other.
    Without a mask, once the query tiles alone fill the GPU a split only adds the
    partial results' round trip (B1 H8 N8192 d128: 256 us unsplit, 269 us in two
    pieces), so it picks 1; causal tiles of unequal length still gain (B2 H8 N4096
    d128 causal: 125 us unsplit, 97 us in two pieces)."""
    rows, per_cu = (256, 2) if d == 128 else (128, 4)
    tiles = B * Hq * ((N + rows - 1) // rows)
    if tiles == 0:                      # an empty call: nothing to split
        return 1
    if not causal and tiles >= cus:
        return 1
    want = -(-per_cu * cus // tiles)
    blocks = (N + 63) // 64
    return max(1, min(16, want, blocks // 4))


def fwd_split(q, k, v, causal: bool = False, scale: float | None = None, num_splits=None, *,
              o=None, lse=None, o_part=None, lse_part=None, stream=None):
    """Split-KV attention forward (16-bit inputs, d = 64 or 128): returns (o, lse).

    num_splits defaults to split_count(); the fp32 workspaces o_part
    [S,B,Hq,N,d] and lse_part [S,B,Hq,N] are allocated with torch unless given.
    """
    import torch
    L = lib()
    B, Hq, Hkv, N, _, d = _qkv_shapes(q, k, v)
    _dtype_code(q.dtype)
    if num_splits is None:
        num_splits = split_count(B, Hq, N, causal, d=d)
    S = int(num_splits)
    if S < 1:
        raise FA355Error(ERR_ARG, f"num_splits must be >= 1 (got {S})")
    _given("o", o, (B, Hq, N, d), q.dtype)
    _given("lse", lse, (B, Hq, N), torch.float32)
    _given("o_part", o_part, (S, B, Hq, N, d), torch.float32)
    _given("lse_part", lse_part, (S, B, Hq, N), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, o_part=o_part, lse_part=lse_part)
    f32 = dict(dtype=torch.float32, device=q.device)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, N), **f32) if lse is None else lse
    o_part = torch.empty((S, B, Hq, N, d), **f32) if o_part is None else o_part
    lse_part = torch.empty((S, B, Hq, N), **f32) if lse_part is None else lse_part
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _dtype_code(q.dtype),
                        S, o_part.data_ptr(), lse_part.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse


def fwd_bias(q, k, v, bias, causal: bool = False, scale: float | None = None, *, o=None,
             lse=None, stream=None):
    """Attention forward with an additive bias: softmax(Q K^T scale + bias) V.

    bias: a tensor of q's dtype that broadcasts to [B,Hq,N,N] (size-1 leading
    dimensions are shared); its last dimension must be contiguous.  A layout whose
    strides are not multiples of 4 elements is first copied to a padded one.
    Returns (o, lse).
    """
    import torch
    L = lib()
    B, Hq, Hkv, N, _, d = _qkv_shapes(q, k, v)
    _dtype_code(q.dtype)
    _given("o", o, (B, Hq, N, d), q.dtype)
    _given("lse", lse, (B, Hq, N), torch.float32)
    if bias.dim() != 4 or tuple(bias.shape[2:]) != (N, N) or bias.shape[0] not in (1, B) \
            or bias.shape[1] not in (1, Hq) or bias.dtype != q.dtype or bias.stride(3) != 1:
        raise FA355Error(ERR_SHAPE, f"bias {tuple(bias.shape)} does not fit [B,Hq,N,N] of q's dtype")
    if bias.stride(2) % 4 or (bias.shape[1] > 1 and bias.stride(1) % 4) or \
            (bias.shape[0] > 1 and bias.stride(0) % 4) or bias.data_ptr() % 8:
        # The kernel reads four keys per 8-byte load: give rows a stride that is a
        # multiple of 4 elements (a padded copy).
        Np = (N + 3) // 4 * 4
        padded = torch.zeros(tuple(bias.shape[:3]) + (Np,), dtype=bias.dtype, device=bias.device)
        padded[..., :N] = bias
        bias = padded[..., :N]
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if not bias.is_cuda or bias.device != q.device:
        raise FA355Error(ERR_ARG, f"bias must be a tensor on {q.device}")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    sh = 0 if bias.shape[1] == 1 else bias.stride(1)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       bias.data_ptr(), sb, sh, bias.stride(2), B, Hq, Hkv, N, d,
                       int(bool(causal)), float(scale), _dtype_code(q.dtype),
                       ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse


def fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
            causal: bool = False, scale: float | None = None, *, o=None, lse=None,
            stream=None):
    """Attention forward on e4m3 inputs: returns (o bf16, lse fp32).

    q: [B,Hq,N,d]; k, v: [B,Hkv,N,d]; contiguous device tensors of e4m3 codes
    (torch.uint8 or torch.float8_e4m3fn), d = 64 or 128.  The value of each element
    is its tensor's descale times the code's e4m3 value.
    """
    import torch
    L = lib()
    B, Hq, Hkv, N, _, d = _qkv_shapes(q, k, v)
    ok = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if q.dtype not in ok:
        raise FA355Error(ERR_UNSUPPORTED, "q, k, v must hold e4m3 codes (uint8 or float8_e4m3fn)")
    _given("o", o, (B, Hq, N, d), torch.bfloat16)
    _given("lse", lse, (B, Hq, N), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse)
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q.device) if o is None else o
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, Hq, Hkv, N, d, int(bool(causal)), float(scale), float(q_descale),
                      float(k_descale), float(v_descale), ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse


def decode_split_count(B: int, Hkv: int, Nk: int, cus: int = 256) -> int:
    """Key-range pieces for fwd_decode: about 512 keys per piece, but at least one
    workgroup per compute unit; each piece at least four 32-key blocks, at most 256
    pieces.  (Measured on MI355X: B8 Hkv8 Nk8192 best at 16 pieces, B1 Hkv8 Nk32768
    at 32-64; fewer keys per piece lose to the per-piece set-up and merge.)  When the
    (batch, K/V head) pairs alone fill the GPU, about two workgroups per compute
    unit: B32 Hkv8 Nk4096 runs 97 us in 2 pieces against 104 in 8, B64 Hkv8 Nk2048
    103 us unsplit against 108 in 4."""
    blocks = (Nk + 31) // 32
    units = B * Hkv
    if units == 0 or blocks == 0:       # an empty call or an empty cache: one piece
        return 1
    if units >= cus:
        want = -(-2 * cus // units)
    else:
        want = max(-(-blocks // 16), -(-cus // units))
    return max(1, min(256, want, blocks // 4))


def fwd_decode(q, k, v, causal: bool = True, scale: float | None = None, num_splits=None, *,
               o=None, lse=None, o_part=None, lse_part=None, stream=None):
    """Decoding against a key/value cache: returns (o, lse).

    q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d] (the cache, new positions included); one
    16-bit dtype, d = 64 or 128, (Hq/Hkv)*Nq <= 32.  causal: query i sees keys
    j <= i + Nk - Nq.  num_splits defaults to decode_split_count(); the fp32
    workspaces are allocated with torch unless given.
    """
    import torch
    L = lib()
    B, Hq, Hkv, Nq, Nk, d = _qkv_shapes(q, k, v, same_len=False)
    _dtype_code(q.dtype)
    S = int(decode_split_count(B, Hkv, Nk) if num_splits is None else num_splits)
    if S < 1:
        raise FA355Error(ERR_ARG, f"num_splits must be >= 1 (got {S})")
    _given("o", o, (B, Hq, Nq, d), q.dtype)
    _given("lse", lse, (B, Hq, Nq), torch.float32)
    _given("o_part", o_part, (S, B, Hq, Nq, d), torch.float32)
    _given("lse_part", lse_part, (S, B, Hq, Nq), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, o_part=o_part, lse_part=lse_part)
    f32 = dict(dtype=torch.float32, device=q.device)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Nq), **f32) if lse is None else lse
    o_part = torch.empty((S, B, Hq, Nq, d), **f32) if o_part is None else o_part
    lse_part = torch.empty((S, B, Hq, Nq), **f32) if lse_part is None else lse_part
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale), _dtype_code(q.dtype),
                         S, o_part.data_ptr(), lse_part.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse


# Size of the library's own decoding workspace on each GPU (fa_fwd_decode_noalloc).
NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc_bytes(B: int, Hq: int, Nq: int, d: int, num_splits: int) -> int:
    """Workspace bytes fwd_decode_noalloc needs: the fp32 partial outputs rounded up
    to 256 bytes, then the fp32 partial lse values."""
    rows = num_splits * B * Hq * Nq
    return (rows * d * 4 + 255) // 256 * 256 + rows * 4


def fwd_decode_noalloc(q, k, v, o, lse=None, causal: bool = True, scale: float | None = None,
                       num_splits=None, *, stream=None):
    """fwd_decode writing into the caller's o (and lse, if given) with the partial
    results in the library's static per-GPU workspace: neither the library nor this
    binding allocates device memory.  Calls that overlap in time on one GPU share
    that workspace and race.  Returns (o, lse)."""
    import torch
    L = lib()
    B, Hq, Hkv, Nq, Nk, d = _qkv_shapes(q, k, v, same_len=False)
    _dtype_code(q.dtype)
    S = int(decode_split_count(B, Hkv, Nk) if num_splits is None else num_splits)
    if S < 1:
        raise FA355Error(ERR_ARG, f"num_splits must be >= 1 (got {S})")
    if o is None:
        raise FA355Error(ERR_ARG, "fwd_decode_noalloc writes into a given o")
    _given("o", o, (B, Hq, Nq, d), q.dtype)
    _given("lse", lse, (B, Hq, Nq), torch.float32)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    rc = L.fa_fwd_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 None if lse is None else lse.data_ptr(),
                                 B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                 _dtype_code(q.dtype), S, ctypes.c_void_p(s.cuda_stream))
    _check(rc)
    return o, lse
