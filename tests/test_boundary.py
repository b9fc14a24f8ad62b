"""The C ABI on the CPU: the library loads, exports every declared symbol, and its
validation rejects every bad argument before touching HIP (no GPU needed)."""
import ctypes
import os
import re

import pytest

import io_aware_attention_amd as F
from io_aware_attention_amd import fa355 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

BASE = 1 << 40      # fake, aligned, never dereferenced addresses
SPAN = 1 << 32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for path in (B.LIB_PATH, B.LDS_POISON_LIB_PATH):
        L = ctypes.CDLL(path)
        for n in names:
            assert hasattr(L, n), (path, n)


def test_version_and_status_strings():
    L = F.lib()
    assert L.fa_version() == 150
    for s in range(-6, 1):
        assert F.status_str(s) and F.status_str(s) != "unknown status"
    assert F.status_str(-99) == "unknown status"


def check(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
          B_=1, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.1, dt=F.BF16, odt=None,
          tuning=None):
    p = B.Plan()
    t = None if tuning is None else ctypes.byref(B.Tuning(*tuning))
    rc = F.lib().fa_fwd_check(q, k, v, o, lse, B_, Hq, Hkv, N, d, causal, scale, dt,
                              dt if odt is None else odt, t, ctypes.byref(p))
    return rc, p


def test_valid_call_plans_a_launch():
    rc, p = check(B_=1, Hq=32, Hkv=32, N=4096, d=128)
    assert rc == 0 and (p.br, p.bc, p.waves, p.grid) == (256, 64, 8, 512)
    # two stages of 16-byte slots: K rows of 16 + 1 pad slots (rounded up to whole
    # 64-slot (1 KB) DMA instructions), unpadded V rows of 16 slots
    ceil64 = lambda n: (n + 63) // 64 * 64
    assert p.lds_bytes == 2 * 16 * (ceil64(64 * 17) + 64 * 16) == 67584
    rc, p = check(B_=1, Hq=32, Hkv=32, N=2048, d=128)
    assert rc == 0 and (p.br, p.bc, p.waves, p.grid) == (128, 64, 4, 512)
    assert p.lds_bytes == 2 * 16 * (ceil64(64 * 17) + 64 * 16) == 67584
    rc, p = check(B_=1, Hq=32, Hkv=32, N=2048, d=128, tuning=(128, 32))
    assert p.lds_bytes == 2 * 16 * (ceil64(32 * 17) + 32 * 16) == 34816
    rc, p = check(B_=4, Hq=32, Hkv=8, N=8192)
    assert rc == 0 and (p.br, p.bc, p.grid) == (256, 64, 4 * 32 * 32)
    rc, p = check(B_=1, Hq=1, Hkv=1, N=128, d=64, dt=F.F32, tuning=(32, 32))
    assert rc == 0 and (p.br, p.bc, p.grid) == (32, 32, 4)
    rc, p = check(d=256, N=8192, Hq=8, Hkv=8)
    assert rc == 0 and (p.br, p.bc) == (128, 32)
    # Head dim 256 by default: eight wavefronts split by role; three stages of 32-key
    # blocks, P operands of four groups in two buffers (16 KB), rescale factors
    # (1 KB) and flags (32 B), final row sums (512 B).
    ceil64 = lambda n: (n + 63) // 64 * 64
    stage32 = 16 * (ceil64(32 * 33) + 32 * 32)
    assert p.waves == 8 and p.lds_bytes == 3 * stage32 + 16384 + 1024 + 32 + 512 == 119328
    # The wavefront pairs at 128 x 64: two stages, the pairs' P operands (16 KB),
    # block maxima and row sums (2 x 1 KB), rescale flags (32 B).
    rc, p = check(d=256, N=8192, Hq=8, Hkv=8, tuning=(128, 64))
    stage = 16 * (ceil64(64 * 33) + 64 * 32)
    assert rc == 0 and p.waves == 8 and p.lds_bytes == 2 * stage + 16384 + 2048 + 32 == 151584
    # d = 64: fp16 takes 128 x 32 for short rows, 256 x 64 without a mask from 2048 and
    # 128 x 64 with one from 4096; bf16 takes 256 x 64, except causal rows below 2048.
    f16 = lambda N, c: (check(d=64, N=N, dt=F.F16, causal=c)[1].br, check(d=64, N=N, dt=F.F16, causal=c)[1].bc)
    assert f16(512, 0) == (128, 32) and f16(2047, 0) == (128, 32) and f16(2048, 0) == (256, 64)
    assert f16(512, 1) == (128, 32) and f16(4095, 1) == (128, 32) and f16(4096, 1) == (128, 64)
    assert (check(d=64, N=512, causal=0)[1].br, check(d=64, N=512, causal=0)[1].bc) == (256, 64)
    assert (check(d=64, N=2047, causal=1)[1].br, check(d=64, N=2047, causal=1)[1].bc) == (128, 32)
    assert (check(d=64, N=2048, causal=1)[1].br, check(d=64, N=2048, causal=1)[1].bc) == (256, 64)
    # d = 128: 256 x 64 from N = 4096, or from N = 2048 without a mask; 128 x 64 below.
    assert check(N=2048, causal=1)[1].br == 128 and check(N=2048, causal=0)[1].br == 256
    assert check(N=2047, causal=0)[1].br == 128 and check(N=4096, causal=1)[1].br == 256
    assert check(N=100, causal=1)[1].bc == 64 and check(N=4095, causal=1)[1].bc == 64
    rc, p = check(lse=None)
    assert rc == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B_=-1), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Hq=-2, Hkv=-1), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(N=-5), -2), (dict(N=1 << 30), -2),
    (dict(d=96), -3), (dict(d=32), -3), (dict(d=512), -3), (dict(dt=F.F32, d=128), -3),
    (dict(dt=7), -3), (dict(odt=F.F16), -3), (dict(dt=F.F32, d=64, odt=F.BF16), -3),
    (dict(tuning=(96, 64)), -3), (dict(tuning=(128, 48)), -3),
    # every launch stays below 2^32 work-items per grid dimension
    (dict(B_=1024, Hq=1024, Hkv=1024, N=2048, d=64, q=1 << 44, k=2 << 44, v=3 << 44, o=4 << 44,
          lse=5 << 44), -2),
    (dict(dt=F.F32, d=64, tuning=(128, 64)), -3),
    (dict(scale=float("inf")), -5), (dict(scale=float("nan")), -5),
    (dict(q=BASE + 2), -4), (dict(o=BASE + 3 * SPAN + 8), -4), (dict(lse=BASE + 4 * SPAN + 2), -4),
    (dict(o=BASE), -5), (dict(o=BASE + SPAN + 4096), -5), (dict(lse=BASE + 2 * SPAN + 64), -5),
    (dict(lse=BASE + 3 * SPAN), -5),
])
def test_rejections(kw, code):
    rc, _ = check(**kw)
    assert rc == code, (kw, rc)


def test_grid_work_item_limit():
    # 2^20 heads x 8 query tiles x 512 threads = 2^32 work-items: rejected; one head
    # fewer fits.  Pointers are spaced 2^44 bytes apart (the tensors are 2^38 bytes).
    far = dict(q=1 << 44, k=2 << 44, v=3 << 44, o=4 << 44, lse=5 << 44, N=2048, d=64)
    assert check(B_=1024, Hq=1024, Hkv=1024, **far)[0] == -2
    rc, p = check(B_=1024, Hq=1023, Hkv=1023, **far)
    assert rc == 0 and p.grid * 64 * p.waves < 1 << 32
    # Decoding: the merge launch has 256 work-items per (batch, head, query) row.
    L = F.lib()
    big = [ctypes.c_void_p(n << 44) for n in range(1, 8)]
    rows_limit = (1 << 32) // 256                      # 2^24 rows
    B_ = rows_limit // 32                              # Hq = 32, Nq = 1
    assert L.fa_fwd_decode(big[0], big[1], big[2], big[3], big[4], B_, 32, 1, 1, 64, 64, 1, 0.1,
                           F.BF16, 1, big[5], big[6], None) == -2
    # Backward: dQ, dK/dV and delta launches are held to the same limit.
    assert L.fa_bwd(*big[:5], ctypes.c_void_p(6 << 44), ctypes.c_void_p(8 << 44),
                    ctypes.c_void_p(9 << 44), ctypes.c_void_p(10 << 44), ctypes.c_void_p(11 << 44),
                    1 << 16, 1 << 10, 1 << 10, 256, 64, 1, 0.1, F.BF16, None) == -2


def test_empty_calls_return_ok_without_touching_anything():
    # No query rows: every entry point returns FA355_OK before any HIP call, with
    # NULL buffers; only the sizes are checked.
    L = F.lib()
    for B_, N in ((0, 100), (1, 0), (0, 0)):
        assert L.fa_fwd(None, None, None, None, None, B_, 4, 2, N, 128, 1, 0.1, F.BF16, None) == 0
        assert L.fa_fwd_ex(None, None, None, None, None, B_, 4, 2, N, 96, 1, 0.1, F.BF16, F.BF16,
                           None, None) == 0
        assert L.fa_bwd(None, None, None, None, None, None, None, None, None, None,
                        B_, 4, 2, N, 128, 1, 0.1, F.BF16, None) == 0
        assert L.fa_fwd_split(None, None, None, None, None, B_, 4, 2, N, 128, 1, 0.1, F.BF16, 0,
                              None, None, None) == 0
        assert L.fa_fwd_bias(None, None, None, None, None, None, 0, 0, 0, B_, 4, 2, N, 128, 1, 0.1,
                             F.BF16, None) == 0
        assert L.fa_fwd_fp8(None, None, None, None, None, B_, 4, 2, N, 128, 1, 0.1, 1.0, 1.0, 1.0,
                            None) == 0
        assert L.fa_fwd_decode(None, None, None, None, None, B_, 8, 2, N, 100, 128, 1, 0.1, F.BF16,
                               0, None, None, None) == 0
    # The plan of an empty call launches nothing.
    rc, p = check(q=None, k=None, v=None, o=None, lse=None, B_=0)
    assert rc == 0 and (p.br, p.bc, p.waves, p.grid, p.lds_bytes) == (0, 0, 0, 0, 0)
    # Sizes are still checked.
    assert check(q=None, B_=0, Hq=3, Hkv=2)[0] == -2
    assert check(q=None, B_=0, Hkv=0)[0] == -2
    assert check(q=None, N=0, B_=-1)[0] == -2
    assert L.fa_fwd_decode(None, None, None, None, None, 1, 8, 2, 0, -1, 128, 1, 0.1, F.BF16,
                           4, None, None, None) == -2
    assert L.fa_fwd_decode(None, None, None, None, None, 1, 8, 2, 0, 0, 128, 1, 0.1, F.BF16,
                           4, None, None, None) == 0


def test_largest_sizes_accepted_and_one_more_rejected():
    # One head of 16-bit K or V must fit 32-bit byte offsets with 64 KiB to spare.
    n_max = (2**31 - 1 - 65536) // 256                # d = 128: 8,388,351 rows
    assert check(B_=1, Hq=1, Hkv=1, N=n_max)[0] == 0
    assert check(B_=1, Hq=1, Hkv=1, N=n_max + 1)[0] == -2
    n64 = (2**31 - 1 - 65536) // 128
    assert check(B_=1, Hq=1, Hkv=1, N=n64, d=64)[0] == 0
    assert check(B_=1, Hq=1, Hkv=1, N=n64 + 1, d=64)[0] == -2
    # Decoding reads one 32-key block past the cache's end: n_max - 32 keys is the
    # largest cache (run on the GPU in test_gpu_maxsize.py); one more is rejected.
    assert decode_call(Nk=n_max - 32 + 1, Nq=2) == -2


def test_tensors_above_2_40_elements_are_too_large():
    # Byte extents of such tensors could wrap a 64-bit count; they are rejected as too
    # large before any extent is computed (not misreported as an overlap).
    far = 1 << 46                                     # fake tensors 64 TiB apart
    kw = dict(q=BASE, k=BASE + far, v=BASE + 2 * far, o=BASE + 3 * far, lse=BASE + 4 * far)
    assert check(**kw, B_=2048, Hq=4096, Hkv=4096, N=8192, d=128)[0] == -2      # 2^43
    assert check(**kw, B_=2**30, Hq=2**30, Hkv=2**30, N=4096, d=128)[0] == -2
    # Exactly 2^40 elements passes the size check, but its 2^25 workgroups of 512
    # work-items exceed a grid dimension's 2^32; with 64-bit extents the overlap
    # check still runs first (fake tensors 4 GiB apart overlap).
    assert check(**kw, B_=256, Hq=4096, Hkv=4096, N=8192, d=128)[0] == -2
    assert check(**kw, B_=2, Hq=4096, Hkv=4096, N=8192, d=128)[0] == 0        # 2^33 elements
    assert check(B_=256, Hq=4096, Hkv=4096, N=8192, d=128)[0] == -5            # 4 GiB apart: overlap
    L = F.lib()
    assert L.fa_fwd_bias(BASE, BASE + SPAN, BASE + 2 * SPAN, BASE + 3 * SPAN, BASE + 4 * SPAN,
                         BASE + 5 * SPAN, 2**62, 0, 128, 2, 4, 2, 100, 128, 1, 0.1, F.BF16, None) == -2
    assert L.fa_fwd_bias(BASE, BASE + SPAN, BASE + 2 * SPAN, BASE + 3 * SPAN, BASE + 4 * SPAN,
                         BASE + 5 * SPAN, 2**63 - 4, 2**63 - 4, 128, 1024, 4, 2, 100, 128, 1, 0.1,
                         F.BF16, None) == -2
    assert decode_call(B_=2**30, Hq=8, Hkv=8, Nq=1, Nk=8388000, S=256) == -2


def test_fwd_validates_before_any_hip_call():
    # Invalid arguments return their code from fa_fwd / fa_fwd_ex without a GPU.
    L = F.lib()
    assert L.fa_fwd(None, BASE, BASE, BASE, None, 1, 1, 1, 8, 128, 0, 1.0, F.BF16, None) == -1
    assert L.fa_fwd(BASE, BASE, BASE, BASE + SPAN, None, 1, 1, 1, 8, 96, 0, 1.0, F.BF16, None) == -3
    assert L.fa_fwd_ex(BASE, BASE, BASE, BASE, None, 1, 1, 1, 8, 128, 0, 1.0, F.BF16, F.BF16,
                       None, None) == -5


def test_fp32_output_allowed_for_16_bit_inputs():
    assert check(odt=F.F32)[0] == 0
    assert check(dt=F.F16, odt=F.F32)[0] == 0
    assert check(dt=F.F32, d=64, odt=F.F32)[0] == 0


def test_python_plan_helper():
    import torch
    p = F.plan(16, 16, 16, 512, 64, False, torch.float16)
    assert p.grid == 16 * 16 * 4
    with pytest.raises(F.FA355Error):
        F.plan(1, 1, 1, 8, 80, False, torch.bfloat16)


def bwd_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, do=BASE + 4 * SPAN,
             lse=BASE + 5 * SPAN, dq=BASE + 6 * SPAN, dk=BASE + 7 * SPAN, dv=BASE + 8 * SPAN,
             delta=BASE + 9 * SPAN, B_=1, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.1,
             dt=F.BF16):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, B_, Hq, Hkv, N, d, causal,
                          scale, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(do=None), -1), (dict(lse=None), -1), (dict(delta=None), -1),
    (dict(dq=None), -1), (dict(B_=-1), -2), (dict(Hq=3, Hkv=2), -2), (dict(N=-1), -2),
    (dict(d=32), -3), (dict(d=96), -3), (dict(dt=F.F32, d=64), -3), (dict(dt=9), -3),
    (dict(scale=float("nan")), -5), (dict(q=BASE + 8), -4), (dict(dk=BASE + 7 * SPAN + 4), -4),
    (dict(lse=BASE + 5 * SPAN + 2), -4), (dict(dq=BASE), -5), (dict(dv=BASE + 7 * SPAN + 64), -5),
    (dict(delta=BASE + 4 * SPAN + 128), -5), (dict(dk=BASE + 6 * SPAN + 4096), -5),
])
def test_bwd_rejections(kw, code):
    assert bwd_call(**kw) == code, kw


def split_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
               B_=1, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.1, dt=F.BF16, S=4,
               op=BASE + 5 * SPAN, lp=BASE + 6 * SPAN):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_fwd_split(q, k, v, o, lse, B_, Hq, Hkv, N, d, causal, scale, dt, S, op, lp,
                                None)


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), -1), (dict(lp=None), -1), (dict(q=None), -1), (dict(S=0), -5), (dict(S=17), -5),
    (dict(d=256), -3), (dict(dt=F.F32, d=64), -3), (dict(N=-1), -2), (dict(op=BASE + 5 * SPAN + 8), -4),
    (dict(lp=BASE + 6 * SPAN + 2), -4), (dict(op=BASE + 8192), -5), (dict(lp=BASE + 5 * SPAN + 64), -5),
])
def test_split_rejections(kw, code):
    assert split_call(**kw) == code, kw


def bias_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
              bias=BASE + 5 * SPAN, sb=0, sh=100 * 100, si=100, B_=1, Hq=4, Hkv=2, N=100, d=128,
              causal=1, scale=0.1, dt=F.BF16):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_fwd_bias(q, k, v, o, lse, bias, sb, sh, si, B_, Hq, Hkv, N, d, causal, scale,
                               dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bias=None), -1), (dict(q=None), -1), (dict(si=99), -5), (dict(sb=-4), -5),
    (dict(bias=BASE + 5 * SPAN + 2), -4), (dict(si=102), -4), (dict(sh=10002), -4),
    (dict(d=256), -3), (dict(dt=F.F32, d=64), -3), (dict(bias=BASE + 3 * SPAN + 64), -5),
    (dict(N=1 << 16, si=1 << 16, sh=1 << 32), -2), (dict(Hq=3), -2),
])
def test_bias_rejections(kw, code):
    assert bias_call(**kw) == code, kw


def fp8_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
             B_=1, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.1, dq=0.01, dk=0.01, dv=0.01):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_fwd_fp8(q, k, v, o, lse, B_, Hq, Hkv, N, d, causal, scale, dq, dk, dv, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(B_=-1), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(N=-1), -2), (dict(N=1 << 30), -2), (dict(d=256), -3),
    (dict(d=96), -3), (dict(scale=float("inf")), -5), (dict(dq=0.0), -5), (dict(dk=-1.0), -5),
    (dict(dv=float("nan")), -5), (dict(dq=float("inf")), -5), (dict(dq=1e30, dk=1e30), -5),
    (dict(q=BASE + 8), -4), (dict(o=BASE + 3 * SPAN + 2), -4), (dict(lse=BASE + 4 * SPAN + 1), -4),
    (dict(o=BASE + 32), -5), (dict(lse=BASE + 2 * SPAN + 16), -5), (dict(lse=BASE + 3 * SPAN + 64), -5),
])
def test_fp8_rejections(kw, code):
    assert fp8_call(**kw) == code, kw


def test_split_count_heuristic():
    # About two 256-row workgroups per CU at head dim 128, four 128-row ones at 64,
    # at least four 64-key blocks per split, never above 16, 1 when the tiles
    # already fill the GPU.
    assert F.split_count(1, 2, 16384, True) == 4
    assert F.split_count(1, 2, 16384, True, d=64) == 4
    assert F.split_count(1, 32, 4096, True) == 1
    assert F.split_count(1, 1, 64, True) == 1
    assert F.split_count(1, 1, 8192, True) == 16        # 32 tiles: capped at 16
    assert F.split_count(1, 8, 8192, False) == 1        # 256 tiles without a mask: no split
    assert F.split_count(2, 8, 4096, True) == 2         # 256 causal tiles: still two pieces
    assert F.split_count(1, 1, 1 << 20, True) == 1      # 4096 tiles fill the GPU
    assert F.split_count(1, 1, 1024, False) == 4     # 16 key blocks: at most 4 splits


def decode_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
                B_=1, Hq=8, Hkv=2, Nq=2, Nk=100, d=128, causal=1, scale=0.1, dt=F.BF16, S=4,
                op=BASE + 5 * SPAN, lp=BASE + 6 * SPAN):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_fwd_decode(q, k, v, o, lse, B_, Hq, Hkv, Nq, Nk, d, causal, scale, dt, S,
                                 op, lp, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(op=None), -1), (dict(lp=None), -1), (dict(o=None), -1),
    (dict(B_=-1), -2), (dict(Nq=-1), -2), (dict(Nk=0), -2), (dict(Hq=3), -2),
    (dict(Nq=101), -2), (dict(Nk=1 << 30), -2),
    (dict(Nq=9), -3), (dict(Hq=64, Hkv=1, Nq=1), -3), (dict(d=256), -3), (dict(dt=F.F32, d=64), -3),
    (dict(S=0), -5), (dict(S=257), -5), (dict(scale=float("nan")), -5),
    (dict(q=BASE + 8), -4), (dict(op=BASE + 5 * SPAN + 4), -4), (dict(lse=BASE + 4 * SPAN + 2), -4),
    (dict(o=BASE + 64), -5), (dict(op=BASE + 3 * SPAN + 64), -5), (dict(lp=BASE + 5 * SPAN + 16), -5),
])
def test_decode_rejections(kw, code):
    assert decode_call(**kw) == code, kw


def decode_noalloc_call(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN,
                        lse=BASE + 4 * SPAN, B_=1, Hq=8, Hkv=2, Nq=2, Nk=100, d=128, causal=1,
                        scale=0.1, dt=F.BF16, S=4):
    # Invalid arguments only: every call below must be rejected before any HIP call.
    return F.lib().fa_fwd_decode_noalloc(q, k, v, o, lse, B_, Hq, Hkv, Nq, Nk, d, causal, scale,
                                         dt, S, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1),
    (dict(B_=-1), -2), (dict(Nk=0), -2), (dict(Hq=3), -2), (dict(Nq=101), -2),
    (dict(Nq=9), -3), (dict(d=256), -3), (dict(dt=F.F32, d=64), -3),
    (dict(S=0), -5), (dict(S=257), -5), (dict(scale=float("inf")), -5),
    (dict(q=BASE + 8), -4), (dict(lse=BASE + 4 * SPAN + 2), -4), (dict(o=BASE + 64), -5),
    # The library's workspace holds 16 MiB: 256 pieces of 16 x 8 rows of d = 128 need
    # 16 MiB of partial outputs plus 128 KiB of partial lse values.
    (dict(B_=16, Hq=8, Hkv=1, Nq=1, Nk=1 << 16, S=256), -2),
    (dict(B_=16, Hq=32, Hkv=1, Nq=1, Nk=1 << 16, S=256, d=64, causal=0), -2),
])
def test_decode_noalloc_rejections(kw, code):
    assert decode_noalloc_call(**kw) == code, kw


def test_decode_noalloc_workspace_size():
    assert F.NOALLOC_SCRATCH_BYTES == 16 << 20
    # 256 pieces x 15 batches x 8 heads: 15 MiB of outputs + 120 KiB of lse fit.
    assert F.decode_noalloc_bytes(15, 8, 1, 128, 256) == 30720 * 512 + 30720 * 4
    assert F.decode_noalloc_bytes(15, 8, 1, 128, 256) <= F.NOALLOC_SCRATCH_BYTES
    assert F.decode_noalloc_bytes(16, 8, 1, 128, 256) > F.NOALLOC_SCRATCH_BYTES
    assert F.decode_noalloc_bytes(1, 1, 1, 64, 1) == 256 + 4        # lse on a 256-byte boundary


def test_decode_allows_more_queries_than_keys_without_causal_mask():
    # Nq > Nk is only an error under the causal mask (checked before any HIP call).
    assert decode_call(Nq=2, Nk=1, S=0, causal=0) == -5


def test_decode_split_count_heuristic():
    assert F.decode_split_count(8, 8, 8192) == 16          # 512 keys per piece
    assert F.decode_split_count(1, 8, 32768) == 64
    assert F.decode_split_count(1, 8, 4096) == 32          # one workgroup per CU
    assert F.decode_split_count(1, 1, 100) == 1            # at least four blocks a piece
    assert F.decode_split_count(1, 1, 1 << 22) == 256
    assert F.decode_split_count(32, 8, 4096) == 2          # 256 (batch, head) pairs: 2 per CU
    assert F.decode_split_count(64, 8, 2048) == 1


def test_library_imports_no_allocating_or_copying_call():
    """The library allocates, clears and copies nothing (the forward pass keeps O(N)
    state, never an N x N matrix): of the HIP runtime it imports only kernel
    registration, the launch and the per-kernel LDS attribute."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not installed")
    allowed = {"__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
               "__hipRegisterFunction", "__hipUnregisterFatBinary", "hipFuncSetAttribute",
               "hipLaunchKernel",
               # the static workspace of fa_fwd_decode_noalloc and its per-GPU address
               "__hipRegisterVar", "hipGetSymbolAddress", "hipStreamGetDevice", "hipGetDevice",
               "hipSetDevice"}
    for path in (B.LIB_PATH, B.LDS_POISON_LIB_PATH):
        out = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True,
                             check=True).stdout
        hip = {line.split()[-1].split("@")[0] for line in out.splitlines()
               if "hip" in line.lower()}
        assert hip and hip <= allowed, (path, sorted(hip - allowed))


def test_use_library_restores_the_previous_library():
    before = B.lib()
    with pytest.raises(RuntimeError):
        with B.use_library(B.LDS_POISON_LIB_PATH) as dbg:
            assert B.lib() is dbg and dbg is not before
            raise RuntimeError("leave the block")
    assert B.lib() is before
    with pytest.raises(B.FA355Error):
        with B.use_library(B.LIB_PATH + ".missing"):
            pass
    assert B.lib() is before


def test_binding_rejects_mismatched_tensors_before_any_launch():
    # Every entry point of the binding checks the 4-D shapes of q, k, v and their
    # agreement, one dtype, and the exact shape and dtype of any output or workspace
    # it is given, before a device is touched: these raise on a machine without a GPU.
    import torch
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros(1, 4, 64, 128, **bf)
    k = torch.zeros(1, 2, 64, 128, **bf)
    short = torch.zeros(1, 2, 63, 128, **bf)
    f32 = dict(dtype=torch.float32)

    def raises(status, fn, *a, **kw):
        with pytest.raises(F.FA355Error) as e:
            fn(*a, **kw)
        assert e.value.status == status, (fn.__name__, e.value)

    for fn in (F.fwd, F.fwd_split):
        raises(B.ERR_SHAPE, fn, q, short, short)                      # k shorter than q
        raises(B.ERR_SHAPE, fn, q, k, short)                          # v unlike k
        raises(B.ERR_SHAPE, fn, q[0], k, k)                           # not 4-D
        raises(B.ERR_UNSUPPORTED, fn, q, k.half(), k)                 # mixed dtypes
        raises(B.ERR_ARG, fn, q, k, k, o=torch.zeros(1, 4, 64, 64, **bf))
        raises(B.ERR_ARG, fn, q, k, k, lse=torch.zeros(1, 4, 64, **bf))
        raises(B.ERR_ARG, fn, q, k, k)                                # host tensors
    raises(B.ERR_ARG, F.fwd_split, q, k, k, num_splits=4, o_part=torch.zeros(3, 1, 4, 64, 128, **f32))
    raises(B.ERR_ARG, F.fwd_split, q, k, k, num_splits=4, lse_part=torch.zeros(4, 1, 4, 64, **bf))
    raises(B.ERR_ARG, F.fwd_split, q, k, k, num_splits=0)
    bias = torch.zeros(1, 1, 64, 64, **bf)
    raises(B.ERR_SHAPE, F.fwd_bias, q, short, short, bias)
    raises(B.ERR_UNSUPPORTED, F.fwd_bias, q, k, k.half(), bias)
    raises(B.ERR_ARG, F.fwd_bias, q, k, k, bias, o=torch.zeros(1, 4, 64, 128, **f32))
    raises(B.ERR_ARG, F.fwd_bias, q.transpose(2, 3).contiguous().transpose(2, 3), k, k, bias)
    raises(B.ERR_SHAPE, F.fwd_bias, q, k, k, torch.zeros(1, 1, 64, 63, **bf))
    u8 = dict(dtype=torch.uint8)
    q8, k8 = torch.zeros(1, 4, 64, 128, **u8), torch.zeros(1, 2, 64, 128, **u8)
    raises(B.ERR_SHAPE, F.fwd_fp8, q8, k8[:, :, :32], k8[:, :, :32], 1.0, 1.0, 1.0)
    raises(B.ERR_UNSUPPORTED, F.fwd_fp8, q, k, k, 1.0, 1.0, 1.0)
    raises(B.ERR_ARG, F.fwd_fp8, q8, k8, k8, 1.0, 1.0, 1.0, lse=torch.zeros(1, 4, 64, **bf))
    raises(B.ERR_ARG, F.fwd_fp8, q8, k8, k8, 1.0, 1.0, 1.0, o=torch.zeros(1, 4, 64, 128, **f32))
    # Decoding: queries and cache may differ in length, nothing else.
    qd = torch.zeros(1, 8, 1, 128, **bf)
    kd = torch.zeros(1, 2, 300, 128, **bf)
    raises(B.ERR_SHAPE, F.fwd_decode, qd, kd, kd[:, :, :200])
    raises(B.ERR_SHAPE, F.fwd_decode, qd, torch.zeros(2, 2, 300, 128, **bf), torch.zeros(2, 2, 300, 128, **bf))
    raises(B.ERR_ARG, F.fwd_decode, qd, kd, kd, num_splits=8, o_part=torch.zeros(4, 1, 8, 1, 128, **f32))
    raises(B.ERR_ARG, F.fwd_decode, qd, kd, kd, num_splits=8, lse_part=torch.zeros(8, 1, 8, 2, **f32))
    raises(B.ERR_ARG, F.fwd_decode, qd, kd, kd, o=torch.zeros(1, 8, 1, 128, **f32))
    # Backward: gradients and workspace must be fp32 of the exact shapes.
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(1, 4, 64, **f32)
    raises(B.ERR_SHAPE, F.bwd, q, short, short, o, do, lse)
    raises(B.ERR_ARG, F.bwd, q, k, k, o, do, lse, dk=torch.zeros(1, 4, 64, 128, **f32))
    raises(B.ERR_ARG, F.bwd, q, k, k, o, do, lse, delta=torch.zeros(1, 4, 64, **bf))
    raises(B.ERR_ARG, F.bwd, q, k, k, o, do, lse)                                 # host tensors
