"""Benchmark of the FlashAttention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --profile-run      # a few launches + a calibration copy, for rocprofv3
    python bench.py --bwd [...]        # the backward pass (fa_bwd) on the same workload
    python bench.py --split [S] [...]  # the split-KV forward (fa_fwd_split)
    python bench.py --bias KIND [...]  # the forward with an additive bias (fa_fwd_bias)
    python bench.py --fp8 [...]        # the e4m3-input forward (fa_fwd_fp8), same layer shape
    python bench.py --decode [...]     # decoding against a key/value cache (fa_fwd_decode)

A step is one pass of the whole hot path -- one fused forward kernel -- over one
batch of seeded synthetic inputs already resident in device memory.  Before the W
warm-up steps, the step is launched back to back for 0.25 s (settle): out of idle
the clock takes ~20 ms to ramp, and steps timed inside the ramp run 10-30 % slow.  The default
workload is the causal bf16 layer B=1, H=32, N=4096, d=128.  Prints one JSON line.

value       = algorithmic FLOPs (4*B*Hq*N^2*d, halved when causal) * K / wall time of
              the K timed steps, bracketed by device synchronisation.
roofline    = the kernel's own rate: FLOPs per launch / average launch duration from
              HIP events recorded on the launch stream around the timed region, against
              the 2.5 PFLOP/s dense bf16 MFMA peak -- or, for a workload whose FLOPs per
              compulsory byte fall below the ridge point, compulsory bytes / duration
              against 8 TB/s of HBM.  traffic = HBM bytes per launch from
              rocprofv3 FETCH_SIZE / WRITE_SIZE counters, calibrated on a copy of known
              size (read from profiles/, null when the kernel sources changed since).
cpu_baseline = the fp64 CPU oracle, as it stands, on a bounded sample of query rows of
              the same workload, on this host's cores, in the same unit; its
              `parity` compares the GPU's output on that sample with the oracle's.
Also reported, after the timed region: the median and minimum of the time per
launch over chunks of 10 back-to-back launches, each chunk bracketed by HIP events
(roofline.kernel_us_median / kernel_us_min); the shader clock, measured by timing
a spin kernel of known cycle counts between the kernel's launches, with the
matrix-core peak scaled to it, beside amd-smi's readings (clock); and, for
HBM-bound lines, the same with a 512 MB buffer read before each
launch so that no input is left in L2 or the MALL, the reads timed alone and
subtracted (cold).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak (causal, d=128, N=4096)"
METRIC_BWD = "attention bwd TFLOP/s and % of MI355X bf16 MFMA peak"
METRIC_FP8 = "attention fwd TFLOP/s and % of MI355X fp8 MFMA peak (e4m3 inputs, causal, d=128, N=4096)"
FP8_WORKLOAD = "e4m3_h32_n4096_d128_causal"
METRIC_DECODE = "attention decode GB/s (K/V cache read) and % of MI355X HBM bandwidth"
DECODE_WORKLOAD = "bf16_decode_b8_hq32_hkv8_nk8192_d128"
BWD_FLOP_RATIO = 2.5   # backward = 5 matrix products (S, dP, dV, dK, dQ) vs the forward's 2
DEFAULT_WORKLOAD = "bf16_h32_n4096_d128_causal"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "e4m3": 5000.0}
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CONFIG_WORKLOADS = ("f32_h1_n128_d64", "f16_b16_h16_n512_d64_qbias",
                    "bf16_gqa_b4_hq32_hkv8_n8192_d128_causal", "bf16_h16_n32768_d128_causal_x3",
                    "bf16_h8_n8192_d256_causal_x3")


def _elf_sections(b: bytes):
    """(name, offset, size, addr, type, link, entsize) of every section of an ELF64 image."""
    import struct
    shoff = struct.unpack_from("<Q", b, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    raw = [struct.unpack_from("<IIQQQQIIQQ", b, shoff + i * shentsize) for i in range(shnum)]
    stroff = raw[shstrndx][4]
    out = []
    for nm, typ, _flags, addr, off, size, link, _info, _align, entsize in raw:
        name = b[stroff + nm:b.index(b"\0", stroff + nm)].decode()
        out.append((name, off, size, addr, typ, link, entsize))
    return out


def _code_object_symbols(co: bytes):
    """{symbol: bytes} of the functions (their machine code) and objects (kernel
    descriptors) of one AMDGPU code object."""
    import struct
    secs = _elf_sections(co)
    out = {}
    for name, off, size, _addr, typ, link, entsize in secs:
        if typ != 2:                                   # SHT_SYMTAB
            continue
        stroff = secs[link][1]
        for i in range(size // entsize):
            st_name, st_info, _other, shndx, value, sz = struct.unpack_from("<IBBHQQ", co, off + i * entsize)
            kind = st_info & 0xF
            if kind not in (1, 2) or sz == 0 or shndx == 0 or shndx >= len(secs):
                continue
            sym = co[stroff + st_name:co.index(b"\0", stroff + st_name)].decode()
            _n, soff, _s, saddr, _t, _l, _e = secs[shndx]
            out[sym] = co[soff + value - saddr:soff + value - saddr + sz]
    return out


def kernel_code_hashes(lib_path: str) -> dict:
    """sha256 (first 16 hex digits) of each gfx950 kernel's machine code together with
    its kernel descriptor, read from the library's embedded device code objects.  Two
    builds with the same hash for a kernel run the same instructions with the same
    register and LDS allocation, whatever else changed in the sources."""
    import struct
    with open(lib_path, "rb") as fh:
        so = fh.read()
    fat = [(off, size) for name, off, size, *_ in _elf_sections(so) if name == ".hip_fatbin"]
    hashes = {}
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    for off, size in fat:
        blob = so[off:off + size]
        pos = blob.find(magic)
        while pos >= 0:
            n = struct.unpack_from("<Q", blob, pos + 24)[0]
            q = pos + 32
            for _ in range(n):
                eoff, esize, tlen = struct.unpack_from("<QQQ", blob, q)
                triple = blob[q + 24:q + 24 + tlen].decode()
                q += 24 + tlen
                if "gfx950" in triple and esize:
                    syms = _code_object_symbols(blob[pos + eoff:pos + eoff + esize])
                    for sym, code in syms.items():
                        if sym.endswith(".kd"):
                            continue
                        h = hashlib.sha256(code + syms.get(sym + ".kd", b""))
                        hashes[sym] = h.hexdigest()[:16]
            pos = blob.find(magic, pos + 1)
    return hashes


def fwd_kernel_symbol(dtype: str, d: int, bc: int, waves: int, causal: bool) -> str:
    """Mangled name of the forward kernel a plan launches (output in the input type,
    no split, no bias).  Head dim 256 with eight wavefronts is the kernel split by
    role (32-key blocks) or the wavefront-pair kernel (64-key blocks)."""
    t = {"bf16": "4BF16", "f16": "3F16"}[dtype]
    if d == 256 and waves == 8:
        kind = "18fa_fwd_role_kernel" if bc == 32 else "18fa_fwd_pair_kernel"
        return f"_ZN5fa355{kind}INS_{t}ELb{int(causal)}ELb0EEEvNS_7FwdArgsE"
    return (f"_ZN5fa35513fa_fwd_kernelINS_{t}ELi{d}ELi{bc}ELi{waves}ELb{int(causal)}"
            f"ELb0ELb0ELb0EEEvNS_7FwdArgsE")


def load_traffic(workload: str, kernels=None):
    """HBM bytes per launch from the committed counter summary, or None unless every
    kernel the summary was taken on still has the machine code it had then (and,
    when `kernels` is given, the summary covers exactly those kernels)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            e = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not e:
        return None
    import io_aware_attention_amd as F
    current = kernel_code_hashes(F.fa355.LIB_PATH)
    recorded = e.get("kernels", {})
    if not recorded or any(current.get(k) != h for k, h in recorded.items()):
        return None
    if kernels is not None and set(kernels) != set(recorded):
        return None
    return e.get("bytes_per_launch")


def _pmc_rows(path: str):
    """(kernel name, counter, value) per dispatch row of a rocprofv3 counter CSV."""
    import csv
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            yield row.get("Kernel_Name", ""), row.get("Counter_Name", ""), float(row.get("Counter_Value", 0)), \
                row.get("Dispatch_Id", "")


def record_traffic(workload: str, fetch_csv: str, write_csv: str, kernels: list, command: str) -> dict:
    """Reduces two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch)
    of `bench.py --profile-run --workload W` to HBM bytes per launch, each counter
    scaled by what it reads for the run's calibration copy of known size, and stores
    them in profiles/traffic.json with the machine-code hash of every kernel counted."""
    import io_aware_attention_amd as F

    def per_kernel(path, counter):
        by = {}
        for name, cname, val, disp in _pmc_rows(path):
            if cname != counter:
                continue
            by.setdefault(name, {}).setdefault(disp, 0.0)
            by[name][disp] += val
        return {k: sum(v.values()) / len(v) for k, v in by.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = 64 * 2 ** 20 * 4                      # the calibration copy: 64 Mi fp32
    copy = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy:
        raise RuntimeError(f"no calibration copy kernel among {sorted(fetch)}")
    ck = copy[0]
    ffac = copy_bytes / (fetch[ck] * 1024.0)
    wfac = copy_bytes / (write[ck] * 1024.0)
    hashes = kernel_code_hashes(F.fa355.LIB_PATH)
    names = {}
    fkib = wkib = 0.0
    for sym in kernels:
        demangled = [k for k in fetch if _matches(sym, k)]
        if len(demangled) != 1:
            raise RuntimeError(f"{sym}: no unique dispatch name among {sorted(fetch)}")
        names[sym] = hashes[sym]
        fkib += fetch[demangled[0]]
        wkib += write[demangled[0]]
    entry = {"kernels": names, "bytes_per_launch": int(round(fkib * 1024 * ffac + wkib * 1024 * wfac)),
             "fetch_kib_per_dispatch": round(fkib, 1), "write_kib_per_dispatch": round(wkib, 1),
             "fetch_factor": round(ffac, 4), "write_factor": round(wfac, 4),
             "calibration": f"{ck.split('(')[0][:80]} copying {copy_bytes} bytes in the same run",
             "command": command}
    try:
        with open(TRAFFIC_FILE) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[workload] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return entry


def _matches(sym: str, demangled: str) -> bool:
    """Does a rocprofv3 (demangled) kernel name denote the mangled symbol `sym`?"""
    import re
    m = re.match(r"_ZN5fa355(\d+)(\w+?)I(.*)EEvNS_\d+\w+E$", sym)
    if not m:
        return False
    base = sym[len("_ZN5fa355") + len(m.group(1)):len("_ZN5fa355") + len(m.group(1)) + int(m.group(1))]
    if f"fa355::{base}<" not in demangled:
        return False
    args = re.findall(r"Li(\d+)E|Lb(\d)E|NS_\d+(\w+?)E", m.group(3))
    want = []
    for num, b, t in args:
        want.append(num if num else ("true" if b == "1" else "false") if b else f"fa355::{t}")
    got = demangled[demangled.index("<") + 1:demangled.rindex(">")]
    return [g.strip() for g in got.split(",")] == want


SETTLE_S = 0.25   # untimed launches before the warm-up steps: the clock ramps for ~20 ms


def settle(step, sync, seconds: float = SETTLE_S) -> int:
    """Launches `step` back to back for `seconds` of wall time (synchronising every
    16 launches), so that the timed steps see the clock the kernel sustains rather
    than the ramp out of idle: on an idle MI355X the first ~20 ms of launches of the
    headline kernel run 10-30 % slower than the steady state.  Returns the count."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            step()
        n += 16
        sync()
    return n


def _amd_smi_gfx_mhz():
    """Mean current gfx clock over the XCDs from `amd-smi metric -c --json`, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(r.stdout[r.stdout.index("{"):])
        clocks = d["gpu_data"][0]["clock"] if "gpu_data" in d else d[0]["clock"]
        vals = [v["clk"]["value"] for k, v in clocks.items()
                if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        return sum(vals) / len(vals) if vals else None
    except Exception:  # noqa: BLE001 -- the tool is optional; no clock is reported then
        return None


def sustained_clock(step, sync, launch_us: float, samples: int = 2) -> dict | None:
    """The gfx clock under this kernel's own sustained load.

    After the timed region, keeps launching `step` (synchronising after about 20 ms
    of queued launches) while a thread reads the clock `samples` times with
    amd-smi; returns the mean reading, or None when amd-smi is unavailable.
    """
    import threading

    got = []

    def sampler():
        time.sleep(0.3)
        for _ in range(samples):
            got.append(_amd_smi_gfx_mhz())

    th = threading.Thread(target=sampler)
    th.start()
    chunk = max(16, int(20000.0 / max(launch_us, 1.0)))
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < 60:
        for _ in range(chunk):
            step()
        sync()
    th.join()
    vals = sorted(g for g in got if g)
    if not vals:
        return None
    return {"sclk_mhz": round(vals[len(vals) // 2], 1), "samples_mhz": [round(v, 1) for v in vals],
            "source": "amd-smi metric -c (mean of the XCDs' current gfx clock; median of the "
                      "readings), read during sustained launches of the same kernel after the "
                      "timed region"}


CHUNK = 10   # launches per timed chunk for the median / minimum


def _chunk_us(stream, chunks: int, body):
    """Per-chunk times (us) of `chunks` runs of `body`, each bracketed by HIP events on
    the launch stream, enqueued back to back and read after one synchronisation."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(chunks)]
    for a, b in ev:
        a.record(stream)
        body()
        b.record(stream)
    stream.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def probe_clock_mhz(step, stream, rounds: int = 5) -> float:
    """The shader clock while the kernel runs: torch's spin kernel waits a given
    number of shader-clock cycles (the s_memtime counter); timed between launches of
    `step` at two lengths, the slope cycles / time is the clock, free of the fixed
    cost an event pair adds.  Median over `rounds`."""
    import torch

    short, long_ = 200_000, 2_200_000
    est = []
    for _ in range(rounds):
        t = []
        for cyc in (short, long_):
            for _ in range(4):
                step()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            torch.cuda._sleep(cyc)
            b.record(stream)
            for _ in range(4):
                step()
            stream.synchronize()
            t.append(a.elapsed_time(b) * 1e3)
        est.append((long_ - short) / (t[1] - t[0]))
    est.sort()
    return round(est[len(est) // 2], 1)


def per_launch_us(step, stream, reps: int, flush=None):
    """Median and minimum over chunks of CHUNK back-to-back launches of the time per
    launch (an event pair around a single launch adds ~25 us here).  With `flush`,
    each launch is preceded by it, and the same chunks of flushes alone, timed
    alternately, are subtracted."""
    chunks = max(5, reps // CHUNK)

    def launches():
        for _ in range(CHUNK):
            if flush is not None:
                flush()
            step()

    if flush is None:
        per = sorted(t / CHUNK for t in _chunk_us(stream, chunks, launches))
    else:
        def flushes():
            for _ in range(CHUNK):
                flush()
        per = []
        for _ in range(chunks):
            both = _chunk_us(stream, 1, launches)[0]
            alone = _chunk_us(stream, 1, flushes)[0]
            per.append((both - alone) / CHUNK)
        per.sort()
    return per[len(per) // 2], per[0]


def cache_flusher(dev, nbytes: int = 512 << 20):
    """Reads a 512 MB scratch buffer (twice the 256 MB MALL) on the current stream.

    A read rather than a write: written lines would still be dirty in L2 and the
    MALL when the kernel starts, and their write-back would be charged to it."""
    import torch

    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    return lambda: torch.sum(buf, dim=0, out=out)


def add_protocol_fields(line, step, stream, dev, reps, work, unit_scale, peak, cold):
    """Per-launch median / minimum, the sustained clock, and (for HBM-bound lines) a
    cold-cache variant, added beside the contract's fields.  `work` is the
    algorithmic FLOPs or bytes of one launch, `unit_scale` turns work/us into the
    roofline unit."""
    import torch

    sync = lambda: torch.cuda.synchronize(dev)  # noqa: E731
    settle(step, sync, 0.1)
    med, mn = per_launch_us(step, stream, reps)
    r = line["roofline"]
    r["kernel_us_median"] = round(med, 2)
    r["kernel_us_min"] = round(mn, 2)
    r["achieved_median"] = round(work / med * unit_scale, 2)
    if cold:
        fl = cache_flusher(dev)
        cmed, cmn = per_launch_us(step, stream, reps, flush=fl)
        line["cold"] = {"kernel_us_median": round(cmed, 2), "kernel_us_min": round(cmn, 2),
                        "achieved_median": round(work / cmed * unit_scale, 2), "unit": r["unit"],
                        "frac": round(work / cmed * unit_scale / peak, 4),
                        "how": "a 512 MB buffer read (summed) before each launch; chunks of "
                               "10 (read, launch) pairs minus chunks of 10 reads alone"}
    settle(step, sync, 0.1)
    clk = {"sclk_mhz": probe_clock_mhz(step, stream),
           "source": "shader-clock cycles of torch's spin kernel (two lengths, slope of their "
                     "HIP-event times) enqueued between launches of the kernel, after settling"}
    smi = sustained_clock(step, sync, r["kernel_us"])
    if smi is not None:
        clk["amd_smi"] = smi
    if r["bound"] != "hbm":
        # Matrix-core peak scales with the gfx clock (2400 MHz nominal); HBM's does not.
        clk["peak_at_sclk"] = round(peak * clk["sclk_mhz"] / 2400.0, 1)
        clk["frac_at_sclk"] = round(r["achieved"] / clk["peak_at_sclk"], 4)
    line["clock"] = clk


def device_inputs(x, dev):
    import torch
    out = []
    for n in "qkv":
        a = getattr(x, n)
        t = torch.from_numpy(a).view(torch.bfloat16) if x.dtype == "bf16" else torch.from_numpy(a)
        out.append(t.to(dev))
    return out


def _half_ulp(x, dtype: str):
    """Half the spacing of a 16-bit float format at each |x| (one RNE store)."""
    import numpy as np
    p, emin = {"bf16": (8, -126), "f16": (11, -14)}[dtype]
    _, e = np.frexp(np.abs(x))
    e = np.where(x == 0, emin, np.maximum(e.astype(np.int64) - 1, emin))
    return np.ldexp(0.5, e - (p - 1))


def parity_of(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype: str, fp8: bool = False) -> dict:
    """Errors of the GPU's output on the oracle's sample: max |O - O_ref| and
    |lse - lse_ref|, and the worst ratio to the tolerance (1e-5 for fp32 outputs,
    2e-2 plus half an output ulp for 16-bit ones; lse 1e-3).  e4m3 inputs have no
    fixed tolerance (their per-element bounds follow from the e4m3 rounding of the
    weights, computed by the GPU tests): errors only."""
    import numpy as np
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    out = {"max_abs_o": float(err.max()), "max_abs_lse": float(lerr.max())}
    if fp8:
        out["tolerance"] = "per-element bounds from the e4m3 rounding (GPU tests)"
        out["lse_err_over_1e-3"] = round(out["max_abs_lse"] / 1e-3, 3)
        out["lse_within_1e-3"] = bool((lerr <= 1e-3).all())
        return out
    bound = 1e-5 if out_dtype == "f32" else 2e-2 + _half_ulp(o_ref, out_dtype)
    out["worst_o_err_over_tolerance"] = float((err / bound).max())
    out["within_tolerance"] = bool((err <= bound).all() and (lerr <= 1e-3).all())
    return out


def physical_cores() -> int | None:
    """Distinct (package, core) pairs in /proc/cpuinfo (None if it cannot be read)."""
    try:
        pairs, phys = set(), None
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "physical id":
                    phys = val.strip()
                elif key == "core id":
                    pairs.add((phys, val.strip()))
        return len(pairs) or None
    except OSError:
        return None


def oracle_single_thread_small() -> float:
    """Seconds for the oracle on the smallest workload (fp32 B1 H1 N128 d64) on one thread."""
    import oracle
    import fa_inputs as G
    x = G.workload("f32_h1_n128_d64")
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    t0 = time.perf_counter()
    oracle.attention(q, k, v, x.causal, x.scale, threads=1)
    return time.perf_counter() - t0


def cpu_baseline(x, budget_s: float = 15.0, gpu=None) -> dict:
    """Time the oracle on a bounded sample of the workload and scale to TFLOP/s.

    The sample is whole query heads (b = 0, heads 0, 1, ...) when one head takes
    less than the budget, otherwise every k-th query row of head 0.  FLOPs are
    counted as for the GPU: 4*d per visible (query, key) pair.  With `gpu` = (o,
    lse, output dtype) of the same workload, the GPU's rows of the sample are
    compared with the oracle's (`parity`).
    """
    import numpy as np

    import oracle
    from fa_inputs import storage_to_f64

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    G = x.Hq // x.Hkv

    def f64(name, h0, h1):
        a = storage_to_f64(np.ascontiguousarray(getattr(x, name)[0:1, h0:h1]), x.dtype)
        if x.descale is not None:
            a *= x.descale["qkv".index(name)]
        return a

    def row_flops(rows):
        keys = (rows + 1) if x.causal else np.full(len(rows), x.N)
        return float(4.0 * x.d * keys.sum())

    # Calibrate on a few rows spread over the causal range of head 0.
    q, k, v = f64("q", 0, 1), f64("k", 0, 1), f64("v", 0, 1)
    rows = np.arange(x.N - 1, -1, -31, dtype=np.int64)[::-1].copy()
    t0 = time.perf_counter()
    oracle.attention(q, k, v, x.causal, x.scale, rows=rows, threads=threads)
    rate = row_flops(rows) / max(time.perf_counter() - t0, 1e-3)
    head_flops = row_flops(np.arange(x.N))
    n_heads = int(rate * budget_s // head_flops)

    if n_heads >= 1:
        n_heads = min(x.Hq, max(G, n_heads // G * G))
        q, k, v = f64("q", 0, n_heads), f64("k", 0, n_heads // G), f64("v", 0, n_heads // G)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention(q, k, v, x.causal, x.scale, threads=threads)
        dt = time.perf_counter() - t0
        flops = head_flops * n_heads
        sample = f"all {x.N} query rows of heads 0..{n_heads - 1} (batch 0) of {x.recipe}"
        pick = (0, slice(0, n_heads))
    else:
        every = int(math.ceil(head_flops / (rate * budget_s)))
        rows = np.arange(0, x.N, every, dtype=np.int64)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention(q, k, v, x.causal, x.scale, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        flops = row_flops(rows)
        sample = f"every {every}th query row of head (0,0) of {x.recipe}"
        pick = (0, slice(0, 1), rows)
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{sample}; {dt:.1f} s in fp64 on {threads} threads",
           "host": {"threads_used": threads, "logical_cpus": os.cpu_count(),
                    "physical_cores": physical_cores(),
                    "single_thread_s_fp32_b1_h1_n128_d64": round(oracle_single_thread_small(), 6)}}
    if gpu is not None:
        o, lse, odt = gpu
        import torch  # noqa: F401 -- the GPU tensors are torch's
        ri = None if len(pick) == 2 else torch.from_numpy(pick[2]).to(o.device)
        og, lg = o[pick[0], pick[1]], lse[pick[0], pick[1]]
        if ri is not None:
            og, lg = og.index_select(1, ri), lg.index_select(1, ri)
        out["parity"] = parity_of(og.float().cpu().double().numpy(), lg.cpu().double().numpy(),
                                  o_ref[0], l_ref[0], odt, fp8=x.dtype == "e4m3")
    return out


def cpu_baseline_bwd(x, budget_s: float) -> dict:
    """The fp64 gradient oracle, as it stands, on whole heads of the workload."""
    import oracle

    threads = os.cpu_count() or 1
    G = x.Hq // x.Hkv
    # Gradient units are whole K/V groups; take as many as there are threads.
    groups = max(1, min(x.Hkv, threads))
    nh = groups * G

    def f64(name, h0, h1):
        from fa_inputs import storage_to_f64
        return storage_to_f64(getattr(x, name)[0:1, h0:h1], x.dtype)

    import fa_inputs
    g = fa_inputs.storage_to_f64(fa_inputs.make_grad_output(4242, (1, nh, x.N, x.d), x.dtype), x.dtype)
    t0 = time.perf_counter()
    oracle.grads(f64("q", 0, nh), f64("k", 0, groups), f64("v", 0, groups), g, x.causal, x.scale,
                 threads=threads)
    dt = time.perf_counter() - t0
    flops = BWD_FLOP_RATIO * x.flops / (x.B * x.Hq) * nh
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, groups),
            "kind": "oracle",
            "sample": f"all {x.N} rows of heads 0..{nh - 1} (batch 0) of {x.recipe}, gradients; "
                      f"{dt:.1f} s in fp64 on {min(threads, groups)} threads"}


def decode_bytes(x) -> int:
    """Compulsory HBM bytes of one decode call: the K/V cache and Q read once, O and
    lse written once (the split workspace is not counted)."""
    e = 2
    return (2 * x.B * x.Hkv * x.Nk * x.d * e + 2 * x.B * x.Hq * x.Nq * x.d * e
            + 4 * x.B * x.Hq * x.Nq)


def cpu_baseline_decode(x, gpu=None) -> dict:
    """The fp64 oracle, as it stands, on the whole decode workload, in GB/s of the
    same compulsory bytes; with `gpu` = (o, lse), the GPU's result is compared with
    it (`parity`)."""
    import oracle
    from fa_inputs import storage_to_f64

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    q, k, v = (storage_to_f64(getattr(x, n), x.dtype) for n in "qkv")
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_kv(q, k, v, x.causal, x.scale, threads=threads)
    dt = time.perf_counter() - t0
    out = {"value": decode_bytes(x) / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole {x.recipe} workload; {dt:.2f} s in fp64 on {threads} threads"}
    if gpu is not None:
        o, lse = gpu
        out["parity"] = parity_of(o.float().cpu().double().numpy(), lse.cpu().double().numpy(),
                                  o_ref, l_ref, x.dtype)
    return out


def decode_kernels(x) -> list:
    """Mangled names of the two kernels one decoding call launches."""
    t = {"bf16": "4BF16", "f16": "3F16"}[x.dtype]
    return [f"_ZN5fa35516fa_decode_kernelINS_{t}ELi{x.d}ELb{int(x.causal)}EEEvNS_10DecodeArgsE",
            f"_ZN5fa35522fa_decode_merge_kernelINS_{t}ELi{x.d}EEEvNS_7FwdArgsE"]


def fwd_kernels(x, plan) -> list:
    """Mangled name of the forward kernel a workload launches (plan: fa_fwd_check's)."""
    if x.dtype == "e4m3":
        return [f"_ZN5fa35517fa_fwd_fp8_kernelILi{x.d}ELb{int(x.causal)}ELi4EEEvNS_7FwdArgsE"]
    if x.dtype == "f32":
        return [f"_ZN5fa35517fa_fwd_f32_kernelILi{plan.waves}ELb{int(x.causal)}EEEvNS_7FwdArgsE"]
    return [fwd_kernel_symbol(x.dtype, x.d, plan.bc, plan.waves, x.causal)]


def code_provenance(kernels: list) -> dict:
    """The machine-code hash of each kernel the line timed, from the loaded library."""
    import io_aware_attention_amd as F
    h = kernel_code_hashes(F.fa355.LIB_PATH)
    return {k: h.get(k) for k in kernels}


def run_decode(args) -> dict:
    import torch

    import fa_inputs as G
    import io_aware_attention_amd as F

    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", 0)))
    torch.cuda.set_device(dev)
    x = G.workload(args.workload)
    q, k, v = device_inputs(x, dev)
    S = args.split or F.decode_split_count(x.B, x.Hkv, x.Nk)
    o = torch.empty_like(q)
    lse = torch.empty((x.B, x.Hq, x.Nq), dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    o_part = torch.empty((S, x.B, x.Hq, x.Nq, x.d), **f32)
    lse_part = torch.empty((S, x.B, x.Hq, x.Nq), **f32)
    stream = torch.cuda.current_stream(dev)

    def step():
        F.fwd_decode(q, k, v, causal=x.causal, scale=x.scale, num_splits=S, o=o, lse=lse,
                     o_part=o_part, lse_part=lse_part, stream=stream)

    if args.profile_run:
        for _ in range(3):
            step()
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"profile_run": args.workload, "copy_bytes": src.numel() * 4}), flush=True)
        return {}
    settled = settle(step, lambda: torch.cuda.synchronize(dev))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    kernel_ms = e0.elapsed_time(e1) / args.steps
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output")
    nbytes = decode_bytes(x)
    ms_per_step = wall * 1e3 / args.steps
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC_DECODE,
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": x.B, "Hq": x.Hq, "Hkv": x.Hkv, "Nq": x.Nq,
                   "Nk": x.Nk, "d": x.d, "causal": x.causal, "scale": x.scale, "seed": x.seed,
                   "num_splits": S, "bytes": nbytes, "flops": x.flops,
                   "pass": "decoding against a key/value cache (fa_fwd_decode: packed "
                           "query-head groups over key pieces, then the merge kernel)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(args.workload, decode_kernels(x)),
                     "kernel_us": round(kernel_ms * 1e3, 2)},
    }
    line["roofline"]["kernel_code"] = code_provenance(decode_kernels(x))
    line["settle"] = {"seconds": SETTLE_S, "launches": settled}
    add_protocol_fields(line, step, stream, dev, args.steps, nbytes, 1e-3, PEAK_HBM_GBS, cold=True)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_decode(x, gpu=(o, lse))
    return line


def sampled_rows(N: int, br: int) -> "np.ndarray":
    """Query rows checked against the oracle for a config line: the first rows, both
    sides of the first tile boundary, the middle and the last rows."""
    import numpy as np
    rows = {0, 1, 2, br - 1, br, br + 1, N // 2, N - 2, N - 1}
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)


def measure_config(name: str, dev, stream) -> dict:
    """Per-launch time of the forward pass on one more named workload (its default
    launch), its rate against its roofline, and the GPU's error on sampled rows of
    two heads against the fp64 oracle."""
    import numpy as np
    import torch

    import fa_inputs as G
    import io_aware_attention_amd as F
    import oracle
    from fa_inputs import storage_to_f64

    x = G.workload(name)
    tuning = G.WORKLOADS[name].get("tuning")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x.dtype]
    plan = F.plan(x.B, x.Hq, x.Hkv, x.N, x.d, x.causal, tdt, tuning=tuning, scale=x.scale)
    q, k, v = device_inputs(x, dev)
    o = torch.empty_like(q)
    lse = torch.empty((x.B, x.Hq, x.N), dtype=torch.float32, device=dev)

    def step():
        F.fwd(q, k, v, causal=x.causal, scale=x.scale, o=o, lse=lse, tuning=tuning, stream=stream)

    sync = lambda: torch.cuda.synchronize(dev)  # noqa: E731
    settle(step, sync, 0.1)
    med, mn = per_launch_us(step, stream, 50)
    nbytes = x.q.nbytes + x.k.nbytes + x.v.nbytes + o.numel() * o.element_size() + x.B * x.Hq * x.N * 4
    peak_flops = PEAK_TFLOPS[x.dtype]
    if x.flops / nbytes < peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, unit, peak, work, scale_ = "hbm", "GB/s", PEAK_HBM_GBS, nbytes, 1e-3
    else:
        bound, unit, peak, work, scale_ = "mfma", "TFLOP/s", peak_flops, x.flops, 1e-6
    out = {"workload": name, "tile": [plan.br, plan.bc], "kernel_us": round(med, 2),
           "kernel_us_min": round(mn, 2), "bound": bound, "achieved": round(work / med * scale_, 2),
           "unit": unit, "peak": peak, "frac": round(work / med * scale_ / peak, 4),
           "tflops": round(x.flops / med * 1e-6, 2),
           "kernel_code": code_provenance(fwd_kernels(x, plan))}
    if bound == "hbm":
        cmed, cmn = per_launch_us(step, stream, 50, flush=cache_flusher(dev))
        out["cold"] = {"kernel_us": round(cmed, 2), "achieved": round(work / cmed * scale_, 2),
                       "frac": round(work / cmed * scale_ / peak, 4),
                       "how": "a 512 MB buffer read before each launch, the reads timed alone and subtracted"}
    # The oracle on sampled rows of the first and the last query head.
    step()
    sync()
    rows = sampled_rows(x.N, plan.br)
    G_ = x.Hq // x.Hkv
    errs = []
    for b, h in ((0, 0), (x.B - 1, x.Hq - 1)):
        f64 = lambda n, hh: storage_to_f64(np.ascontiguousarray(getattr(x, n)[b:b + 1, hh:hh + 1]), x.dtype)  # noqa: E731
        o_ref, l_ref = oracle.attention(f64("q", h), f64("k", h // G_), f64("v", h // G_), x.causal,
                                        x.scale, rows=rows)
        ri = torch.from_numpy(rows).to(dev)
        og = o[b, h].index_select(0, ri).float().cpu().double().numpy()
        lg = lse[b, h].index_select(0, ri).cpu().double().numpy()
        errs.append(parity_of(og, lg, o_ref[0, 0], l_ref[0, 0], x.dtype))
    out["parity"] = {"rows": f"{len(rows)} rows of heads (0,0) and ({x.B - 1},{x.Hq - 1})",
                     "max_abs_o": max(e["max_abs_o"] for e in errs),
                     "max_abs_lse": max(e["max_abs_lse"] for e in errs),
                     "within_tolerance": all(e["within_tolerance"] for e in errs)}
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def run(args) -> dict:
    import torch

    import fa_inputs as G
    import io_aware_attention_amd as F

    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", 0)))
    torch.cuda.set_device(dev)
    x = G.workload(args.workload)
    fp8 = x.dtype == "e4m3"
    tuning = G.WORKLOADS[args.workload].get("tuning")
    if fp8:
        plan = None
    else:
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x.dtype]
        plan = F.plan(x.B, x.Hq, x.Hkv, x.N, x.d, x.causal, tdt, tuning=tuning, scale=x.scale)
    q, k, v = device_inputs(x, dev)
    o = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev) if fp8 else torch.empty_like(q)
    lse = torch.empty((x.B, x.Hq, x.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        F.fwd(q, k, v, causal=x.causal, scale=x.scale, o=o, lse=lse, tuning=tuning, stream=stream)

    if fp8:
        def step():  # noqa: F811
            F.fwd_fp8(q, k, v, *x.descale, causal=x.causal, scale=x.scale, o=o, lse=lse,
                      stream=stream)

    if args.split is not None:
        S = args.split or F.split_count(x.B, x.Hq, x.N, x.causal, d=x.d)
        f32 = dict(dtype=torch.float32, device=dev)
        o_part = torch.empty((S, x.B, x.Hq, x.N, x.d), **f32)
        lse_part = torch.empty((S, x.B, x.Hq, x.N), **f32)

        def step():  # noqa: F811
            F.fwd_split(q, k, v, causal=x.causal, scale=x.scale, num_splits=S, o=o, lse=lse,
                        o_part=o_part, lse_part=lse_part, stream=stream)

    if args.bias is not None:
        shape = {"shared": (1, 1, x.N, x.N), "head": (1, x.Hq, x.N, x.N),
                 "full": (x.B, x.Hq, x.N, x.N)}[args.bias]
        bias = torch.from_numpy(G.make_normal(4243, shape, x.dtype))
        bias = (bias.view(torch.bfloat16) if x.dtype == "bf16" else bias).to(dev)

        def step():  # noqa: F811
            F.fwd_bias(q, k, v, bias, causal=x.causal, scale=x.scale, o=o, lse=lse, stream=stream)

    if args.bwd:
        # The backward pass over the forward pass's own O and lse.
        step()
        dout = torch.from_numpy(G.make_grad_output(4242, (x.B, x.Hq, x.N, x.d), x.dtype))
        dout = (dout.view(torch.bfloat16) if x.dtype == "bf16" else dout).to(dev)
        f32 = dict(dtype=torch.float32, device=dev)
        dq = torch.empty((x.B, x.Hq, x.N, x.d), **f32)
        dk = torch.empty((x.B, x.Hkv, x.N, x.d), **f32)
        dv = torch.empty((x.B, x.Hkv, x.N, x.d), **f32)
        delta = torch.empty((x.B, x.Hq, x.N), **f32)

        def step():  # noqa: F811
            F.bwd(q, k, v, o, dout, lse, causal=x.causal, scale=x.scale, dq=dq, dk=dk, dv=dv,
                  delta=delta, stream=stream)

    if args.profile_run:
        for _ in range(3):
            step()
        # Calibration copy of known size for the HBM byte counters.
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"profile_run": args.workload, "copy_bytes": src.numel() * 4}), flush=True)
        return {}

    settled = settle(step, lambda: torch.cuda.synchronize(dev))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    kernel_ms = e0.elapsed_time(e1) / args.steps
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output")

    flops = x.flops * (BWD_FLOP_RATIO if args.bwd else 1.0)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    # Compulsory HBM bytes: Q, K, V read once; O and lse written once.  Below the
    # ridge point (peak FLOP/s / peak bytes/s) the kernel is bounded by HBM.
    nbytes = x.q.nbytes + x.k.nbytes + x.v.nbytes + o.numel() * o.element_size() + x.B * x.Hq * x.N * 4
    peak_flops = PEAK_TFLOPS[x.dtype]
    if not args.bwd and flops / nbytes < peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    else:
        bound, unit, peak = "mfma", "TFLOP/s", peak_flops
        achieved = flops / (kernel_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC_BWD if args.bwd else (METRIC_FP8 if fp8 else METRIC),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": x.B, "Hq": x.Hq, "Hkv": x.Hkv, "N": x.N,
                   "d": x.d, "causal": x.causal, "scale": x.scale, "seed": x.seed,
                   "tile": [128, 64] if fp8 else [plan.br, plan.bc],
                   "waves": 4 if fp8 else plan.waves,
                   "grid": x.B * x.Hq * -(-x.N // 128) if fp8 else plan.grid},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None if args.bwd else load_traffic(args.workload, fwd_kernels(x, plan)),
                     "kernel_us": round(kernel_ms * 1e3, 2)},
    }
    if not args.bwd and args.split is None and args.bias is None:
        line["roofline"]["kernel_code"] = code_provenance(fwd_kernels(x, plan))
    if args.bias is not None:
        line["config"]["pass"] = f"forward with an additive bias (fa_fwd_bias, bias {list(shape)})"
        line["config"].pop("tile"), line["config"].pop("waves"), line["config"].pop("grid")
        line["roofline"]["traffic"] = None
    if args.split is not None:
        line["config"]["pass"] = f"split-KV forward (fa_fwd_split, {S} splits: partials + merge)"
        line["config"].pop("tile"), line["config"].pop("waves"), line["config"].pop("grid")
        line["roofline"]["traffic"] = None
    if fp8:
        line["config"]["pass"] = ("forward with e4m3 inputs and per-tensor descales (fa_fwd_fp8), "
                                  "bf16 output")
        line["config"]["descale"] = list(x.descale)
    if args.bwd:
        line["config"]["pass"] = "backward (fa_bwd: delta, dK/dV, dQ kernels)"
        line["config"].pop("tile"), line["config"].pop("waves"), line["config"].pop("grid")
    line["settle"] = {"seconds": SETTLE_S, "launches": settled}
    add_protocol_fields(line, step, stream, dev, args.steps, nbytes if bound == "hbm" else flops,
                        1e-3 if bound == "hbm" else 1e-6, peak, cold=bound == "hbm")
    if args.configs and not (args.bwd or fp8 or args.split is not None or args.bias is not None):
        del q, k, v
        torch.cuda.empty_cache()
        line["configs"] = [measure_config(name, dev, stream) for name in CONFIG_WORKLOADS
                           if name != args.workload]
    if not args.no_cpu:
        # The bias line times the same oracle without its bias: no parity there.
        odt = "bf16" if fp8 else x.dtype
        gpu = None if (args.bwd or args.bias is not None) else (o, lse, odt)
        line["cpu_baseline"] = (cpu_baseline_bwd(x, args.cpu_seconds) if args.bwd
                                else cpu_baseline(x, args.cpu_seconds, gpu=gpu))
    return line


def record_traffic_for(workload: str, fetch_csv: str, write_csv: str, command: str) -> dict:
    """record_traffic for the kernels a named workload's default launch uses."""
    import fa_inputs as G
    import io_aware_attention_amd as F
    if "decode" in workload:
        kernels = decode_kernels(G.workload(workload))
    else:
        x = G.workload(workload)
        plan = None
        if x.dtype != "e4m3":
            import torch
            tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x.dtype]
            plan = F.plan(x.B, x.Hq, x.Hkv, x.N, x.d, x.causal, tdt,
                          tuning=G.WORKLOADS[workload].get("tuning"), scale=x.scale)
        kernels = fwd_kernels(x, plan)
    return record_traffic(workload, fetch_csv, write_csv, kernels, command)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--split", type=int, nargs="?", const=0, default=None,
                    help="time the split-KV forward (fa_fwd_split) with this many splits "
                         "(no value: the binding's split_count)")
    ap.add_argument("--bias", choices=("shared", "head", "full"), default=None,
                    help="time fa_fwd_bias with an N(0,1) bias of shape [1,1,N,N], "
                         "[1,Hq,N,N] or [B,Hq,N,N]")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (fa_bwd) instead; FLOPs = 2.5x the forward's")
    ap.add_argument("--decode", action="store_true",
                    help=f"time decoding against a key/value cache (fa_fwd_decode) on "
                         f"{DECODE_WORKLOAD} (--split sets the key pieces)")
    ap.add_argument("--fp8", action="store_true",
                    help=f"time the e4m3-input forward (fa_fwd_fp8) on {FP8_WORKLOAD}")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the per-launch timing of the other named workloads")
    ap.add_argument("--record-traffic", metavar="WORKLOAD", default=None,
                    help="reduce two rocprofv3 counter CSVs (--fetch-csv, --write-csv) of "
                         "`--profile-run --workload WORKLOAD` into profiles/traffic.json")
    ap.add_argument("--fetch-csv", default=None)
    ap.add_argument("--write-csv", default=None)
    ap.add_argument("--command", default="", help="the profiling command, stored with the entry")
    args = ap.parse_args(argv)
    if args.record_traffic:
        print(json.dumps(record_traffic_for(args.record_traffic, args.fetch_csv, args.write_csv,
                                            args.command)), flush=True)
        return 0
    if args.fp8:
        if args.bwd or args.split is not None or args.bias is not None:
            ap.error("--fp8 times the forward pass alone")
        args.workload = FP8_WORKLOAD
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the forward pass of one device's share is "
              f"the whole hot path here; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    if args.decode:
        if args.bwd or args.fp8 or args.bias is not None:
            ap.error("--decode times the decoding call alone")
        if args.workload == DEFAULT_WORKLOAD:
            args.workload = DECODE_WORKLOAD
    line = run_decode(args) if args.decode else run(args)
    if line:
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
