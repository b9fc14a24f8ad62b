"""The benchmark's kernel provenance, checked on the CPU against the built library.

bench.py names the kernel each measured workload launches (fwd_kernels), reports the
sha256 of that kernel's gfx950 machine code from libfa355.so, and reports HBM
traffic only while profiles/traffic.json was taken at the same code.  These tests
pin that the names it derives from the library's own launch plans exist in the
library, that head dim 256 maps to the kernel split by role at its default tile
and to the wavefront pairs at 128 x 64, and that every committed traffic record
matches the kernels as built.
"""
import json
import os
import sys
import types

import pytest
import torch

import fa_inputs as G
import io_aware_attention_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _plan_and_shape(name):
    w = G.WORKLOADS[name]
    x = types.SimpleNamespace(dtype=w["dtype"], d=w["d"], causal=w["causal"])
    p = F.plan(w["B"], w["Hq"], w["Hkv"], w["N"], w["d"], w["causal"], TDT[w["dtype"]],
               tuning=w.get("tuning"))
    return x, p


@pytest.mark.parametrize("name", (bench.DEFAULT_WORKLOAD,) + bench.CONFIG_WORKLOADS)
def test_every_measured_kernel_is_in_the_library(name):
    hashes = bench.kernel_code_hashes(F.fa355.LIB_PATH)
    x, p = _plan_and_shape(name)
    for sym in bench.fwd_kernels(x, p):
        assert sym in hashes, f"{name}: {sym} not among the library's kernels"


def test_head_dim_256_kernel_names():
    hashes = bench.kernel_code_hashes(F.fa355.LIB_PATH)
    p = F.plan(1, 8, 8, 8192, 256, True, torch.bfloat16)
    assert (p.br, p.bc, p.waves) == (128, 32, 8)
    role = bench.fwd_kernel_symbol("bf16", 256, p.bc, p.waves, True)
    assert "fa_fwd_role_kernel" in role and role in hashes
    p = F.plan(1, 8, 8, 8192, 256, True, torch.bfloat16, tuning=(128, 64))
    pair = bench.fwd_kernel_symbol("bf16", 256, p.bc, p.waves, True)
    assert "fa_fwd_pair_kernel" in pair and pair in hashes
    assert hashes[role] != hashes[pair]


def test_traffic_records_match_the_built_kernels():
    hashes = bench.kernel_code_hashes(F.fa355.LIB_PATH)
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        table = json.load(fh)
    assert table
    for workload, entry in table.items():
        for sym, h in entry["kernels"].items():
            assert hashes.get(sym) == h, f"{workload}: {sym} built as {hashes.get(sym)}, counted at {h}"
        assert bench.load_traffic(workload) == entry["bytes_per_launch"]
