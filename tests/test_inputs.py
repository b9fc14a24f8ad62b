"""The seeded input generator: stream, normals and single-rounding to dtypes."""
import math

import numpy as np
import torch

import fa_inputs as G

_M64 = (1 << 64) - 1


def _splitmix64_sequential(seed, n):
    """SplitMix64 as a state machine (the published form), one output per call."""
    x = seed & _M64
    out = []
    for _ in range(n):
        x = (x + 0x9E3779B97F4A7C15) & _M64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_matches_sequential_form():
    for seed in (0, 1, 1002, 2**63 + 5, _M64):
        seq = _splitmix64_sequential(seed, 300)
        assert [int(z) for z in G.splitmix64(seed, 0, 300)] == seq
        assert [int(z) for z in G.splitmix64(seed, 123, 50)] == seq[123:173]


def test_splitmix64_known_vector():
    # First outputs of the reference splitmix64.c for seed 1234567.
    assert [int(z) for z in G.splitmix64(1234567, 0, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_normals_box_muller_and_stream_positions():
    st = G.Stream(99)
    n = st.normals(7)
    assert st.pos == 8
    u = G._uniform53(G.splitmix64(99, 0, 8))
    for p in range(4):
        r = math.sqrt(-2.0 * math.log(1.0 - u[2 * p]))
        ref = (r * math.cos(2 * math.pi * u[2 * p + 1]), r * math.sin(2 * math.pi * u[2 * p + 1]))
        for e in range(2):
            if 2 * p + e < 7:
                assert abs(n[2 * p + e] - ref[e]) <= 1e-15 * max(1.0, abs(ref[e]))
    big = G.Stream(5).normals(400_001)
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1.0) < 0.01


def test_round_f16_matches_numpy_direct_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [0.0, -0.0, 65504.0, 65520.0, 70000.0, -1e6, 2.0 ** -24, 2.0 ** -25,
                         3 * 2.0 ** -26, np.inf, -np.inf]])
    r = G.round_to_dtype(x, "f16")
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(r, ref)


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * 10.0 ** rng.integers(-40, 38, 50000)).astype(np.float32)
    x = np.concatenate([x, np.float32([1e-45, -3e-39, 3.3e38, np.inf, 0.0])])
    r = G.round_to_dtype(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(r, ref)


def test_round_bf16_ties_and_single_rounding():
    one = 1.0
    assert G.round_to_dtype(np.array([one + 2 ** -8]), "bf16")[0] == 1.0            # tie -> even
    assert G.round_to_dtype(np.array([one + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6  # tie -> even
    # Just above a tie, but a detour through fp32 would land on the tie and go down.
    x = one + 2 ** -8 + 2 ** -40
    assert G.round_to_dtype(np.array([x]), "bf16")[0] == 1 + 2 ** -7
    assert G.round_to_dtype(np.array([np.nan]), "bf16")[0] != 0  # NaN stays NaN


def test_storage_roundtrip():
    x = G.round_to_dtype(np.random.default_rng(3).standard_normal(1000) * 3, "bf16")
    s = G.to_storage(x, "bf16")
    assert s.dtype == np.int16
    assert np.array_equal(G.storage_to_f64(s, "bf16"), x)
    t = torch.from_numpy(s).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(t, x)


def test_make_inputs_fill_order_and_bias():
    a = G.make_inputs(1003, 2, 3, 3, 5, 4, "f64", False, q_head_bias=True)
    st = G.Stream(1003)
    q = st.normals(2 * 3 * 5 * 4).reshape(2, 3, 5, 4)
    k = st.normals(2 * 3 * 5 * 4).reshape(2, 3, 5, 4)
    v = st.normals(2 * 3 * 5 * 4).reshape(2, 3, 5, 4)
    beta = 2.0 * st.uniforms(3)
    assert np.array_equal(a.k, k) and np.array_equal(a.v, v)
    assert np.array_equal(a.q, q + beta[None, :, None, None])
    assert ((0 <= beta) & (beta < 2)).all()
    b = G.make_inputs(1003, 2, 3, 3, 5, 4, "bf16", False, q_head_bias=True)
    assert np.array_equal(b.f64("q"), G.round_to_dtype(q + beta[None, :, None, None], "bf16"))
    assert G.make_inputs(7, 1, 1, 1, 3, 2, "f32", True).scale == float(np.float32(1 / math.sqrt(2)))


def test_e4m3_codec_matches_torch_float8_e4m3fn():
    # Every code decodes as torch's OCP e4m3 type does (NaN where it has NaN), and
    # every finite value encodes back to its code (+0 and -0 distinct).
    codes = np.arange(256, dtype=np.uint8)
    v = G.storage_to_f64(codes, "e4m3")
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    fin = ~np.isnan(v)
    assert np.array_equal(v[fin], t[fin])
    assert np.array_equal(G.to_storage(v[fin], "e4m3"), codes[fin])
    assert np.isnan(v).sum() == 2 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6


def test_round_e4m3_matches_torch_on_fp32_values():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 3, 100000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    x = np.concatenate([x, np.float32([2.0 ** -10, 3 * 2.0 ** -10, 1 + 2 ** -4, 1 + 3 * 2 ** -4, 232.0,
                                       -2.0 ** -11, 0.0])])
    r = G.round_to_dtype(x.astype(np.float64), "e4m3")
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(r, ref)


def test_quantize_e4m3_per_tensor_descale():
    x = G.Stream(11).normals(4096) * 3.0
    codes, ds = G.quantize_e4m3(x)
    vals = ds * G.storage_to_f64(codes, "e4m3")
    assert ds == float(np.float32(np.abs(x).max() / 448.0))
    assert np.abs(vals).max() <= 448.0 * ds * (1 + 1e-7)
    # one rounding to e4m3 (relative 2^-4 for normals, absolute 2^-10 * ds below)
    assert (np.abs(vals - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * ds) * (1 + 1e-6)).all()
    a = G.make_inputs(21, 1, 2, 1, 50, 64, "e4m3", True)
    assert a.q.dtype == np.uint8 and len(a.descale) == 3
    st = G.Stream(21)
    q = st.normals(2 * 50 * 64).reshape(1, 2, 50, 64)
    cq, dq = G.quantize_e4m3(q)
    assert np.array_equal(a.q, cq) and a.descale[0] == dq
    assert np.array_equal(a.f64("q"), dq * G.storage_to_f64(cq, "e4m3"))


def test_every_workload_matches_its_stored_hash():
    """Each named workload's inputs are bit-identical to those the stored hashes were
    taken from (tests/golden/make_input_hashes.py, which calls only this module)."""
    import importlib.util
    import json
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_input_hashes",
                                                  os.path.join(here, "make_input_hashes.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(here, "input_hashes.json")) as f:
        stored = json.load(f)
    assert set(stored) == set(G.WORKLOADS) | set(G.DECODE_WORKLOADS)
    for name, want in stored.items():
        assert mk.digest(G.workload(name)) == want, name
