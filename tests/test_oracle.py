"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


def test_brute_force(lib):
    P.pin_brute_force(lib)


def test_torch_sdpa(lib):
    P.pin_torch_sdpa(lib)


def test_closed_forms(lib):
    P.pin_closed_forms(lib)


def test_invariants(lib):
    P.pin_invariants(lib)


def test_blocked_reference_agrees(lib):
    P.pin_blocked_agrees(lib)


def test_rejects_bad_arguments(lib):
    q = np.zeros((1, 3, 4, 8))
    k = np.zeros((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, False, 1.0, lib=lib)          # 3 % 2 != 0
    q = np.zeros((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, False, 1.0, rows=[4], lib=lib)  # row out of range
