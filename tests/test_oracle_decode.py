"""The oracle's cached-decode path (queries against a longer key sequence) against
its pins (CPU only)."""
import oracle
import decode_pins as DP


def test_decode_matches_torch_sdpa():
    DP.pin_decode_torch(oracle._get(None))


def test_decode_brute_force():
    DP.pin_decode_brute_force(oracle._get(None))


def test_decode_suffix_of_square_causal():
    DP.pin_decode_suffix(oracle._get(None))


def test_decode_closed_forms():
    DP.pin_decode_closed_forms(oracle._get(None))
