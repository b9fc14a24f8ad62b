"""The oracle's additive-bias path against its pins (CPU only)."""
import oracle
import bias_pins as BP


def test_bias_reduces_to_plain_and_causal():
    BP.pin_bias_reductions(oracle._get(None))


def test_bias_row_shift_invariance():
    BP.pin_bias_row_shift(oracle._get(None))


def test_bias_matches_torch():
    BP.pin_bias_torch(oracle._get(None))


def test_bias_broadcast_and_fully_masked_rows():
    BP.pin_bias_broadcast_and_empty_rows(oracle._get(None))
