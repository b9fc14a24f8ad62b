"""The gradient oracle against its pins (CPU only)."""
import oracle
import grad_pins as GP


def test_grads_match_finite_differences():
    GP.pin_grad_finite_differences(oracle._get(None))


def test_grads_match_torch_autograd():
    GP.pin_grad_autograd(oracle._get(None))


def test_grad_invariants():
    GP.pin_grad_invariants(oracle._get(None))


def test_grad_closed_forms():
    GP.pin_grad_closed_forms(oracle._get(None))
