"""Pins of the gradient oracle (oracle/ssd_oracle_grad.c), all on the CPU.

The gradients are checked against central finite differences of the fp64 forward, which
is itself checked to be bitwise the pinned forward oracle on float32-representable
inputs, plus closed forms that follow from the recurrence (tests/grad_pins.py).
"""
import pytest

import oracle
from grad_pins import FD_CASES, pin_closed_forms, pin_finite_differences, \
    pin_forward64_is_forward, pin_single_token


def test_forward64_is_the_forward_oracle():
    pin_forward64_is_forward(oracle)


@pytest.mark.parametrize("shape,sample", FD_CASES)
def test_gradients_match_finite_differences(shape, sample):
    pin_finite_differences(oracle, shape, sample)


def test_closed_forms():
    pin_closed_forms(oracle)


def test_single_token_by_hand():
    pin_single_token(oracle)
