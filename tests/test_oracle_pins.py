"""The oracle against its pins (CPU only). See ``oracle_pins.py`` for what each pin fixes."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin()


def test_hand_count(oracle_lib):
    P.pin_hand_count()
