"""The fp64 oracle against the pages' closed forms, invariants and form
equivalences (CPU only)."""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_forms_agree_ragged():
    # ragged L = 37: the last chunk is short for every B that does not divide it
    P.pin_forms_agree(oracle, L=37, chunks=(1, 2, 3, 5, 8, 16, 32, 36, 37, 64), seed=5)


def test_forms_agree_multibatch():
    P.pin_forms_agree(oracle, L=23, flags_list=(1, 15), chunks=(4, 9), b=3, h=4, dk=6, dv=5, seed=9)
