"""Each plausible mistake planted in oracle R must fail at least one pin.

The mistakes are compiled into separate CPU builds of the oracle source
(``-DKDA_MUTANT=n``); the oracle proper is built without the flag.  This runs
on the CPU only and never touches the GPU.
"""
import functools

import pytest

import oracle
from tests import oracle_pins as P

MUTANTS = {
    1: "predict before the forget step",
    2: "gate indexed by value channel",
    3: "beta dropped from the correction",
    4: "sign of the error flipped",
    5: "read before the write",
    6: "outer product transposed",
    7: "query scale dropped",
    8: "gate applied again after the write",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_catch_mutant(mutant):
    rec = functools.partial(oracle.recurrent, mutant=mutant)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(rec)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mutant}: {MUTANTS[mutant]}"
