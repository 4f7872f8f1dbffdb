"""The CPU oracle against its pins, and planted mistakes against the pins.

Runs on the CPU only.  Every pin must hold for the real oracle.  Each planted
build (one deliberate mistake compiled into the oracle with -DORC_PLANT=n)
must fail at least one pin, which shows the pins would catch that mistake.
"""
import pytest

import oracle
import oracle_pins as P

PLANTS = {
    1: "Q4_K min added instead of subtracted",
    2: "Q4_K high nibbles given the low sub-block's scale",
    3: "Q4_K upper scales take their high bits from the wrong byte",
    4: "Q6_K high 2 bits shifted by g instead of 2g",
    5: "Q6_K quant not centred by 32",
    6: "Q6_K scale index i/32 instead of i/16",
    7: "RMSNorm eps added outside the square root",
    8: "second norm of the tail sees the residual before the add",
    9: "SiLU without its sigmoid factor",
    10: "f16 exponent bias 16",
    11: "matvec drops the last superblock of each row",
    12: "activation index reversed inside each superblock",
    13: "threaded row split leaves one row of each range uncomputed",
    14: "Q5_K high bit taken from bit c of the chunk, not bit 2c or 2c+1",
    15: "Q5_K high bit worth 32 instead of 16",
    16: "Q5_K low nibbles read from the high-bit bytes' offset",
}


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.get())


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda n: f"plant{n}")
def test_planted_mistake_is_caught(plant):
    o = oracle.Oracle(plant)
    assert o.lib.orc_plant() == plant
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"no pin catches plant {plant} ({PLANTS[plant]})"


def test_real_oracle_has_no_plant():
    assert oracle.get().lib.orc_plant() == 0
