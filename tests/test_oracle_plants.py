"""Plant a mistake in the oracle (on the CPU) and check that a pin catches it.

Each ``KVO_PLANT`` variant of ``oracle/kvpub_oracle.c`` is a plausible slip:
ties away from zero, overflow to NaN, a dropped sign, a wrong range constant,
an amax that skips an element, scales or RoPE bytes out of order, a wrong
scale offset, page and offset swapped, pads counted as invalid, a replica
skipped, a wrong subnormal step, truncation instead of rounding, the tile
scale as a multiply by RN(1/448), the quotient as a multiply by RN(1/scale); on the
reader side a sign dropped on decode, bf16 truncation, scales of the wrong
tile, subnormal binary32 products flushed to zero, bf16 subnormals flushed."""
import pytest

import oracle
import pins

PLANTS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20]


@pytest.mark.parametrize("plant", PLANTS)
def test_planted_mistake_is_caught(plant):
    orc = oracle.Oracle(plant=plant, rebuild=True)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:120]))
    assert caught, f"planted mistake {plant} passed every pin"
