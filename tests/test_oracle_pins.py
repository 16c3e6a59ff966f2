"""The CPU oracle against its pins (no GPU)."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.FAST_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_f16_conversion_exhaustive(orc):
    """Every binary32 bit pattern converts to the same binary16 bits as the
    library routine (NaNs: any quiet NaN)."""
    pins.pin_f16_exhaustive(orc)


def test_closed_forms_cover_each_rule():
    """The golden file exercises each rule it claims to: ties, a negative
    absmax, binary16-subnormal scales and binary16 ties in the scale."""
    cases = {c["name"]: c for c in pins.load_closed_forms()}
    ties = cases["ties_half_away"]
    frac = [abs(k) % 2 == 1 for k in ties["k"]]
    assert sum(frac) >= 20
    neg = cases["negative_absmax"]
    assert min(neg["k"]) == -127 and max(neg["k"]) < 127
    assert cases["subnormal_scale"]["d16"] < 0x0400
    assert cases["subnormal_scale_rounded"]["d16"] == 0x0001
