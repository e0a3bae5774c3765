"""The oracle against its pins (CPU only).  See tests/pins.py for what each
pin checks and where its expected values come from."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_g32(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", [pins.pin_decode_trace, pins.pin_decode_bruteforce,
                                 pins.pin_decode_partition_invariance,
                                 pins.pin_prefill_trace, pins.pin_prefill_vs_decode,
                                 pins.pin_prefill_uint8_w],
                         ids=lambda f: f.__name__)
def test_pin_g64(orc, pin):
    pin(orc, G=64)
