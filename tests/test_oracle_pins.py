"""The CPU oracle against its pins (library routines, closed forms, brute
force, and the invariants the pages state). CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_BASIC, ids=lambda f: f.__name__)
def test_basic_pins(pin):
    pin()


@pytest.mark.parametrize("cfg", [pins.TINY_F32, pins.TINY_BF16, pins.TINY_MOE], ids=lambda c: c.name)
@pytest.mark.parametrize("pin", pins.MODEL_PINS, ids=lambda f: f.__name__)
def test_model_pins(pin, cfg):
    pin(cfg)


@pytest.mark.parametrize("pin", pins.MOE_PINS, ids=lambda f: f.__name__)
def test_moe_pins(pin):
    pin()


@pytest.mark.parametrize("cfg", [pins.TINY_F32, pins.TINY_BF16, pins.TINY_MOE], ids=lambda c: c.name)
@pytest.mark.parametrize("pin", pins.VARIANT_PINS, ids=lambda f: f.__name__)
def test_variant_pins(pin, cfg):
    pin(cfg)


@pytest.mark.parametrize("cfg", [pins.TINY_F32, pins.TINY_BF16, pins.TINY_MOE], ids=lambda c: c.name)
@pytest.mark.parametrize("pin", pins.FORWARD_PINS, ids=lambda f: f.__name__)
def test_forward_pins(pin, cfg):
    pin(cfg)
