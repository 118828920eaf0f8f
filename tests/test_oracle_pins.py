"""The CPU oracle against closed forms, textbook tables, library routines, brute force and
statistical laws (no GPU)."""
import pytest

from tests import pins

CHECKS = [name for name in dir(pins) if name.startswith("check_")]


@pytest.mark.parametrize("name", CHECKS)
def test_pin(name):
    getattr(pins, name)()
