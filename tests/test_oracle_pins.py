"""The CPU oracle against its pins (hand-worked groups, numpy fp16, closed forms,
brute force, the pages' byte arithmetic).  No GPU."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(orc, check):
    check(orc)
