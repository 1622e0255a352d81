"""The fp64 oracle against facts it does not define itself (closed forms,
invariants, limits, a hand-derived example).  CPU only."""
import pytest

import oracle
import oracle.scan as oscan
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    ok, detail = pin(oscan)
    assert ok, f"{pin.__name__}: {detail}"


def test_softplus_special_values():
    import math
    import numpy as np
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    # softplus(v) - softplus(-v) = v for every v
    v = np.linspace(-40, 40, 161)
    np.testing.assert_allclose(oracle.softplus(v) - oracle.softplus(-v), v, rtol=0, atol=1e-13)
    # far tails: log1p(e^v) ~ e^v for v << 0 and ~ v for v >> 0
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-15)
    assert oracle.softplus(50.0) == pytest.approx(50.0, rel=1e-15)


def test_silu_special_values():
    import math
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert oracle.silu(-math.log(3.0)) == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300
    assert oracle.silu(800.0) == pytest.approx(800.0, rel=1e-15)
