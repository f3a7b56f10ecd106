"""Pins of the oracle's epilogue activation (SiLU, the activation of the kernel contract in
"Hardware support and kernel ABI contracts") against facts that do not restate its
formula: the odd-part identity, the asymptotes, the Taylor series at 0, and the closed
form of its minimum through the Lambert W function.  Each pin is a predicate on a
function, run on the oracle (must hold) and on planted mistakes (must fail)."""
import math

import numpy as np
import pytest
from scipy.optimize import minimize_scalar
from scipy.special import lambertw

import oracle


def _f(fn, x):
    return np.asarray(fn(np.asarray(x, dtype=np.float64)), dtype=np.float64)


def odd_part_is_identity(fn):
    # sigmoid(x) + sigmoid(-x) = 1  =>  silu(x) - silu(-x) = x for every x
    x = np.concatenate([np.linspace(-30, 30, 601), [1e-30, 3.5, 7.25, 1e5]])
    return np.allclose(_f(fn, x) - _f(fn, -x), x, rtol=1e-14, atol=1e-300)


def asymptotes_and_zero(fn):
    ok = _f(fn, [0.0])[0] == 0.0
    # x -> +inf: silu(x) -> x with error x e^-x;  x -> -inf: silu(x) ~ x e^x
    for x in (40.0, 100.0, 1e6):
        ok &= abs(_f(fn, [x])[0] - x) <= x * math.exp(-x) * 1.01 + 1e-300
    for x in (-40.0, -100.0):
        ok &= math.isclose(_f(fn, [x])[0], x * math.exp(x), rel_tol=1e-12)
    return bool(ok)


def taylor_at_zero(fn):
    # x sigmoid(x) = x/2 + x^2/4 - x^4/48 + O(x^6)
    return all(abs(_f(fn, [h])[0] - (h / 2 + h * h / 4 - h ** 4 / 48)) <= abs(h) ** 6 + 1e-18
               for h in (1e-2, 1e-3, 1e-4, -1e-3))


def minimum_closed_form(fn):
    # d/dx x sigmoid(x) = 0  <=>  1 + x (1 - sigmoid(x)) = 0, root x* = -1 - W(1/e), where
    # silu(x*) = x* + 1 = -W(1/e)
    w = float(np.real(lambertw(1.0 / math.e)))
    res = minimize_scalar(lambda t: _f(fn, [t])[0], bracket=(-3.0, -1.0, 0.0), tol=1e-12)
    return abs(res.x - (-1.0 - w)) < 1e-6 and abs(res.fun - (-w)) < 1e-12


PINS = [odd_part_is_identity, asymptotes_and_zero, taylor_at_zero, minimum_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_silu_meets_pin(pin):
    assert pin(oracle.silu)


MISTAKES = {
    "exponent sign": lambda v: v / (1.0 + np.exp(v)),
    "result sign": lambda v: -oracle.silu(v),
    "dropped x": lambda v: 1.0 / (1.0 + np.exp(-v)),
    "sigmoid of 2x": lambda v: v / (1.0 + np.exp(-2.0 * v)),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_reject_planted_mistake(name):
    with np.errstate(over="ignore"):
        assert not all(pin(MISTAKES[name]) for pin in PINS)
