"""CPU checks of numerical building blocks the kernels use."""
import math

import numpy as np


def erf_as7126_f32(x):
    """float32 emulation of the kernels' erf: Abramowitz & Stegun 7.1.26."""
    x = np.asarray(x, dtype=np.float32)
    ax = np.abs(x)
    t = np.float32(1.0) / (np.float32(0.3275911) * ax + np.float32(1.0))
    q = np.float32(1.061405429)
    for c in (-1.453152027, 1.421413741, -0.284496736, 0.254829592):
        q = q * t + np.float32(c)
    q = q * t
    e = np.exp2(-ax * ax * np.float32(1.4426950408889634)).astype(np.float32)
    return np.copysign(np.float32(1.0) - q * e, x)


def test_erf_as7126_within_published_bound():
    xs = np.linspace(-8.0, 8.0, 400001, dtype=np.float64)
    ref = np.array([math.erf(v) for v in xs])
    # the formula itself, evaluated in double: the published 1.5e-7 bound
    t = 1.0 / (1.0 + 0.3275911 * np.abs(xs))
    q = t * (0.254829592 + t * (-0.284496736 + t * (1.421413741 + t * (-1.453152027
                                                                   + t * 1.061405429))))
    assert np.max(np.abs(np.sign(xs) * (1.0 - q * np.exp(-xs * xs)) - ref)) < 1.5e-7
    # evaluated in float32 as the kernels do: rounding in 1 - q*exp(-x^2)
    # adds up to ~5e-7 near x = 0 (where GELU multiplies it by |v|/2 ~ 0)
    got = erf_as7126_f32(xs.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-6
    assert erf_as7126_f32(0.0) == 0.0
    assert np.all(np.abs(erf_as7126_f32(np.array([10.0, -10.0, 40.0]))) == 1.0)


def test_gelu_from_as7126_meets_tolerance():
    """GELU(v) = 0.5 v (1 + erf(v / sqrt 2)) built on the approximation stays
    far inside the 2e-4 output tolerance over the range conv outputs take."""
    v = np.linspace(-12.0, 12.0, 200001)
    ref = 0.5 * v * (1.0 + np.array([math.erf(t / math.sqrt(2.0)) for t in v]))
    vf = v.astype(np.float32)
    got = (np.float32(0.5) * vf * (np.float32(1.0) + erf_as7126_f32(vf * np.float32(0.70710678118654752))))
    assert np.max(np.abs(got.astype(np.float64) - ref)) < 5e-6
