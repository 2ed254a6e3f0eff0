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


def _fma32(a, b, c):
    """fmaf: the exact a*b+c (float32 operands, so exact in double up to
    one rounding of the sum) rounded once to float32."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(np.float32)


def mul_lrelu_gelu_folded_f32(y, m, slope):
    """float32 emulation of the fused epilogue (b) as the kernels evaluate
    it: multiplier pre-scaled by kGeluIn = sqrt(log2(e)/2), A&S 7.1.26 with
    p' = p / sqrt(log2 e), coefficients scaled by c = 1 / (2 kGeluIn),
    exp(-x^2) as 2^(-z^2), and 1 + erf picked by the LeakyReLU compare as
    |base - q e| with base 1/kGeluIn or 0 (one fused rounding).  The
    reciprocal and exp2 are correctly rounded here; the hardware forms are
    within 1 ulp of these."""
    f = np.float32
    k_in = f(0.8493218002880191)
    c = f(0.5887050112577373)
    y = np.asarray(y, np.float32)
    mk = (np.asarray(m, np.float32) * k_in).astype(np.float32)
    u = (y * mk).astype(np.float32)
    pos = (u >= 0) | (slope < 0)
    z = np.where(u >= 0, u, (f(slope) * u).astype(np.float32)).astype(np.float32)
    t = (f(1.0) / _fma32(f(0.2727374808792225), np.abs(z), f(1.0))).astype(np.float32)
    q = (f(1.061405429) * c).astype(np.float32) * np.ones_like(z)
    for a in (-1.453152027, 1.421413741, -0.284496736, 0.254829592):
        q = _fma32(q, t, f(a) * c)
    q = (q * t).astype(np.float32)
    e = np.exp2(-(z * z).astype(np.float32)).astype(np.float32)
    base = np.where(pos, f(1.1774100225154747), f(0.0)).astype(np.float32)
    return (z * np.abs(_fma32(-q, e, base))).astype(np.float32)


def test_folded_gelu_constants_derive_from_the_published_ones():
    """The folded constants are the A&S 7.1.26 ones rescaled: p' = p /
    sqrt(log2 e), c = 1 / (2 kGeluIn), 1 / kGeluIn, kGeluIn^2 = log2(e)/2."""
    k_in = math.sqrt(math.log2(math.e) / 2.0)
    assert abs(k_in - 0.8493218002880191) < 1e-16
    assert abs(0.3275911 / math.sqrt(math.log2(math.e)) - 0.2727374808792225) < 1e-16
    assert abs(1.0 / (2.0 * k_in) - 0.5887050112577373) < 1e-16
    assert abs(1.0 / k_in - 1.1774100225154747) < 1e-15


def test_folded_gelu_matches_exact_gelu():
    """The folded evaluation of GELU(LeakyReLU(y * m)) against the erf-based
    definition in double, over [-12, 12], for the slope of the workload and
    for zero, negative and >1 slopes, with multipliers of both signs."""
    y = np.linspace(-12.0, 12.0, 120001)
    for slope in (0.01, 0.0, -0.5, 1.5):
        for m in (1.0, 0.93, -1.07):
            u = y * np.float64(np.float32(m))
            v = np.where(u >= 0, u, slope * u)
            ref = 0.5 * v * (1.0 + np.array([math.erf(t / math.sqrt(2.0)) for t in v]))
            got = mul_lrelu_gelu_folded_f32(y.astype(np.float32), m, slope).astype(np.float64)
            err = np.abs(got - ref)
            # absolute error far inside the parity bar; and a relative bound
            # where the result is not small (A&S 7.1.26 bounds erf's
            # absolute error, so the relative error of the far negative
            # tail, where 1 + erf is tiny, is not bounded this way)
            assert err.max() < 2e-5, (slope, m, err.max())
            big = np.abs(ref) > 0.05
            assert (err[big] / np.abs(ref[big])).max() < 1e-5, (slope, m)
    # special values: GELU(0) = 0; large positive -> identity; y = -10 with
    # slope 0.01 is GELU(-0.1) = -0.05 (1 - erf(0.1 / sqrt 2)); slope 1 and
    # y = -10 is the far tail, -10 Phi(-10) ~ -7.6e-23
    assert mul_lrelu_gelu_folded_f32(np.float32(0.0), 1.0, 0.01) == 0.0
    assert abs(float(mul_lrelu_gelu_folded_f32(np.float32(10.0), 1.0, 0.01)) - 10.0) < 1e-5
    g = -0.05 * (1.0 - math.erf(0.1 / math.sqrt(2.0)))
    assert abs(float(mul_lrelu_gelu_folded_f32(np.float32(-10.0), 1.0, 0.01)) - g) < 1e-7
    assert abs(float(mul_lrelu_gelu_folded_f32(np.float32(-10.0), 1.0, 1.0))) < 1e-12


def test_folded_gelu_catches_a_wrong_constant():
    """A plausible slip -- the unfolded p = 0.3275911 in the folded form --
    is caught by the comparison above."""
    y = np.linspace(-6.0, 6.0, 20001)
    ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in y])
    f = np.float32
    z = (y * 0.8493218002880191).astype(np.float32)
    t = f(1.0) / (f(1.0) + f(0.3275911) * np.abs(z))
    c = 0.5887050112577373
    q = t * (0.254829592 * c + t * (-0.284496736 * c + t * (1.421413741 * c + t * (
        -1.453152027 * c + t * 1.061405429 * c))))
    r = q * np.exp2(-z * z)
    bad = z * np.where(z >= 0, 1.1774100225154747 - r, r)
    assert np.abs(bad - ref).max() > 1e-3


def tanh_e2_f32(x):
    """float32 emulation of the kernels' tanh: sign(x) (1 - e) / (1 + e),
    e = 2^(-2|x| log2 e)."""
    x = np.asarray(x, dtype=np.float32)
    e = np.exp2(np.abs(x) * np.float32(-2.8853900817779268)).astype(np.float32)
    return np.copysign((np.float32(1.0) - e) / (np.float32(1.0) + e), x).astype(np.float32)


def test_tanh_e2_matches_tanh():
    xs = np.linspace(-20.0, 20.0, 400001)
    got = tanh_e2_f32(xs).astype(np.float64)
    ref = np.tanh(xs)
    assert np.max(np.abs(got - ref)) < 1e-6
    # tanh(tanh(x)), as the channel-min epilogue applies it
    got2 = tanh_e2_f32(tanh_e2_f32(xs)).astype(np.float64)
    assert np.max(np.abs(got2 - np.tanh(np.tanh(xs)))) < 1e-6
    # the special values
    assert tanh_e2_f32(np.float32(0.0)) == 0.0
    assert np.signbit(tanh_e2_f32(np.float32(-0.0)))
    assert tanh_e2_f32(np.float32(np.inf)) == 1.0 and tanh_e2_f32(np.float32(-np.inf)) == -1.0
    assert np.isnan(tanh_e2_f32(np.float32(np.nan)))
    # odd, and monotone on a fine grid around 0
    assert np.array_equal(tanh_e2_f32(-xs), -tanh_e2_f32(xs))
    small = np.linspace(-1e-3, 1e-3, 20001)
    assert np.all(np.diff(tanh_e2_f32(small).astype(np.float64)) >= 0.0)


def test_tanh_e2_catches_a_wrong_constant():
    """The pin above fails for a plausible slip: exp instead of exp2 with the
    same constant."""
    x = np.linspace(-4.0, 4.0, 10001)
    e = np.exp(np.abs(x) * -2.8853900817779268)
    wrong = np.copysign((1.0 - e) / (1.0 + e), x)
    assert np.max(np.abs(wrong - np.tanh(x))) > 1e-2
