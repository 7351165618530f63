"""The INT8 pack kernel takes the code of an entry x of a column with scale
s as the nearest integer (half to even) of the product y = x (1 / s), with
1 / s correctly rounded, and falls back to the correctly rounded quotient
x / s when y lies within 6e-5 of a half-integer.  Eq. 10 ([dasc] Appendix
E.1) rounds the fp32 quotient, so the product route is exact only if y and
the quotient are closer than that band for every |x| <= 127 s.  This
checks that claim on many fp32 pairs (random entries, exact ties and their
neighbours, every binade of s the kernels meet), in IEEE fp32 arithmetic
on the CPU, with no GPU and no part of the oracle."""
import numpy as np

GUARD = np.float32(0.5 - 6e-5)


def _pairs(rng, n):
    f = np.float32
    s = (np.ldexp(1.0, rng.integers(-60, 100, n)) * rng.uniform(1, 2, n)).astype(f)
    k = rng.integers(-127, 127, n).astype(np.float64)
    kind = rng.integers(0, 4, n)
    ulp = np.spacing(np.abs((k + 0.5) * s.astype(np.float64)).astype(f)).astype(np.float64)
    d = np.where(kind == 0, 0.0,                                     # exact half
        np.where(kind == 1, rng.integers(-4, 5, n) * ulp,            # a few ulps off
        np.where(kind == 2, rng.uniform(-1e-4, 1e-4, n) * s,         # inside / near the band
                 rng.uniform(-0.5, 0.5, n) * s)))                    # anywhere in the step
    x = ((k + 0.5) * s.astype(np.float64) + d).astype(f)
    # keep |x| <= 127 s, as within one column (s = max |x| / 127)
    x = np.clip(x, -f(127) * s, f(127) * s)
    return x, s


def test_product_code_equals_quotient_code_outside_the_band():
    rng = np.random.default_rng(10)
    worst = 0.0
    for _ in range(20):
        x, s = _pairs(rng, 500_000)
        inv = np.float32(1) / s
        y = x * inv
        q = x / s
        worst = max(worst, float(np.max(np.abs(y.astype(np.float64) - q))))
        r = np.rint(y)
        safe = np.abs(y - r) <= GUARD
        assert np.array_equal(r[safe], np.rint(q)[safe])
        assert (~safe).sum() > 0          # the band is exercised
    assert worst < 2.3e-5                  # the bound the band is sized from


def test_scale_from_column_maximum_keeps_quotients_within_127():
    # s = max / 127 rounded: every |x| <= max has |x / s| <= 127 (1 + 2^-23)
    rng = np.random.default_rng(11)
    m = (np.ldexp(1.0, rng.integers(-26, 127, 1_000_000)) * rng.uniform(1, 2, 1_000_000)).astype(np.float32)
    s = m / np.float32(127)
    assert np.all(np.abs(m.astype(np.float64) / s.astype(np.float64)) <= 127 * (1 + 2.0 ** -23))


def test_clip_never_binds_on_either_route():
    # the kernel leaves out Eq. 10's clip to [-127, 127]: for the column
    # maximum itself (the largest |x| of a column), both the fp32 product
    # m (1 / s) and the fp32 quotient m / s round to at most 127
    rng = np.random.default_rng(12)
    f = np.float32
    m = (np.ldexp(1.0, rng.integers(-26, 127, 2_000_000)) * rng.uniform(1, 2, 2_000_000)).astype(f)
    m = np.concatenate([m, np.array([1e-8, np.finfo(f).max, np.finfo(f).tiny], f)])
    s = np.maximum(m, f(1e-8)) / f(127)
    inv = f(1) / s
    assert np.all(np.abs(np.rint(m * inv)) <= 127)
    assert np.all(np.abs(np.rint(m / s)) <= 127)
    assert np.all(np.abs(m * inv) < 127.5)
