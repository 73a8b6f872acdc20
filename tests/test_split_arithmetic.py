"""The two-term bf16 split that the fp32 kernels take their products from, modelled in numpy,
against the bounds stated for it in include/linattn.h: hi is x truncated to bf16, lo the bf16
rounding (to nearest even) of x - hi, with +-inf clamped to the largest finite value before the
residual and an x that bf16 holds exactly given lo = x 2^-100.  Checked here:
  * |x - hi - lo| <= 2^-16 |x| and lo has the sign of x (or is zero only for x = 0);
  * the four products hi hi + hi lo + lo hi + lo lo are within 2^-15 |x y| of x y, and their
    errors have either sign (no drift when they are summed);
  * products with an infinity keep fp32's IEEE class.
This is the arithmetic the kernels are built on, not the kernels themselves (the GPU tests
check those against the oracle)."""
import numpy as np

F32MAX = np.float32(np.finfo(np.float32).max)


def _bf16_trunc(x):
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _bf16_rne(x):
    b = x.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


def split(x):
    x = np.asarray(x, np.float32)
    hi = _bf16_trunc(x)
    xc = np.clip(x, -F32MAX, F32MAX)
    with np.errstate(over="ignore", invalid="ignore"):
        r = (xc - _bf16_trunc(xc)).astype(np.float32)
        r = (xc.astype(np.float64) * 2.0 ** -100 + r).astype(np.float32)
    return hi, _bf16_rne(r)


def four(x, y):
    (xh, xl), (yh, yl) = split(x), split(y)
    f = lambda a, b: a.astype(np.float64) * b.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        return ((f(xl, yl) + f(xl, yh)) + f(xh, yl)) + f(xh, yh)


def test_split_holds_each_value_to_2_pow_minus_16():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    hi, lo = split(x)
    err = np.abs(x.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64))
    assert np.all(err <= 2.0 ** -16 * np.abs(x.astype(np.float64)))
    assert np.all((np.sign(lo) == np.sign(x)) | (x == 0))
    assert np.all(lo != 0)


def test_four_products_within_2_pow_minus_15_and_unbiased():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(200000).astype(np.float32)
    y = rng.standard_normal(200000).astype(np.float32)
    exact = x.astype(np.float64) * y.astype(np.float64)
    rel = (four(x, y) - exact) / np.abs(exact)
    assert np.all(np.abs(rel) <= 2.0 ** -15)
    # errors of either sign: the mean relative error is far below its size
    assert abs(np.mean(rel)) < 0.05 * np.mean(np.abs(rel))
    # dropping lo lo (three terms) would leave an error of one sign, about 2^-16 on average
    (xh, xl), (yh, yl) = split(x), split(y)
    three = four(x, y) - xl.astype(np.float64) * yl.astype(np.float64)
    rel3 = (three - exact) / exact
    assert np.mean(rel3) < -0.5 * 2.0 ** -16


def test_values_bf16_holds_exactly():
    x = np.array([1.0, -0.5, 2.5, 3.0, -1.0], np.float32)
    hi, lo = split(x)
    assert np.array_equal(hi, x)
    assert np.all(lo != 0) and np.all(np.abs(lo) <= np.abs(x) * 2.0 ** -99)
    hi0, lo0 = split(np.array([0.0, -0.0], np.float32))
    assert np.all(hi0 == 0) and np.all(lo0 == 0)


def test_infinities_keep_their_class():
    inf = np.float32(np.inf)
    finite = np.array([1.0, -0.5, 2.5, 1.2345678, -3.3333333, 1e-30], np.float32)
    for s in (1, -1):
        got = four(np.full(finite.shape, s * inf, np.float32), finite)
        assert np.all(got == s * np.sign(finite) * np.inf)
        got = four(finite, np.full(finite.shape, s * inf, np.float32))
        assert np.all(got == s * np.sign(finite) * np.inf)
    assert np.isnan(four(np.array([inf]), np.array([0.0], np.float32)))[0]
    assert np.isnan(four(np.array([np.nan], np.float32), np.array([1.0], np.float32)))[0]
