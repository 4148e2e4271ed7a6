"""The exact bf16 parts the block-form scan kernels multiply with.

With bf16 (or f16) q and k, both scan kernels form their products with the
f32 state on the bf16 matrix cores.  The state and Cs enter as three bf16
parts, and f16 q and k as two.  The kernels' comments claim the following,
and this module checks it on the host:
  - f32 x: hi = x with its low 16 bits cleared, mid the same of x - hi, and
    lo = x - hi - mid.  Every step is exact.  For |x| >= 2^-110, lo is a
    bf16 value as it stands and hi + mid + lo == x.  Below that, lo reaches
    f32's subnormal range and its bf16 form drops bits under 2^-133: an
    absolute error under 2^-133 (about 9e-41).
  - f16 x: hi = x (in f32) with its low 16 bits cleared and lo = x - hi.
    Both are bf16 values and hi + lo == x.
So a product of bf16 q or k values with these parts is exact in f32 term by
term, and the kernels' sums differ from the f32 products only in the order
of the additions.
"""
import numpy as np
import pytest

MASK = np.uint32(0xFFFF0000)


def trunc16(x):
    """x (float32) with its low 16 bits cleared: its top 8 significant bits."""
    return (x.view(np.uint32) & MASK).view(np.float32)


def is_bf16(x):
    return np.all((x.view(np.uint32) & np.uint32(0xFFFF)) == 0)


def split3(x):
    hi = trunc16(x)
    r1 = (x - hi).astype(np.float32)
    mid = trunc16(r1)
    lo = (r1 - mid).astype(np.float32)
    return hi, mid, lo, r1


def f32_samples(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    special = np.array([0.0, -0.0, 1.0, -1.0, 1.5, np.pi, 1e-45, -1e-45, 1.17549435e-38,
                        1.1754942e-38, 3.4028235e38, -3.4028235e38, 2.0**-126, 2.0**-149,
                        1.0 + 2.0**-23, 1.0 - 2.0**-24, 0.02, 7e-5],
                       dtype=np.float32)
    normal = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    return np.concatenate([x, special, normal])


@pytest.mark.parametrize("seed", [0, 1])
def test_three_parts_of_f32_are_exact(seed):
    x = f32_samples(1 << 20, seed)
    hi, mid, lo, r1 = split3(x)
    # the residual after hi is exact everywhere: hi + r1 == x in f64
    assert np.array_equal(hi.astype(np.float64) + r1.astype(np.float64), x.astype(np.float64))
    assert is_bf16(hi) and is_bf16(mid)
    lo16 = trunc16(lo)  # lo as the kernels pass it to the matrix cores
    total = hi.astype(np.float64) + mid.astype(np.float64) + lo16.astype(np.float64)
    big = np.abs(x.astype(np.float64)) >= 2.0**-110
    assert big.sum() > len(x) // 2
    # |x| >= 2^-110: lo is a bf16 value, and the three add back to x exactly
    assert is_bf16(lo[big])
    assert np.array_equal(total[big], x[big].astype(np.float64))
    # below: within 2^-133 (the bits of lo under f32's smallest bf16 subnormal)
    assert np.all(np.abs(total[~big] - x[~big].astype(np.float64)) < 2.0**-133)


def test_three_parts_take_the_significant_bits_in_order():
    # 1 + 2^-8 + 2^-17 + 2^-23: hi keeps 1 + 2^-7 rounded down (1.0 here:
    # 2^-8 is bit 8 below the leading one, outside hi's 8 bits), mid 2^-8 ..
    x = np.array([1.0 + 2.0**-8 + 2.0**-17 + 2.0**-23], dtype=np.float32)
    hi, mid, lo, _ = split3(x)
    assert hi[0] == 1.0
    assert mid[0] == np.float32(2.0**-8)
    assert lo[0] == np.float32(2.0**-17 + 2.0**-23)
    # a bf16 value is its own hi, with zero mid and lo
    y = np.array([0.375, -96.0, 2.0**-130], dtype=np.float32)
    hy, my, ly, _ = split3(y)
    assert np.array_equal(hy, y) and not my.any() and not ly.any()


def test_two_parts_of_every_f16_value_are_exact():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    x = h.astype(np.float32)  # exact
    hi = trunc16(x)
    lo = (x - hi).astype(np.float32)
    assert is_bf16(hi) and is_bf16(lo)
    assert np.array_equal(hi.astype(np.float64) + lo.astype(np.float64), h.astype(np.float64))


def test_products_of_bf16_values_are_exact_in_f32():
    # the reason the parts give f32-exact terms: 8 x 8 significant bits fit in 24
    rng = np.random.default_rng(3)
    a = trunc16(rng.standard_normal(1 << 16).astype(np.float32))
    b = trunc16((rng.standard_normal(1 << 16) * 1e-3).astype(np.float32))
    p32 = (a * b).astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), a.astype(np.float64) * b.astype(np.float64))
