"""The identity behind the quantising append kernel's quotient.

The kernel computes value / scale for a bfloat16 value as the float64
product of the value with the float64 reciprocal of the scale, rounded to
float32, in place of a float32 division.  For bfloat16 values (8
significant bits) and finite positive float32 scales this equals the IEEE
float32 quotient; the argument is in the kernel's source.  This checks the
identity on the host with numpy's IEEE arithmetic, for every bfloat16 code
at edge-case scales and a few thousand random ones spread over the whole
float32 range.  It says nothing about the GPU; the GPU tests compare the
kernel's codes with the oracle's.
"""
import numpy as np

F32 = np.finfo(np.float32)
EDGE_SCALES = [1.0, 0.0123, 1 / 448, 3.7, 0.5, 1 / 3, 3.0, 7.0, 0.1,
               float(F32.tiny), float(F32.max), float(F32.smallest_subnormal),
               float(np.nextafter(np.float32(2), np.float32(0)))]


def _bf16_values():
    codes = np.arange(1 << 16, dtype=np.uint32)
    x = (codes << 16).view(np.float32)
    return x[~np.isnan(x)]


def _random_scales(n, seed):
    rng = np.random.default_rng(seed)
    normal = rng.integers(0x00800000, 0x7F800000, n, dtype=np.uint32)
    sub = rng.integers(1, 0x00800000, n // 8, dtype=np.uint32)
    return np.concatenate([normal, sub]).view(np.float32)


def test_reciprocal_product_is_the_float32_quotient():
    x = _bf16_values()
    x64 = x.astype(np.float64)
    scales = np.concatenate([np.array(EDGE_SCALES, dtype=np.float32),
                             _random_scales(3000, 11)])
    with np.errstate(over="ignore", under="ignore"):
        for s in scales:
            want = x / np.float32(s)
            got = (x64 * (1.0 / np.float64(s))).astype(np.float32)
            # bitwise: also the sign of zero and the infinities
            assert np.array_equal(want.view(np.uint32), got.view(np.uint32)), s


def test_single_float32_reciprocal_would_not_do():
    """The float64 product matters: a float32 product with a float32
    reciprocal differs from the quotient for some values (so the check
    above can tell the two apart)."""
    x = _bf16_values()
    with np.errstate(over="ignore", under="ignore"):
        s = np.float32(0.0123)
        want = x / s
        got = x * (np.float32(1) / s)
    assert not np.array_equal(want.view(np.uint32), got.view(np.uint32))
