"""Quantiser of new K/V values into an fp8 e4m3fn pool.

FP8 KV storage halves a block's bytes relative to 16-bit storage
("PagedAttention：KV cache 即虚拟内存（block manager & 碎片）", section
"面试官追问").  A pool stores value / scale per tensor (stored value * scale
= real value).  Writing a new 16-bit token into such a pool therefore
divides by the tensor's scale and rounds to the nearest e4m3fn value.

Readings (the pages give no quantiser):

* the quotient is the IEEE float32 quotient of the float32 widening of the
  input and the float32 scale;
* it saturates to the largest finite magnitude, 448, instead of becoming
  NaN (e4m3fn has no infinity);
* it rounds to the nearest e4m3fn value, ties to the code with an even
  mantissa (round-to-nearest-even); the sign of zero is kept;
* a NaN input gives the code 0x7F.

This is written from the e4m3fn definition (``numerics.E4M3FN_TABLE``: the
exact value of every code): for each input the two neighbouring
representable magnitudes are found and the nearer one chosen.  Test
infrastructure, not product code.
"""
import numpy as np

from .append import kv_append
from .numerics import E4M3FN_TABLE, bf16_bits_to_f64

E4M3FN_MAX = 448.0
NAN_CODE = 0x7F

# non-negative finite codes 0x00 .. 0x7E, increasing in value
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def quotient_f32(x, scale) -> np.ndarray:
    """float32 quotient x / scale (IEEE, round to nearest even)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return (np.asarray(x, dtype=np.float32) /
                np.float32(scale)).astype(np.float32)


def e4m3fn_round(v) -> np.ndarray:
    """Nearest e4m3fn code of each float value (saturating, ties to even)."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    neg = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3FN_MAX)
    # index of the largest representable magnitude <= a
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) &
                               (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = code | np.where(neg, 0x80, 0)
    return np.where(nan, NAN_CODE, code).astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """e4m3fn codes of x / scale (x: values exactly representable in
    float32, e.g. widened bf16)."""
    return e4m3fn_round(quotient_f32(x, scale))


def kv_append_quant(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale,
                    v_scale):
    """Quantising append: fp8 pools (uint8 codes) after writing bf16 rows
    k_new / v_new (uint16 bits) at their slots, skipping negative and
    out-of-pool slots.  Layouts as in ``append.kv_append``."""
    kq = quantize(bf16_bits_to_f64(k_new), k_scale)
    vq = quantize(bf16_bits_to_f64(v_new), v_scale)
    return kv_append(k_pool, v_pool, kq, vq, slot_mapping)
