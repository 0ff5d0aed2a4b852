"""Exact decoders from storage bits to float64.

* bf16: the upper half of an IEEE binary32; value = binary32 whose high 16
  bits are the code and low 16 bits are zero.
* fp8 e4m3fn (the OCP "FN" variant): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the pattern
  S.1111.111 is NaN; there are no infinities, so the largest finite value is
  1.75 * 2^8 = 448.  FP8 KV storage halves a block's bytes relative to 16-bit
  storage ("PagedAttention：KV cache 即虚拟内存", section "面试官追问").

Both are exact: every bf16 and every e4m3fn value is representable in
float64.
"""
import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    as_u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN codes widen to NaN
        return as_u32.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)],
                        dtype=np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(bits, dtype=np.uint8)]


def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a raw storage array (float32 / uint16 / uint8) to float64."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "fp8_e4m3fn":
        return e4m3fn_bits_to_f64(raw)
    raise ValueError(f"unknown storage dtype {dtype!r}")
