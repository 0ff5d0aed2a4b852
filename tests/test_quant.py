"""Pins of the oracle's fp8 e4m3fn quantiser (quantising append).

* library routine: torch's float32 -> float8_e4m3fn cast on inputs already
  clamped to +-448 (torch rounds to nearest even there, and gives NaN past
  the largest finite value, which is why the quantiser clamps first);
* round trip of every finite code, ties between neighbouring codes, the
  saturation and NaN rules, the float32 quotient;
* the append lands the quantised rows at their slots only.
"""
import numpy as np
import pytest
import torch

from oracle import numerics, quant

CODES = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                  dtype=np.uint8)


def _torch_e4m3(v):
    t = torch.from_numpy(np.asarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_round_trip_of_every_finite_code():
    vals = numerics.E4M3FN_TABLE[FINITE]
    got = quant.e4m3fn_round(np.where(FINITE == 0x80, -0.0, vals))
    assert np.array_equal(got, FINITE)


def test_ties_go_to_the_even_code():
    for c in range(0x7E):                       # positive neighbours c, c+1
        lo, hi = numerics.E4M3FN_TABLE[c], numerics.E4M3FN_TABLE[c + 1]
        mid = (lo + hi) / 2
        want = c if c % 2 == 0 else c + 1
        assert quant.e4m3fn_round(mid) == want, hex(c)
        assert quant.e4m3fn_round(-mid) == want | 0x80
        # just off the midpoint: the nearer neighbour, whatever its parity
        eps = (hi - lo) * 1e-6
        assert quant.e4m3fn_round(mid - eps) == c
        assert quant.e4m3fn_round(mid + eps) == c + 1


def test_saturation_zero_and_nan():
    assert quant.e4m3fn_round(448.0) == 0x7E
    for v in (449.0, 464.0, 480.0, 1e30, np.inf):
        assert quant.e4m3fn_round(v) == 0x7E
        assert quant.e4m3fn_round(-v) == 0xFE
    assert quant.e4m3fn_round(0.0) == 0x00
    assert quant.e4m3fn_round(-0.0) == 0x80
    assert quant.e4m3fn_round(2.0 ** -10) == 0x00      # tie with 0: even
    assert quant.e4m3fn_round(2.0 ** -10 * 1.0001) == 0x01
    assert quant.e4m3fn_round(np.nan) == quant.NAN_CODE


def test_matches_torch_cast_on_clamped_float32():
    rng = np.random.default_rng(0)
    bf16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = numerics.bf16_bits_to_f64(bf16)
    x = x[np.isfinite(x)].astype(np.float32)
    for scale in (1.0, 0.0123, 3.7e-3, 1.9):
        v = np.clip(quant.quotient_f32(x, scale), -448, 448)
        assert np.array_equal(quant.e4m3fn_round(v), _torch_e4m3(v)), scale
    v = (rng.standard_normal(200_000) * 60).astype(np.float32)
    v = np.clip(v, -448, 448)
    assert np.array_equal(quant.e4m3fn_round(v), _torch_e4m3(v))


def test_quotient_is_the_float32_quotient():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10_000).astype(np.float32)
    s = np.float32(0.0071)
    q = quant.quotient_f32(x, s)
    ref = (torch.from_numpy(x) / torch.tensor(s)).numpy()
    assert np.array_equal(q.view(np.uint32), ref.view(np.uint32))
    # correctly rounded: within half an ulp of the exact quotient
    exact = x.astype(np.float64) / np.float64(s)
    ulp = np.spacing(np.abs(q)).astype(np.float64)
    assert (np.abs(q.astype(np.float64) - exact) <= ulp / 2).all()


def test_planted_truncation_is_caught():
    """Rounding toward zero instead of to nearest breaks the torch pin."""
    v = np.float32([1.1, 2.9, 100.3, -5.7])
    trunc = []
    for x in v:
        mags = numerics.E4M3FN_TABLE[:0x7F]
        i = np.searchsorted(mags, abs(float(x)), side="right") - 1
        trunc.append(i | (0x80 if x < 0 else 0))
    assert not np.array_equal(np.array(trunc, dtype=np.uint8),
                              _torch_e4m3(v))


def test_quantising_append_writes_only_the_slots():
    rng = np.random.default_rng(2)
    nb, hkv, d = 6, 2, 64
    k = rng.integers(0, 256, size=(nb, hkv, 16, d), dtype=np.uint8)
    v = rng.integers(0, 256, size=(nb, hkv, d, 16), dtype=np.uint8)
    kn = torch.randn(3, hkv, d).to(torch.bfloat16)
    vn = torch.randn(3, hkv, d).to(torch.bfloat16)
    knb = kn.view(torch.uint16).numpy()
    vnb = vn.view(torch.uint16).numpy()
    slots = np.array([5, -1, 3 * 16 + 15], dtype=np.int32)
    k1, v1 = quant.kv_append_quant(k, v, knb, vnb, slots, 0.01, 0.02)
    mask = np.zeros((nb, 16), dtype=bool)
    mask[0, 5] = mask[3, 15] = True
    untouched = ~mask
    assert np.array_equal(k1.transpose(0, 2, 1, 3)[untouched],
                          k.transpose(0, 2, 1, 3)[untouched])
    assert np.array_equal(v1.transpose(0, 3, 1, 2)[untouched],
                          v.transpose(0, 3, 1, 2)[untouched])
    want_k = _torch_e4m3(np.clip(kn.float().numpy() / np.float32(0.01),
                                 -448, 448))
    assert np.array_equal(k1[0, :, 5, :], want_k[0])
    assert np.array_equal(k1[3, :, 15, :], want_k[2])
    want_v = _torch_e4m3(np.clip(vn.float().numpy() / np.float32(0.02),
                                 -448, 448))
    assert np.array_equal(v1[3, :, :, 15], want_v[2])
