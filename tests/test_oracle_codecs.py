"""Pins for the oracle's bf16 and E4M3FN codecs (CPU only).

E4M3FN values are checked against a table built here from the format's
definition with exact rational arithmetic, and against torch's own
float8_e4m3fn CPU conversion.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode_satfinite
from workload import f32_to_bf16_bits


def _e4m3_value_exact(code: int):
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def test_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC020, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0
    assert v[1] == -2.5
    assert v[2] == 0.0 and v[3] == 0.0 and np.signbit(v[3])
    assert v[4] == float(Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 7)))
    assert v[5] == 2.0 ** -133
    assert v[6] == 3.140625


def test_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4096).astype(np.float32) * 7
    bits = f32_to_bf16_bits(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), bits)
    assert np.array_equal(bf16_bits_to_f64(bits), t.to(torch.float64).numpy())


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    v = e4m3fn_decode(codes)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        ex = _e4m3_value_exact(c)
        if ex is None:
            assert np.isnan(v[c]) and np.isnan(tv[c]), c
        else:
            assert v[c] == float(ex), c
            assert tv[c] == float(ex), c
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert v[1] == 2.0 ** -9


def test_e4m3_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3fn_encode_satfinite(v), codes)
    # midpoints between neighbours go to the even code
    pos = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    enc = e4m3fn_encode_satfinite(mids).astype(np.int64)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, want)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 3,
        rng.standard_normal(20000) * 1e-2,
        rng.standard_normal(5000) * 1e-3,
    ]).astype(np.float32)
    ours = e4m3fn_encode_satfinite(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_encode_saturates_and_nan():
    x = np.array([449.0, 463.9, 464.0, 1e6, -1e6, np.inf, -np.inf, np.nan], dtype=np.float32)
    c = e4m3fn_encode_satfinite(x)
    assert list(c[:4]) == [0x7E] * 4
    assert list(c[4:7]) == [0xFE, 0x7E, 0xFE]
    assert c[7] == 0x7F


@pytest.mark.parametrize("v,code", [(2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01),
                                    (-2.0 ** -11, 0x80), (3 * 2.0 ** -10, 0x02)])
def test_e4m3_encode_subnormal_rounding(v, code):
    assert e4m3fn_encode_satfinite(np.array([v], np.float32))[0] == code
