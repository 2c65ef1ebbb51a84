"""Pins for oracle/formats.py: format tables, encoders and BF16 rounding,
against hand-derived tables, torch's dtype casts and brute force."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import _golden as gold


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_e2m1_table_matches_golden():
    table = gold.code_table("e2m1_codes.txt")
    assert len(table) == 16
    for code, value in table:
        got = F.e2m1_decode(code)
        assert got == value and np.signbit(got) == np.signbit(value), (code, got, value)


def test_e4m3_points_match_golden():
    for code, value in gold.code_table("e4m3fn_points.txt"):
        got = F.e4m3_decode(code)
        assert got == value and np.signbit(got) == np.signbit(value), (hex(code), got, value)
        assert F.e4m3_encode(np.float64(value)) == code


def test_e4m3_table_against_torch_decode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e4m3_encode_matches_torch_cast_exhaustive_bf16():
    """Every finite BF16 value with |v| <= 448, cast by torch's RNE
    float8_e4m3fn conversion, against the oracle's table search."""
    bits = all_finite_bf16()
    v = F.bf16_to_f64(bits)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v).astype(np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def brute_force_nearest_even(v, mags, sign_bit):
    """Independent brute force: distance to every magnitude, min, ties even."""
    a = np.abs(v)[:, None]
    d = np.abs(a - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(len(mags))[None, :]
    even_cand = cand & (codes % 2 == 0)
    pick = np.where(even_cand.any(axis=1), even_cand.argmax(axis=1), cand.argmax(axis=1))
    return pick | (np.signbit(v).astype(np.int64) << sign_bit)


@pytest.mark.parametrize("fmt", [F.FMT_MXFP4, F.FMT_MXFP8])
def test_encoders_match_brute_force_exhaustive(fmt):
    bits = all_finite_bf16()
    v = F.bf16_to_f64(bits)
    if fmt == F.FMT_MXFP4:
        mags, sb, enc = F.E2M1_MAGNITUDES, F.E2M1_SIGN_BIT, F.e2m1_encode
    else:
        mags, sb, enc = F.E4M3_MAGNITUDES, F.E4M3_SIGN_BIT, F.e4m3_encode
    v = v[np.abs(v) <= mags[-1]]
    assert np.array_equal(enc(v), brute_force_nearest_even(v, mags, sb))


def test_e2m1_tie_table():
    # ties between neighbouring grid points go to the even code
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0])
    want = np.array([0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x8, 0xE])
    assert np.array_equal(F.e2m1_encode(v), want)


def test_encoders_reject_out_of_range():
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([6.5]))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([449.0]))


def test_e8m0_decode():
    assert F.e8m0_decode(127) == 1.0
    assert F.e8m0_decode(0) == 2.0 ** -127
    assert F.e8m0_decode(254) == 2.0 ** 127
    with pytest.raises(ValueError):
        F.e8m0_decode(255)


def test_bf16_roundtrip_exhaustive():
    bits = all_finite_bf16()
    assert np.array_equal(F.f64_to_bf16(F.bf16_to_f64(bits)), bits)


def test_bf16_rounding_matches_torch_on_float32():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-39).astype(np.float32),  # subnormals
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        # exact BF16 midpoints (ties) built from random BF16 neighbours
        (F.bf16_to_f64(rng.integers(0, 0x7F00, 50_000).astype(np.uint16)) * (1 + 2.0 ** -8)).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f64_to_bf16(x.astype(np.float64)), ref)


def test_bf16_single_rounding_from_f64():
    # 1 + 2**-8 + 2**-30 lies just above the midpoint between 1 and 1 + 2**-7.
    # One rounding gives 1 + 2**-7 (0x3F81); going through float32 first
    # would land on the midpoint and tie down to 1.0 (0x3F80).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.f64_to_bf16(np.array([x]))[0] == 0x3F81
    assert F.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80  # tie -> even
    assert F.f64_to_bf16(np.array([-0.0]))[0] == 0x8000
